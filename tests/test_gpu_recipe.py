"""GPU parity of the fused scale update (history, scale, scale_inv bit for bit) and of the
FP8 linear forward / backward (casts bit for bit, GEMMs within tolerance), the launch
sequence as a replayed graph, the weight-cache noop flag and the stale-cache hazard."""
import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, bf16_dev, f32_bits, gemm_close, scalar, to_f64, u8_host

pytestmark = pytest.mark.gpu


def _update(h, s, si, fmts, margin):
    hd = torch.from_numpy(h.copy()).to(DEV)
    sd = torch.from_numpy(s.copy()).to(DEV)
    sid = torch.from_numpy(si.copy()).to(DEV)
    F.fp8_scale_update(hd, sd, sid, fmts, margin)
    torch.cuda.synchronize()
    return hd.cpu().numpy(), sd.cpu().numpy(), sid.cpu().numpy()


def _same(a, b):
    return np.array_equal(f32_bits(a), f32_bits(b))


def test_scale_update_backward_prep_config():
    """History [1024][3]: 1023 seeded log-uniform past amaxes in [1e-3, 1e3] for x and W, the
    current dy slot from its cast; margin 0; one fused launch for the three tensors."""
    L, T = 1024, 3
    h = np.zeros((L, T), np.float32)
    h[1:, 0] = S.log_uniform_f32(S.seed_for(3, 1), L - 1, 1e-3, 1e3)
    h[1:, 1] = S.log_uniform_f32(S.seed_for(3, 2), L - 1, 1e-3, 1e3)
    dyh = S.normal_bf16(S.seed_for(3, 0), (8192, 4096), 0.01)
    h[0, 2] = oracle.cast_amax(dyh, 1.0, 1)[1]
    h[0, 0] = h[5, 0]
    s = np.array([2.0, 3.0, 5.0], np.float32)
    si = (1 / s).astype(np.float32)
    fm = [F.E4M3, F.E4M3, F.E5M2]
    got = _update(h, s, si, fm, 0)
    ref = oracle.scale_update(h, s, si, fm, 0)
    for g, r in zip(got, ref):
        assert _same(g, r)


@pytest.mark.parametrize("L", [1, 2, 16, 255, 256, 257, 1024, 8192, 8193, 9000])
def test_scale_update_many_steps(L):
    """Windows staged whole in LDS (L <= 8192) and longer ones rolled in chunks."""
    T = 5
    fm = [0, 1, 0, 1, 0]
    h = np.zeros((L, T), np.float32)
    s = np.ones(T, np.float32)
    si = np.ones(T, np.float32)
    hd = torch.from_numpy(h.copy()).to(DEV)
    sd = torch.from_numpy(s.copy()).to(DEV)
    sid = torch.from_numpy(si.copy()).to(DEV)
    am = S.log_uniform_f32(S.seed_for(6, L), 40 * T, 1e-3, 1e3).reshape(40, T)
    am[10:30, 2] = 0.0                      # zero amaxes: previous scale kept
    am[7, 3] = np.float32(2.0 ** -133)      # tiny amax: 448 / a overflows, previous kept
    am[20, 4] = np.inf                      # infinite amax: previous kept
    for k in range(40):
        h[0] = am[k]
        hd[0] = torch.from_numpy(am[k]).to(DEV)
        F.fp8_scale_update(hd, sd, sid, fm, 1 if k % 3 == 0 else 0)
        h, s, si = oracle.scale_update(h, s, si, fm, 1 if k % 3 == 0 else 0)
    torch.cuda.synchronize()
    assert _same(hd.cpu().numpy(), h) and _same(sd.cpu().numpy(), s) and _same(sid.cpu().numpy(), si)


@pytest.mark.parametrize("L,T", [(4, 4096), (9000, 64)])
def test_scale_update_guard_cases_and_many_tensors(L, T):
    h = np.zeros((L, T), np.float32)
    h[:, :] = S.log_uniform_f32(91, L * T, 1e-6, 1e6).reshape(L, T)
    h[:, 0] = 0.0
    h[:, 1] = np.float32(2.0 ** -133)
    h[0, 2] = np.inf
    h[2, 3] = np.nan
    h[:, 4] = np.float32(1e-45)              # smallest subnormal
    h[:, 5] = np.float32(3.4e38)
    s = S.log_uniform_f32(92, T, 0.5, 2.0)
    si = (1 / s).astype(np.float32)
    fm = [int(v) for v in (S.uniform(93, 0, T) < 0.5)]
    for margin in (0, 3, -2, 126):
        got = _update(h, s, si, fm, margin)
        ref = oracle.scale_update(h, s, si, fm, margin)
        for g, r in zip(got, ref):
            assert _same(g, r), margin


@pytest.mark.parametrize("L", [300, 9000])
def test_scale_update_nan_read_by_every_wave(L):
    """A NaN in any row of the window keeps the previous scale, whichever of the block's four
    waves reads it: thread i reads rows i, i + 256, ..., so row r goes to wave (r % 256) // 64.
    Tensor t holds one NaN in a row of wave t (the last tensor none), on the LDS-staged path
    (L = 300) and on the chunked path (L = 9000)."""
    T = 6
    nan_rows = [2, 70, 130, 200, L - 50]          # waves 0, 1, 2, 3 and a late row
    h = S.log_uniform_f32(S.seed_for(6, 77), L * T, 1e-3, 1e3).reshape(L, T)
    for t, r in enumerate(nan_rows):
        h[r, t] = np.nan
    s = S.log_uniform_f32(S.seed_for(6, 78), T, 0.5, 2.0)
    si = (1 / s).astype(np.float32)
    fm = [F.E4M3, F.E5M2, F.E4M3, F.E5M2, F.E4M3, F.E4M3]
    got = _update(h, s, si, fm, 0)
    ref = oracle.scale_update(h, s, si, fm, 0)
    for g, r in zip(got, ref):
        assert _same(g, r)
    assert _same(got[1][:5], s[:5]) and not _same(got[1][5:], s[5:])   # NaN windows kept their scale


@pytest.mark.parametrize("margin", [126, 125])
def test_scale_update_tiny_scale_guard(margin):
    """Amaxes at and around the point where (fp8_max / a) * 2^-margin, or its inverse, leaves
    the float32 range: 448, 896 (scale 2^-127, inverse finite), 1792 (inverse overflows), 1e6
    (subnormal scale), FLT_MAX (scale 0), on the GPU against the oracle."""
    am = np.array([448.0, 896.0, 1792.0, 1e6, 3.4028235e38, 57344.0], np.float32)
    T = am.size
    h = np.zeros((4, T), np.float32)
    h[1] = am
    s = np.full(T, 3.0, np.float32)
    si = (1 / s).astype(np.float32)
    fm = [F.E4M3] * 5 + [F.E5M2]
    got = _update(h, s, si, fm, margin)
    ref = oracle.scale_update(h, s, si, fm, margin)
    for g, r in zip(got, ref):
        assert _same(g, r)


def test_scale_update_rejects_bad_arguments():
    hd = torch.zeros((4, 2), device=DEV)
    sd = torch.ones(2, device=DEV)
    with pytest.raises(F.Fp8dsError):
        F.fp8_scale_update(hd, sd, sd.clone(), [0, 7], 0)
    with pytest.raises(F.Fp8dsError):
        F.fp8_scale_update(hd, sd, sd.clone(), [0, 1], 127)


# ----------------------------------------------------------------------------- linear layer

class Layer:
    """Device buffers of one FP8 linear layer (persistent addresses, as a graph needs)."""

    def __init__(self, M, N, K, L=16, dw_fp32=True):
        u8 = dict(device=DEV, dtype=torch.uint8)
        f32 = dict(device=DEV, dtype=torch.float32)
        self.M, self.N, self.K = M, N, K
        self.hist = torch.zeros((L, 3), **f32)
        self.scale = torch.ones(3, **f32)
        self.scale_inv = torch.ones(3, **f32)
        self.sinv = torch.zeros(3, **f32)          # the FP8 tensors' private inverse scales
        self.x8, self.x8t = torch.empty((M, K), **u8), torch.empty((K, M), **u8)
        self.w8, self.w8t = torch.empty((N, K), **u8), torch.empty((K, N), **u8)
        self.dy8, self.dy8t = torch.empty((M, N), **u8), torch.empty((N, M), **u8)
        self.y = torch.empty((M, N), device=DEV, dtype=torch.bfloat16)
        self.dx = torch.empty((M, K), device=DEV, dtype=torch.bfloat16)
        self.dw = torch.empty((N, K), device=DEV, dtype=torch.float32 if dw_fp32 else torch.bfloat16)
        self.db = torch.empty(N, **f32)
        self.ws = torch.zeros(max(1, F.fp8_dbias_workspace_bytes(M, N)), **u8)
        self.noop = torch.zeros(1, **f32)

    def fwd(self, x, w, b, stream=None, noop=None):
        F.fp8_linear_fwd(x, w, b, self.scale[0:1], self.hist[0, 0:1], self.x8, self.x8t, self.sinv[0:1],
                         self.scale[1:2], self.hist[0, 1:2], self.w8, self.w8t, self.sinv[1:2], noop, self.y,
                         stream=stream)

    def bwd(self, dy, stream=None):
        F.fp8_linear_bwd(dy, self.K, self.scale[2:3], self.hist[0, 2:3], self.dy8, self.dy8t, self.sinv[2:3],
                         self.db, self.ws, self.x8t, self.sinv[0:1], self.w8t, self.sinv[1:2], self.dx, self.dw,
                         stream=stream)

    def update(self, stream=None):
        F.fp8_scale_update(self.hist, self.scale, self.scale_inv, [F.E4M3, F.E4M3, F.E5M2], 0, stream=stream)


def _inputs(M, N, K, cfg):
    x = S.normal_bf16(S.seed_for(cfg, 0), (M, K), 1.0)
    w = S.normal_bf16(S.seed_for(cfg, 1), (N, K), 0.02 if cfg == 4 else 1.0)
    b = S.normal_bf16(S.seed_for(cfg, 2), (N,), 0.1)
    dy = S.normal_bf16(S.seed_for(cfg, 3), (M, N), 0.01)
    return x, w, b, dy


@pytest.mark.parametrize("shape", [(128, 256, 256), (272, 400, 528)])
def test_linear_fwd_bwd_vs_oracle_three_iterations(shape):
    """Three training iterations (fwd, bwd, update) of the small linear layer: FP8 tensors,
    amaxes, private inverse scales, scales and history bit-exact; y, dx, dW within tolerance."""
    M, N, K = shape
    xh, wh, bh, dyh = _inputs(M, N, K, 0)
    x, w, b, dy = bf16_dev(xh), bf16_dev(wh), bf16_dev(bh), bf16_dev(dyh)
    lay = Layer(M, N, K)
    h = np.zeros((16, 3), np.float32)
    s = np.ones(3, np.float32)
    si = np.ones(3, np.float32)
    for it in range(3):
        lay.fwd(x, w, b)
        lay.bwd(dy)
        hb = lay.hist.clone()
        lay.update()
        torch.cuda.synchronize()
        fw = oracle.linear_fwd(xh, wh, bh, s[0], s[1])
        bw = oracle.linear_bwd(dyh, s[2], fw["x8t"], fw["x_sinv"], fw["w8t"], fw["w_sinv"])
        assert np.array_equal(u8_host(lay.x8), fw["x8"]) and np.array_equal(u8_host(lay.x8t), fw["x8t"])
        assert np.array_equal(u8_host(lay.w8), fw["w8"]) and np.array_equal(u8_host(lay.w8t), fw["w8t"])
        assert np.array_equal(u8_host(lay.dy8), bw["dy8"]) and np.array_equal(u8_host(lay.dy8t), bw["dy8t"])
        assert _same(lay.sinv.cpu().numpy(), [fw["x_sinv"], fw["w_sinv"], bw["dy_sinv"]])
        h[0] = [fw["x_amax"], fw["w_amax"], bw["dy_amax"]]
        assert _same(hb.cpu().numpy(), h), it
        gemm_close(to_f64(lay.y), fw["y"], bf16_out=True)
        gemm_close(to_f64(lay.dx), bw["dx"], bf16_out=True)
        gemm_close(to_f64(lay.dw), bw["dw"], bf16_out=False)
        assert np.all(np.abs(lay.db.cpu().numpy() - bw["dbias"]) <= 1e-5 * np.abs(S.bf16_bits_to_f64(dyh)).sum(0) + 1e-30)
        h, s, si = oracle.scale_update(h, s, si, [0, 0, 1], 0)
        assert _same(lay.hist.cpu().numpy(), h) and _same(lay.scale.cpu().numpy(), s)
        assert _same(lay.scale_inv.cpu().numpy(), si)


def test_linear_equals_primitive_sequence():
    """fp8_linear_fwd / fp8_linear_bwd give exactly what the individual calls give."""
    M, N, K = 256, 384, 512
    xh, wh, bh, dyh = _inputs(M, N, K, 0)
    x, w, b, dy = bf16_dev(xh), bf16_dev(wh), bf16_dev(bh), bf16_dev(dyh)
    lay = Layer(M, N, K)
    lay.scale.copy_(torch.tensor([3.0, 40.0, 9000.0]))
    lay.fwd(x, w, b)
    lay.bwd(dy)
    # the same steps one call at a time
    u8 = dict(device=DEV, dtype=torch.uint8)
    x8, x8t, w8, w8t = torch.empty((M, K), **u8), torch.empty((K, M), **u8), torch.empty((N, K), **u8), torch.empty((K, N), **u8)
    dy8, dy8t = torch.empty((M, N), **u8), torch.empty((N, M), **u8)
    sinv = torch.zeros(3, device=DEV)
    am = torch.zeros(3, device=DEV)
    F.fp8_cast_transpose(x, lay.scale[0:1], F.E4M3, x8, x8t, sinv[0:1], am[0:1])
    F.fp8_cast_transpose(w, lay.scale[1:2], F.E4M3, w8, w8t, sinv[1:2], am[1:2])
    y = torch.empty((M, N), device=DEV, dtype=torch.bfloat16)
    F.fp8_gemm_bias(x8, F.E4M3, sinv[0:1], w8, F.E4M3, sinv[1:2], b, y)
    db = torch.empty(N, device=DEV)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(M, N), **u8)
    F.fp8_dbias_cast_transpose(dy, lay.scale[2:3], F.E5M2, dy8, dy8t, db, ws, sinv[2:3], am[2:3])
    dx = torch.empty((M, K), device=DEV, dtype=torch.bfloat16)
    dw = torch.empty((N, K), device=DEV, dtype=torch.float32)
    F.fp8_gemm_bias(dy8, F.E5M2, sinv[2:3], w8t, F.E4M3, sinv[1:2], None, dx)
    F.fp8_gemm_bias(dy8t, F.E5M2, sinv[2:3], x8t, F.E4M3, sinv[0:1], None, dw)
    torch.cuda.synchronize()
    for a, b_ in ((lay.x8, x8), (lay.x8t, x8t), (lay.w8, w8), (lay.w8t, w8t), (lay.dy8, dy8), (lay.dy8t, dy8t)):
        assert torch.equal(a, b_)
    assert torch.equal(lay.y.view(torch.int16), y.view(torch.int16))
    assert torch.equal(lay.dx.view(torch.int16), dx.view(torch.int16))
    assert torch.equal(lay.dw.view(torch.int32), dw.view(torch.int32))
    assert torch.equal(lay.db.view(torch.int32), db.view(torch.int32))
    assert torch.equal(lay.hist[0].view(torch.int32), am.view(torch.int32))
    assert torch.equal(lay.sinv.view(torch.int32), sinv.view(torch.int32))


def test_weight_cache_noop_and_stale_cache():
    """With the noop flag set, the weight's FP8 copy, transpose and private inverse scale stay
    as they were (cached across microbatches); an in-place weight update followed by a recast
    (flag clear) refreshes all three; the scale update alone never touches them."""
    M, N, K = 128, 256, 256
    xh, wh, bh, _ = _inputs(M, N, K, 0)
    x, w, b = bf16_dev(xh), bf16_dev(wh), bf16_dev(bh)
    lay = Layer(M, N, K)
    lay.fwd(x, w, b, noop=lay.noop)
    torch.cuda.synchronize()
    w8_0, w8t_0, s0 = lay.w8.clone(), lay.w8t.clone(), lay.sinv[1].item()
    # the optimizer step changes W in place; the scale changes too
    w.mul_(-0.5)
    lay.scale[1] = 8.0
    lay.noop.fill_(1.0)             # cached: second microbatch reuses the FP8 weight
    lay.fwd(x, w, b, noop=lay.noop)
    torch.cuda.synchronize()
    assert torch.equal(lay.w8, w8_0) and torch.equal(lay.w8t, w8t_0) and lay.sinv[1].item() == s0
    lay.noop.fill_(0.0)             # first microbatch of the next step: recast
    lay.fwd(x, w, b, noop=lay.noop)
    torch.cuda.synchronize()
    rq, rqt, _, rs = oracle.cast_transpose(bf16_host_w(w), 8.0, F.E4M3)
    assert np.array_equal(u8_host(lay.w8), rq) and np.array_equal(u8_host(lay.w8t), rqt)
    assert _same(lay.sinv[1].item(), rs)
    gemm_close(to_f64(lay.y), oracle.gemm_bias(u8_host(lay.x8), 0, lay.sinv[0].item(), rq, 0, rs, bh), bf16_out=True)


def bf16_host_w(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def test_graph_replay_equals_eager_training_steps():
    """The whole iteration (fwd, bwd, fused update) captured once and replayed: every replay
    matches the same sequence run eagerly from the same state, bit for bit."""
    M, N, K = 256, 512, 384
    xh, wh, bh, dyh = _inputs(M, N, K, 0)
    x, w, b, dy = bf16_dev(xh), bf16_dev(wh), bf16_dev(bh), bf16_dev(dyh)
    eager = Layer(M, N, K)
    graph = Layer(M, N, K)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        graph.fwd(x, w, b, stream=cap)
        graph.bwd(dy, stream=cap)
        graph.update(stream=cap)
    # capture only records: reset the graph layer's state to the initial one
    for t in (graph.hist, graph.sinv):
        t.zero_()
    graph.scale.fill_(1.0)
    graph.scale_inv.fill_(1.0)
    torch.cuda.synchronize()
    for it in range(4):
        eager.fwd(x, w, b)
        eager.bwd(dy)
        eager.update()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name in ("hist", "scale", "scale_inv", "sinv", "x8", "x8t", "w8", "w8t", "dy8", "dy8t", "db", "dw"):
            a, b_ = getattr(eager, name), getattr(graph, name)
            assert torch.equal(a.view(torch.uint8), b_.view(torch.uint8)), (it, name)
        for name in ("y", "dx"):
            assert torch.equal(getattr(eager, name).view(torch.int16), getattr(graph, name).view(torch.int16))


def test_resume_from_copied_state():
    """k iterations, copy the recipe state, continue n more; a fresh layer loaded with the copy
    and run n iterations ends in the same state bit for bit."""
    M, N, K = 128, 256, 256
    xh, wh, bh, dyh = _inputs(M, N, K, 0)
    x, w, b, dy = bf16_dev(xh), bf16_dev(wh), bf16_dev(bh), bf16_dev(dyh)
    a = Layer(M, N, K)
    for _ in range(3):
        a.fwd(x, w, b); a.bwd(dy); a.update()
    state = [t.clone() for t in (a.hist, a.scale, a.scale_inv)]
    for _ in range(2):
        a.fwd(x, w, b); a.bwd(dy); a.update()
    c = Layer(M, N, K)
    for dst, src in zip((c.hist, c.scale, c.scale_inv), state):
        dst.copy_(src)
    for _ in range(2):
        c.fwd(x, w, b); c.bwd(dy); c.update()
    torch.cuda.synchronize()
    for name in ("hist", "scale", "scale_inv", "sinv", "y", "dx", "dw"):
        assert torch.equal(getattr(a, name).view(torch.uint8), getattr(c, name).view(torch.uint8)), name


def test_weight_caching_across_microbatches_in_a_graph():
    """One microbatch (fwd with the weight's noop flag, lazy transpose of x, bwd) captured once
    and replayed for 3 microbatches x 3 steps, the scale update captured in a second graph run
    at each step's end.  The host sets the device flag to 0 on a step's first microbatch (recast
    W and refresh its transpose cache) and to 1 on the others (reuse the cached FP8 weight, its
    transpose and its private inverse scale), and writes new x / dy (and, between steps, a new W)
    into the captured input buffers.  Every replay is checked against the oracle run through the
    same sequence: FP8 tensors, inverse scales, history and scales bit-exact, y / dx / dW within
    the GEMM tolerance.  W is also changed in place inside a step, which a cached microbatch must
    not see."""
    M, N, K = 256, 384, 512
    lay = Layer(M, N, K)
    x = torch.empty((M, K), device=DEV, dtype=torch.bfloat16)
    w = torch.empty((N, K), device=DEV, dtype=torch.bfloat16)
    b = bf16_dev(S.normal_bf16(S.seed_for(5, 2), (N,), 0.1))
    dy = torch.empty((M, N), device=DEV, dtype=torch.bfloat16)
    bh = S.normal_bf16(S.seed_for(5, 2), (N,), 0.1)
    cap = torch.cuda.Stream()
    g_mb, g_up = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g_mb, stream=cap):
        # forward: x cast without its transpose (x8_t = NULL), W cast+transpose under the flag
        F.fp8_linear_fwd(x, w, b, lay.scale[0:1], lay.hist[0, 0:1], lay.x8, None, lay.sinv[0:1],
                         lay.scale[1:2], lay.hist[0, 1:2], lay.w8, lay.w8t, lay.sinv[1:2], lay.noop, lay.y,
                         stream=cap)
        # backward needs x^T: the lazy transpose of the FP8 x fills the cache
        F.fp8_transpose(lay.x8, lay.x8t, stream=cap)
        lay.bwd(dy, stream=cap)
    with torch.cuda.graph(g_up, stream=cap):
        lay.update(stream=cap)
    for t in (lay.hist, lay.sinv):
        t.zero_()
    lay.scale.fill_(1.0)
    lay.scale_inv.fill_(1.0)
    torch.cuda.synchronize()

    h = np.zeros((16, 3), np.float32)
    s = np.ones(3, np.float32)
    si = np.ones(3, np.float32)
    cached = None            # oracle's cached FP8 weight: (w8, w8t, w_sinv)
    for step in range(3):
        wh = S.normal_bf16(S.seed_for(5, 16 + step), (N, K), 0.05)
        w.copy_(bf16_dev(wh))
        for mb in range(3):
            print(f"weight caching step {step} microbatch {mb}", flush=True)
            xh = S.normal_bf16(S.seed_for(6, 4 * step + mb), (M, K), 1.0)
            dyh = S.normal_bf16(S.seed_for(7, 4 * step + mb), (M, N), 0.01)
            x.copy_(bf16_dev(xh))
            dy.copy_(bf16_dev(dyh))
            if mb == 2:
                w.mul_(-3.0)      # an in-place change a cached microbatch must not see
            first = mb == 0
            lay.noop.fill_(0.0 if first else 1.0)
            g_mb.replay()
            torch.cuda.synchronize()
            # oracle, same sequence
            x8, x_amax, x_sinv = oracle.cast_amax(xh, s[0], F.E4M3, h[0, 0])
            if first:
                w8, w8t, w_amax, w_sinv = oracle.cast_transpose(wh, s[1], F.E4M3, h[0, 1])
                cached = (w8, w8t, w_sinv)
                h[0, 1] = w_amax
            w8, w8t, w_sinv = cached
            h[0, 0] = x_amax
            x8t = oracle.fp8_transpose(x8)
            y = oracle.gemm_bias(x8, F.E4M3, x_sinv, w8, F.E4M3, w_sinv, bh)
            bw = oracle.linear_bwd(dyh, s[2], x8t, x_sinv, w8t, w_sinv)
            # the dy amax folds into the slot across microbatches
            _, _, dy_amax, _ = oracle.cast_transpose(dyh, s[2], F.E5M2, h[0, 2])
            h[0, 2] = dy_amax
            assert np.array_equal(u8_host(lay.x8), x8) and np.array_equal(u8_host(lay.x8t), x8t)
            assert np.array_equal(u8_host(lay.w8), w8) and np.array_equal(u8_host(lay.w8t), w8t)
            assert np.array_equal(u8_host(lay.dy8t), bw["dy8t"])
            assert _same(lay.sinv.cpu().numpy(), [x_sinv, w_sinv, bw["dy_sinv"]])
            assert _same(lay.hist.cpu().numpy(), h), (step, mb)
            gemm_close(to_f64(lay.y), y, bf16_out=True)
            gemm_close(to_f64(lay.dx), bw["dx"], bf16_out=True)
            gemm_close(to_f64(lay.dw), bw["dw"], bf16_out=False)
        g_up.replay()
        torch.cuda.synchronize()
        h, s, si = oracle.scale_update(h, s, si, [0, 0, 1], 0)
        assert _same(lay.hist.cpu().numpy(), h) and _same(lay.scale.cpu().numpy(), s)
        assert _same(lay.scale_inv.cpu().numpy(), si)


@pytest.mark.parametrize("shape", [(256, 384, 512), (100, 256, 256), (128, 200, 256), (37, 24, 48), (8192, 256, 8448)])
@pytest.mark.parametrize("with_xt", [True, False])
def test_linear_fwd_grouped_casts(shape, with_xt):
    """fp8_linear_fwd casts x and W in one launch when both take the same code path (rows % 16
    and cols % 8), else in two; with and without x's transpose cache.  Codes, transposes, amaxes,
    inverse scales and y against the oracle.  At [8192, 8448] x takes its tiles in bands of 16
    row tiles while W, in the same launch, keeps the default order."""
    M, N, K = shape
    print(f"linear fwd grouped casts M={M} N={N} K={K} x_t={with_xt}", flush=True)
    xh = S.normal_bf16(S.seed_for(8, 0), (M, K), 1.0)
    wh = S.normal_bf16(S.seed_for(8, 1), (N, K), 0.5)
    bh = S.normal_bf16(S.seed_for(8, 2), (N,), 0.1)
    lay = Layer(M, N, K)
    lay.scale.copy_(torch.tensor([3.0, 24.0, 1.0]))
    x8t = lay.x8t if with_xt else None
    F.fp8_linear_fwd(bf16_dev(xh), bf16_dev(wh), bf16_dev(bh), lay.scale[0:1], lay.hist[0, 0:1], lay.x8, x8t,
                     lay.sinv[0:1], lay.scale[1:2], lay.hist[0, 1:2], lay.w8, lay.w8t, lay.sinv[1:2], None, lay.y)
    torch.cuda.synchronize()
    fw = oracle.linear_fwd(xh, wh, bh, 3.0, 24.0, want_x_t=with_xt)
    assert np.array_equal(u8_host(lay.x8), fw["x8"])
    if with_xt:
        assert np.array_equal(u8_host(lay.x8t), fw["x8t"])
    assert np.array_equal(u8_host(lay.w8), fw["w8"]) and np.array_equal(u8_host(lay.w8t), fw["w8t"])
    assert _same(lay.hist[0, :2].cpu().numpy(), [fw["x_amax"], fw["w_amax"]])
    assert _same(lay.sinv[:2].cpu().numpy(), [fw["x_sinv"], fw["w_sinv"]])
    gemm_close(to_f64(lay.y), fw["y"], bf16_out=True)
