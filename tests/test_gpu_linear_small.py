"""The one-launch forward of small layers (fp8_linear_fwd when K is 256, 512 or 1024, N % 16 ==
0, no x transpose, at most 256 x 256 / K output blocks of 64 x 64 and fewer than 40 of 256 x 256;
32 x 32 tiles up to 128 blocks of 64 x 64) against the
individual calls (cast of x, cast+transpose of W, GEMM + bias: every output bit for bit) and
against the oracle (codes, amaxes and inverse scales exact, y within the GEMM tolerance),
including the cached-weight flag, non-finite inputs, scales that are not plain, graph replay, and
the layers just outside the rule (which take the cast launch + GEMM launch)."""
import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, bf16_dev, f32_bits, gemm_close, kernel_names, to_f64, u8_host

pytestmark = pytest.mark.gpu

U8 = dict(device=DEV, dtype=torch.uint8)
F32 = dict(device=DEV, dtype=torch.float32)


class Fwd:
    """Outputs of one forward: codes, transposed weight codes, amax slots, inverse scales, y."""

    def __init__(self, M, N, K):
        self.x8, self.w8, self.w8t = torch.full((M, K), 0xA5, **U8), torch.full((N, K), 0xA5, **U8), \
            torch.full((K, N), 0x5A, **U8)
        self.am = torch.zeros(2, **F32)
        self.sinv = torch.full((2,), -1.0, **F32)
        self.y = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16)


def _layer_call(x, w, b, scales, o, noop=None, stream=None):
    F.fp8_linear_fwd(x, w, b, scales[0:1], o.am[0:1], o.x8, None, o.sinv[0:1], scales[1:2], o.am[1:2], o.w8, o.w8t,
                     o.sinv[1:2], noop, o.y, stream=stream)


def _primitives(x, w, b, scales, o):
    F.fp8_cast_amax(x, scales[0:1], F.E4M3, o.x8, o.sinv[0:1], o.am[0:1])
    F.fp8_cast_transpose(w, scales[1:2], F.E4M3, o.w8, o.w8t, o.sinv[1:2], o.am[1:2])
    F.fp8_gemm_bias(o.x8, F.E4M3, o.sinv[0:1], o.w8, F.E4M3, o.sinv[1:2], b, o.y)


def _equal(a, b):
    for name in ("x8", "w8", "w8t"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert torch.equal(a.am.view(torch.int32), b.am.view(torch.int32))
    assert torch.equal(a.sinv.view(torch.int32), b.sinv.view(torch.int32))
    assert torch.equal(a.y.view(torch.int16), b.y.view(torch.int16))


# the small layer [128, 256] x [256, 256], a ragged M, a narrow N, a wide N, both tile sizes and
# the largest block count (16 x 16 blocks of 64 x 64); K = 512 and 1024 inside their block
# limits; then layers outside the rule: K = 512 at 256 blocks, K = 8192, 288 blocks
@pytest.mark.parametrize("shape", [(128, 256, 256), (100, 48, 256), (64, 1024, 256), (130, 16, 256), (512, 1024, 256),
                                   (1024, 768, 256), (1024, 832, 256), (1024, 1024, 256),
                                   (100, 48, 512), (512, 1024, 512), (130, 16, 1024), (512, 512, 1024),
                                   (1024, 1024, 512), (130, 16, 8192), (768, 1536, 256)])
@pytest.mark.parametrize("with_bias", [True, False])
def test_one_launch_equals_primitives_and_oracle(shape, with_bias):
    M, N, K = shape
    print(f"one-launch forward {shape} bias={with_bias}", flush=True)
    xh = S.normal_bf16(S.seed_for(9, 0), (M, K), 1.0)
    wh = S.normal_bf16(S.seed_for(9, 1), (N, K), 1.0)
    bh = S.normal_bf16(S.seed_for(9, 2), (N,), 0.1)
    x, w = bf16_dev(xh), bf16_dev(wh)
    b = bf16_dev(bh) if with_bias else None
    scales = torch.tensor([2.0, 48.0], **F32)
    a, r = Fwd(M, N, K), Fwd(M, N, K)
    _layer_call(x, w, b, scales, a)
    _primitives(x, w, b, scales, r)
    torch.cuda.synchronize()
    _equal(a, r)
    fw = oracle.linear_fwd(xh, wh, bh if with_bias else None, 2.0, 48.0, want_x_t=False)
    assert np.array_equal(u8_host(a.x8), fw["x8"])
    assert np.array_equal(u8_host(a.w8), fw["w8"]) and np.array_equal(u8_host(a.w8t), fw["w8t"])
    assert np.array_equal(f32_bits(a.am.cpu().numpy()), f32_bits(np.array([fw["x_amax"], fw["w_amax"]], np.float32)))
    assert np.array_equal(f32_bits(a.sinv.cpu().numpy()), f32_bits(np.array([fw["x_sinv"], fw["w_sinv"]], np.float32)))
    gemm_close(to_f64(a.y), fw["y"], bf16_out=True)


@pytest.mark.parametrize("shape", [(128, 256, 256), (1024, 1024, 256), (128, 256, 1024)])
@pytest.mark.parametrize("xs, ws", [(0.0, 1.0), (float("inf"), 2.0), (1.0, 1e30)])
def test_one_launch_specials(xs, ws, shape):
    """Infinities, NaNs and saturating values in x and W, a zero or infinite x scale, a weight
    scale that saturates everything (both tile sizes of the one-launch kernel): every
    output equals the individual calls' (y included, whatever it holds)."""
    M, N, K = shape
    print(f"one-launch specials {shape} xs={xs} ws={ws}", flush=True)
    xh = S.normal_bf16(S.seed_for(9, 3), (M, K), 1.0)
    wh = S.normal_bf16(S.seed_for(9, 4), (N, K), 1.0)
    for (i, j, v) in [(0, 0, 0x7F80), (5, 200, 0xFF80), (127, 255, 0x7FC0), (64, 31, 0x7F7F)]:
        xh[i, j] = v
    for (i, j, v) in [(3, 3, 0x7F80), (255, 128, 0x7FC0), (17, 0, 0xFF7F)]:
        wh[i, j] = v
    bh = S.normal_bf16(S.seed_for(9, 5), (N,), 0.1)
    x, w, b = bf16_dev(xh), bf16_dev(wh), bf16_dev(bh)
    scales = torch.tensor([xs, ws], **F32)
    a, r = Fwd(M, N, K), Fwd(M, N, K)
    _layer_call(x, w, b, scales, a)
    _primitives(x, w, b, scales, r)
    torch.cuda.synchronize()
    for name in ("x8", "w8", "w8t"):
        assert torch.equal(getattr(a, name), getattr(r, name)), name
    assert torch.equal(a.am.view(torch.int32), r.am.view(torch.int32))
    assert torch.equal(a.sinv.view(torch.int32), r.sinv.view(torch.int32))
    assert torch.equal(a.y.view(torch.int16), r.y.view(torch.int16))
    q, am, si = oracle.cast_amax(xh, xs, F.E4M3)
    assert np.array_equal(u8_host(a.x8), q) and f32_bits(a.am[0].item()) == f32_bits(am)


@pytest.mark.parametrize("shape", [(128, 256, 256), (1024, 1024, 256)])
def test_one_launch_without_amax_slots(shape):
    """The amax slots are optional: without them (NULL) the one-launch forward writes the same
    codes, inverse scales and y as with them."""
    M, N, K = shape
    print(f"one-launch forward without amax slots {shape}", flush=True)
    x = bf16_dev(S.normal_bf16(S.seed_for(9, 40), (M, K), 1.0))
    w = bf16_dev(S.normal_bf16(S.seed_for(9, 41), (N, K), 1.0))
    b = bf16_dev(S.normal_bf16(S.seed_for(9, 42), (N,), 0.1))
    scales = torch.tensor([2.0, 32.0], **F32)
    a, r = Fwd(M, N, K), Fwd(M, N, K)
    F.fp8_linear_fwd(x, w, b, scales[0:1], None, a.x8, None, a.sinv[0:1], scales[1:2], None, a.w8, a.w8t,
                     a.sinv[1:2], None, a.y)
    _layer_call(x, w, b, scales, r)
    torch.cuda.synchronize()
    for name in ("x8", "w8", "w8t"):
        assert torch.equal(getattr(a, name), getattr(r, name)), name
    assert torch.equal(a.sinv.view(torch.int32), r.sinv.view(torch.int32))
    assert torch.equal(a.y.view(torch.int16), r.y.view(torch.int16))
    assert not torch.any(a.am)    # untouched


@pytest.mark.parametrize("shape", [(128, 256, 256), (1024, 1024, 256), (128, 256, 512)])
def test_one_launch_cached_weight_and_graph(shape):
    """With the weight's flag at 1 the layer multiplies by the cached codes and inverse scale and
    writes nothing of W (a changed bfloat16 W is not seen); captured once and replayed with the
    flag and x changing between replays, every replay equals the individual calls (both tile
    sizes of the one-launch kernel)."""
    M, N, K = shape
    xh = [S.normal_bf16(S.seed_for(9, 10 + k), (M, K), 1.0) for k in range(3)]
    wh0 = S.normal_bf16(S.seed_for(9, 20), (N, K), 1.0)
    wh1 = S.normal_bf16(S.seed_for(9, 21), (N, K), 3.0)
    bh = S.normal_bf16(S.seed_for(9, 22), (N,), 0.1)
    x = torch.empty((M, K), device=DEV, dtype=torch.bfloat16)
    w = bf16_dev(wh0)
    b = bf16_dev(bh)
    scales = torch.tensor([4.0, 16.0], **F32)
    noop = torch.zeros(1, **F32)
    a = Fwd(M, N, K)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        _layer_call(x, w, b, scales, a, noop=noop, stream=cap)
    r = Fwd(M, N, K)
    for k, flag in enumerate([0.0, 1.0, 1.0]):
        print(f"cached weight replay {k} flag {flag}", flush=True)
        x.copy_(bf16_dev(xh[k]))
        if k == 2:
            w.copy_(bf16_dev(wh1))       # a cached forward must not see this
        noop.fill_(flag)
        a.am.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # reference: the individual calls, the weight cast only when the flag is clear
        r.am.zero_()
        F.fp8_cast_amax(x, scales[0:1], F.E4M3, r.x8, r.sinv[0:1], r.am[0:1])
        if flag == 0.0:
            F.fp8_cast_transpose(w, scales[1:2], F.E4M3, r.w8, r.w8t, r.sinv[1:2], r.am[1:2])
        F.fp8_gemm_bias(r.x8, F.E4M3, r.sinv[0:1], r.w8, F.E4M3, r.sinv[1:2], b, r.y)
        torch.cuda.synchronize()
        _equal(a, r)
        fw = oracle.linear_fwd(xh[k], wh0, bh, 4.0, 16.0, want_x_t=False)
        assert np.array_equal(u8_host(a.w8), fw["w8"]) and np.array_equal(u8_host(a.w8t), fw["w8t"])
        gemm_close(to_f64(a.y), fw["y"], bf16_out=True)


@pytest.mark.parametrize("shape, one", [((128, 256, 256), "k_linear_fwd_small<32, 256>"),
                                        ((512, 1024, 256), "k_linear_fwd_small<32, 256>"),
                                        ((768, 768, 256), "k_linear_fwd_small<64, 256>"),
                                        ((1024, 1024, 256), "k_linear_fwd_small<64, 256>"),
                                        ((128, 256, 512), "k_linear_fwd_small<32, 512>"),
                                        ((512, 512, 1024), "k_linear_fwd_small<32, 1024>"),
                                        ((1024, 1024, 512), None), ((1024, 1024, 1024), None), ((128, 256, 768), None),
                                        ((768, 1536, 256), None)])
def test_dispatch_rule_launches(shape, one):
    """Inside the rule the forward is a single launch of k_linear_fwd_small<TILE, K> (32 x 32
    tiles up to 128 blocks of 64 x 64, 64 x 64 beyond); outside it the cast launch and the GEMM
    launch (all give the same bits; this checks which one ran)."""
    M, N, K = shape
    x = bf16_dev(S.normal_bf16(S.seed_for(9, 30), (M, K), 1.0))
    w = bf16_dev(S.normal_bf16(S.seed_for(9, 31), (N, K), 1.0))
    scales = torch.tensor([2.0, 48.0], **F32)
    o = Fwd(M, N, K)
    _layer_call(x, w, None, scales, o)
    names = kernel_names(lambda: _layer_call(x, w, None, scales, o))
    if names is None:
        pytest.skip("the profiler recorded no GPU kernels on this build")
    fp8 = [n for n in names if "fp8ds" in n]
    print(f"dispatch {shape}: {fp8}", flush=True)
    if one:
        assert len(fp8) == 1 and one in fp8[0]
    else:
        assert not any("k_linear_fwd" in n for n in fp8) and len(fp8) == 2
