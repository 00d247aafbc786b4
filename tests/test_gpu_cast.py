"""GPU parity of the cast family against the CPU oracle: FP8 codes, transposes, amax and the
private inverse scale bit for bit; dbias within its summation bound."""
import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, bf16_dev, f32_bits, scalar, u8_host

pytestmark = pytest.mark.gpu


def _run_cast(xh, scale, fmt, amax0=0.0):
    x = bf16_dev(xh)
    out = torch.full((xh.size,), 0xAB, dtype=torch.uint8, device=DEV)
    sinv = scalar(-1.0)
    slot = scalar(amax0)
    F.fp8_cast_amax(x, scalar(scale), fmt, out, sinv, slot)
    torch.cuda.synchronize()
    return u8_host(out).reshape(xh.shape), slot.item(), sinv.cpu().numpy()[0]


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2])
@pytest.mark.parametrize("n", [1, 15, 16, 17, 1000, 4096 * 16 + 5, 1 << 20])
def test_cast_amax_parity(fmt, n):
    print(f"cast_amax fmt={fmt} n={n}", flush=True)
    xh = S.outlier_bf16(S.seed_for(10, fmt), (n,), 1.0)
    for scale in (1.0, 112.0, 0.3, 5000.0, 2.0 ** -20):
        q, amax, sinv = _run_cast(xh, scale, fmt)
        rq, ramax, rsinv = oracle.cast_amax(xh, scale, fmt)
        assert np.array_equal(q, rq), (scale, np.nonzero(q != rq)[0][:5])
        assert f32_bits(amax) == f32_bits(ramax)
        assert f32_bits(sinv) == f32_bits(rsinv)


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2])
def test_cast_specials_nan_inf_and_odd_scales(fmt):
    """NaN / inf inputs and non-finite or zero scales take the exact per-element path."""
    xh = S.normal_bf16(S.seed_for(11, fmt), (4099,), 1.0)
    xh[[3, 100, 2000]] = [0x7F80, 0xFF80, 0x7FC1]     # +inf, -inf, NaN
    xh[[5, 6]] = [0x8000, 0x0000]                      # -0, +0
    for scale in (1.0, 300.0, float("inf"), 0.0):
        q, amax, sinv = _run_cast(xh, scale, fmt)
        rq, ramax, rsinv = oracle.cast_amax(xh, scale, fmt)
        assert np.array_equal(q, rq), (scale, np.nonzero(q != rq)[0][:5], q[q != rq][:5], rq[q != rq][:5])
        assert np.isnan(amax) and np.isnan(ramax)
        assert f32_bits(sinv) == f32_bits(rsinv)
    # NaN scale: every element NaN
    q, _, _ = _run_cast(xh[:64], float("nan"), fmt)
    rq, _, _ = oracle.cast_amax(xh[:64], float("nan"), fmt)
    assert np.array_equal(q, rq)


def test_cast_amax_folds_into_slot():
    xh = S.normal_bf16(S.seed_for(12, 0), (5000,), 1.0)
    _, a_plain, _ = _run_cast(xh, 1.0, F.E4M3)
    _, a_big, _ = _run_cast(xh, 1.0, F.E4M3, amax0=1e9)
    _, a_small, _ = _run_cast(xh, 1.0, F.E4M3, amax0=a_plain / 4)
    assert a_big == np.float32(1e9) and a_small == a_plain


def _run_ct(xh, scale, fmt, noop=None):
    R, C = xh.shape
    x = bf16_dev(xh)
    out = torch.full((R, C), 0xAB, dtype=torch.uint8, device=DEV)
    out_t = torch.full((C, R), 0xCD, dtype=torch.uint8, device=DEV)
    sinv = scalar(-1.0)
    slot = scalar(0.0)
    F.fp8_cast_transpose(x, scalar(scale), fmt, out, out_t, sinv, slot, noop)
    torch.cuda.synchronize()
    return u8_host(out), u8_host(out_t), slot.item(), sinv.cpu().numpy()[0]


# Below 128 tiles of 256 x 256 the launch takes 64 x 64 tiles ((2048, 3840): 120 tiles, the largest
# here); (4112, 2056) and (3000, 3001) take ragged 256 x 256 tiles on the 16-byte path and on
# the element-wise path.
CT_SHAPES = [(1, 1), (3, 5), (16, 8), (128, 128), (130, 264), (144, 264), (257, 383), (1040, 776), (1024, 1024),
             (2048, 3840), (4112, 2056), (3000, 3001)]


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2])
@pytest.mark.parametrize("shape", CT_SHAPES)
def test_cast_transpose_parity(fmt, shape):
    print(f"cast_transpose fmt={fmt} shape={shape}", flush=True)
    xh = S.outlier_bf16(S.seed_for(13, shape[0] % 7), shape, 1.0)
    for scale in (1.0, 37.5):
        q, qt, amax, sinv = _run_ct(xh, scale, fmt)
        rq, rqt, ramax, rsinv = oracle.cast_transpose(xh, scale, fmt)
        assert np.array_equal(q, rq)
        assert np.array_equal(qt, rqt)
        assert f32_bits(amax) == f32_bits(ramax) and f32_bits(sinv) == f32_bits(rsinv)


@pytest.mark.parametrize("fmt,shape", [(F.E4M3, (8192, 8200)), (F.E5M2, (8192, 8193)), (F.E4M3, (12288, 8448))])
def test_cast_transpose_grouped_tile_order(fmt, shape):
    """Tensors whose rows are a multiple of 4096 (at least 8192) with at least 32 column tiles
    take their tiles in bands of 16 row tiles: every tile is covered once, with a ragged column
    tail on the 16-byte path (8200 columns) and on the element-wise path (8193 columns)."""
    print(f"cast_transpose grouped order fmt={fmt} shape={shape}", flush=True)
    xh = S.outlier_bf16(S.seed_for(13, 11 + shape[1] % 5), shape, 1.0)
    q, qt, amax, sinv = _run_ct(xh, 21.0, fmt)
    rq, rqt, ramax, rsinv = oracle.cast_transpose(xh, 21.0, fmt)
    assert np.array_equal(q, rq)
    assert np.array_equal(qt, rqt)
    assert f32_bits(amax) == f32_bits(ramax) and f32_bits(sinv) == f32_bits(rsinv)


def test_cast_transpose_noop_flag():
    xh = S.normal_bf16(S.seed_for(14, 0), (256, 384), 1.0)
    q, qt, amax, sinv = _run_ct(xh, 1.0, F.E4M3, noop=scalar(1.0))
    assert np.all(q == 0xAB) and np.all(qt == 0xCD) and amax == 0.0 and sinv == -1.0
    q, qt, amax, sinv = _run_ct(xh, 1.0, F.E4M3, noop=scalar(0.0))
    rq, rqt, ramax, _ = oracle.cast_transpose(xh, 1.0, F.E4M3)
    assert np.array_equal(q, rq) and np.array_equal(qt, rqt) and amax == ramax


def test_cast_amax_noop_flag():
    xh = S.normal_bf16(S.seed_for(14, 1), (1000,), 1.0)
    x = bf16_dev(xh)
    out = torch.full((1000,), 0xAB, dtype=torch.uint8, device=DEV)
    slot, sinv = scalar(0.0), scalar(-1.0)
    F.fp8_cast_amax(x, scalar(2.0), F.E4M3, out, sinv, slot, scalar(1.0))
    torch.cuda.synchronize()
    assert torch.all(out == 0xAB) and slot.item() == 0.0 and sinv.item() == -1.0


def test_special_tensors_zero_and_tiny():
    """The all-zero tensor and the 2^-133 tensor of the cast_transpose sweep."""
    z = np.zeros((1024, 1024), np.uint16)
    q, qt, amax, _ = _run_ct(z, 1.0, F.E4M3)
    assert amax == 0.0 and np.all(q == 0) and np.all(qt == 0)
    t = S.tiny_bf16(S.seed_for(2, 5), (1024, 1024))
    q, qt, amax, _ = _run_ct(t, 1.0, F.E4M3)
    rq, rqt, ramax, _ = oracle.cast_transpose(t, 1.0, F.E4M3)
    assert f32_bits(amax)[0] == 0x00010000 and f32_bits(amax) == f32_bits(ramax)
    assert np.array_equal(q, rq) and np.array_equal(qt, rqt)


@pytest.mark.parametrize("shape", [(1024, 1024), (4096, 4096), (8192, 12288)])
def test_cast_transpose_sweep_two_steps(shape):
    """Step 1 casts with the initial scale 1 (outliers saturate), the update derives the
    steady-state scale, step 2 casts with it.  Both steps bit-exact."""
    print(f"cast_transpose sweep {shape}", flush=True)
    idx = {(1024, 1024): 0, (4096, 4096): 1, (8192, 12288): 2}[shape]
    xh = S.outlier_bf16(S.seed_for(1, idx), shape, 1.0)
    L = 16
    hist = torch.zeros((L, 1), dtype=torch.float32, device=DEV)
    scale = torch.ones(1, dtype=torch.float32, device=DEV)
    sinv_m = torch.ones(1, dtype=torch.float32, device=DEV)
    x = bf16_dev(xh)
    R, C = shape
    out = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    out_t = torch.empty((C, R), dtype=torch.uint8, device=DEV)
    tsinv = scalar(0.0)
    F.fp8_cast_transpose(x, scale, F.E4M3, out, out_t, tsinv, hist[0, 0:1])
    h1 = hist.clone()
    F.fp8_scale_update(hist, scale, sinv_m, [F.E4M3], 0)
    s2 = scale.clone()
    F.fp8_cast_transpose(x, scale, F.E4M3, out, out_t, tsinv, hist[0, 0:1])
    torch.cuda.synchronize()
    # oracle, step 1
    rq1, rqt1, ra1, _ = oracle.cast_transpose(xh, 1.0, F.E4M3)
    assert f32_bits(h1[0, 0].item()) == f32_bits(ra1)
    hh, ss, si = oracle.scale_update(h1.cpu().numpy(), np.ones(1, np.float32), np.ones(1, np.float32), [0], 0)
    assert f32_bits(s2.cpu().numpy()) == f32_bits(ss)
    rq2, rqt2, ra2, rs2 = oracle.cast_transpose(xh, ss[0], F.E4M3)
    assert np.array_equal(u8_host(out), rq2)
    assert np.array_equal(u8_host(out_t), rqt2)
    assert f32_bits(tsinv.cpu().numpy()) == f32_bits(rs2)
    assert f32_bits(hist[0, 0].item()) == f32_bits(ra2)


def _dbias_bound(dyh):
    return 1e-5 * np.abs(S.bf16_bits_to_f64(dyh)).sum(axis=0) + 1e-30


@pytest.mark.parametrize("shape", [(1, 1), (3, 5), (130, 264), (144, 264), (257, 383), (8192, 4096), (17297, 136),
                                   (8192, 8200)])
def test_dbias_cast_transpose_parity(shape):
    print(f"dbias_cast_transpose {shape}", flush=True)
    R, C = shape
    dyh = S.normal_bf16(S.seed_for(3, R % 5), shape, 0.01)
    dy = bf16_dev(dyh)
    out = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    out_t = torch.empty((C, R), dtype=torch.uint8, device=DEV)
    db = torch.full((C,), 7.0, dtype=torch.float32, device=DEV)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), dtype=torch.uint8, device=DEV)
    slot, sinv = scalar(0.0), scalar(0.0)
    scale = 4096.0
    F.fp8_dbias_cast_transpose(dy, scalar(scale), F.E5M2, out, out_t, db, ws, sinv, slot)
    torch.cuda.synchronize()
    rq, rqt, ra, rs, rdb = oracle.dbias_cast_transpose(dyh, scale, F.E5M2)
    assert np.array_equal(u8_host(out), rq) and np.array_equal(u8_host(out_t), rqt)
    assert f32_bits(slot.item()) == f32_bits(ra) and f32_bits(sinv.item()) == f32_bits(rs)
    got = db.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - rdb) <= _dbias_bound(dyh))


@pytest.mark.parametrize("R", [8192, 17297])
def test_dbias_constant_columns_exact(R):
    """0.5 everywhere: every partial and final sum is exact, so dbias = R / 2 exactly (68 row
    tiles for R = 17297: whole 16-tile batches of the reduction plus single-tile remainders)."""
    C = 64
    dyh = np.full((R, C), 0x3F00, np.uint16)
    dy = bf16_dev(dyh)
    out = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    out_t = torch.empty((C, R), dtype=torch.uint8, device=DEV)
    db = torch.empty((C,), dtype=torch.float32, device=DEV)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), dtype=torch.uint8, device=DEV)
    F.fp8_dbias_cast_transpose(dy, scalar(1.0), F.E5M2, out, out_t, db, ws)
    torch.cuda.synchronize()
    assert torch.all(db == R / 2)


def test_dbias_deterministic():
    R, C = 2048, 1024
    dyh = S.normal_bf16(S.seed_for(3, 9), (R, C), 0.01)
    dy = bf16_dev(dyh)
    out = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    out_t = torch.empty((C, R), dtype=torch.uint8, device=DEV)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), dtype=torch.uint8, device=DEV)
    a = torch.empty((C,), dtype=torch.float32, device=DEV)
    b = torch.empty((C,), dtype=torch.float32, device=DEV)
    F.fp8_dbias_cast_transpose(dy, scalar(1.0), F.E5M2, out, out_t, a, ws)
    F.fp8_dbias_cast_transpose(dy, scalar(1.0), F.E5M2, out, out_t, b, ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


COUNTER_BYTES = 1024   # FP8DS_DBIAS_COUNTER_BYTES: the strip counters at the start of the workspace


@pytest.mark.parametrize("shape", [(2048, 1024), (300, 700), (8192, 4096)])
def test_dbias_workspace_garbage_reuse_and_graph(shape):
    """Whatever the partial-sum area holds on entry (random bytes, all ones, zeros), with the
    counter bytes zero, dbias is the same bits, call after call on the same workspace, and on
    every replay of a captured graph; every call leaves the counter bytes zero.  (2048, 1024) and
    (8192, 4096) take the one-launch strip form, (300, 700) the tile kernel + reduction.)"""
    R, C = shape
    print(f"dbias workspace reuse {shape}", flush=True)
    dyh = S.normal_bf16(S.seed_for(3, 10), (R, C), 0.01)
    dy = bf16_dev(dyh)
    out = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    out_t = torch.empty((C, R), dtype=torch.uint8, device=DEV)
    nbytes = F.fp8_dbias_workspace_bytes(R, C)
    ws = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    ref = torch.empty((C,), dtype=torch.float32, device=DEV)
    F.fp8_dbias_cast_transpose(dy, scalar(1.0), F.E5M2, out, out_t, ref, ws)
    torch.cuda.synchronize()
    db = oracle.dbias(dyh)
    assert np.all(np.abs(ref.cpu().numpy() - db) <= 1e-5 * np.abs(S.bf16_bits_to_f64(dyh)).sum(0) + 1e-30)
    assert not torch.any(ws[:COUNTER_BYTES])
    fills = [torch.from_numpy(S.random_bytes(S.seed_for(3, 11), (nbytes + 64,))).to(DEV),
             torch.full((nbytes + 64,), 0xFF, dtype=torch.uint8, device=DEV),
             torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)]
    for k, fill in enumerate(fills):
        ws.copy_(fill)
        ws[:COUNTER_BYTES].zero_()
        for rep in range(3):
            got = torch.full((C,), float("nan"), dtype=torch.float32, device=DEV)
            F.fp8_dbias_cast_transpose(dy, scalar(1.0), F.E5M2, out, out_t, got, ws)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (k, rep)
            assert not torch.any(ws[:COUNTER_BYTES]), (k, rep)
    # captured once, replayed
    got = torch.zeros((C,), dtype=torch.float32, device=DEV)
    one = scalar(1.0)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        F.fp8_dbias_cast_transpose(dy, one, F.E5M2, out, out_t, got, ws, stream=cap)
    for rep in range(4):
        got.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), rep
        assert not torch.any(ws[:COUNTER_BYTES]), rep


# Shapes of whole 256 x 256 tiles that take the one-launch strip form: one tile per block
# ([256, 256], [768, 512], [4096, 4096]), two per block ([8192, 4096]; [2560, 12288]: 48 strips x
# 5 slots = 240 blocks for 10 row tiles; [512, 65536]: 256 strips, every counter in use), four
# per block ([4096, 16384]: 64 strips x 4 slots).
@pytest.mark.parametrize("shape", [(256, 256), (768, 512), (4096, 4096), (2560, 12288), (512, 65536), (4096, 16384)])
@pytest.mark.parametrize("fmt", [1, 0])
def test_dbias_strip_form_parity(shape, fmt):
    print(f"dbias strip form {shape} fmt {fmt}", flush=True)
    R, C = shape
    dyh = S.normal_bf16(S.seed_for(3, 40 + R % 7), shape, 0.01)
    dy = bf16_dev(dyh)
    out = torch.full((R, C), 0xA5, dtype=torch.uint8, device=DEV)
    out_t = torch.full((C, R), 0x5A, dtype=torch.uint8, device=DEV)
    db = torch.full((C,), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), dtype=torch.uint8, device=DEV)
    slot, sinv = scalar(0.0), scalar(0.0)
    scale = 4096.0 if fmt == F.E5M2 else 64.0
    F.fp8_dbias_cast_transpose(dy, scalar(scale), fmt, out, out_t, db, ws, sinv, slot)
    torch.cuda.synchronize()
    rq, rqt, ra, rs, rdb = oracle.dbias_cast_transpose(dyh, scale, fmt)
    assert np.array_equal(u8_host(out), rq) and np.array_equal(u8_host(out_t), rqt)
    assert f32_bits(slot.item()) == f32_bits(ra) and f32_bits(sinv.item()) == f32_bits(rs)
    assert np.all(np.abs(db.cpu().numpy().astype(np.float64) - rdb) <= _dbias_bound(dyh))
    assert not torch.any(ws[:COUNTER_BYTES])


@pytest.mark.parametrize("shape", [(1024, 512), (768, 65536)])
@pytest.mark.parametrize("scale", [2.0 ** 10, 0.0, float("inf")])
def test_dbias_strip_form_specials(scale, shape):
    """Infinities, NaNs and saturating values in a strip-form tensor (one tile per block, and
    three per block at [768, 65536]), and scales that are not plain (zero, infinite): the exact
    path re-reads the rows; codes, amax and inverse scale must equal the oracle's; dbias is
    checked where the column holds no non-finite value."""
    R, C = shape
    print(f"dbias strip form specials {shape} scale {scale}", flush=True)
    dyh = S.normal_bf16(S.seed_for(3, 50), (R, C), 1.0)
    for (i, j, v) in [(3, 5, 0x7F80), (700, 5, 0xFF80), (511, 300, 0x7FC0), (R - 1, C - 1, 0x7F7F), (9, 0, 0xFF7F),
                      (256, 256, 0x4780)]:
        dyh[i, j] = v
    dy = bf16_dev(dyh)
    out = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    out_t = torch.empty((C, R), dtype=torch.uint8, device=DEV)
    db = torch.empty((C,), dtype=torch.float32, device=DEV)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), dtype=torch.uint8, device=DEV)
    slot, sinv = scalar(0.0), scalar(0.0)
    F.fp8_dbias_cast_transpose(dy, scalar(scale), F.E5M2, out, out_t, db, ws, sinv, slot)
    torch.cuda.synchronize()
    rq, rqt, ra, rs, rdb = oracle.dbias_cast_transpose(dyh, scale, F.E5M2)
    assert np.array_equal(u8_host(out), rq) and np.array_equal(u8_host(out_t), rqt)
    assert f32_bits(slot.item()) == f32_bits(ra) and f32_bits(sinv.item()) == f32_bits(rs)
    got = db.cpu().numpy().astype(np.float64)
    finite = np.all(np.isfinite(S.bf16_bits_to_f64(dyh)), axis=0)
    assert np.all(np.abs(got[finite] - rdb[finite]) <= _dbias_bound(dyh)[finite])
    assert not torch.any(ws[:COUNTER_BYTES])


def test_dbias_workspace_shared_by_both_forms():
    """One workspace used in turn by a strip-form shape and a tile-kernel shape, new data every
    call: each call's dbias matches the oracle (no partial or counter left by the other form)."""
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(2048, 1024), dtype=torch.uint8, device=DEV)
    for k, (R, C) in enumerate([(2048, 1024), (300, 700), (2048, 1024), (1000, 1024), (512, 512)]):
        print(f"dbias shared workspace call {k} {(R, C)}", flush=True)
        assert F.fp8_dbias_workspace_bytes(R, C) <= ws.numel()
        dyh = S.normal_bf16(S.seed_for(3, 60 + k), (R, C), 0.01)
        out = torch.empty((R, C), dtype=torch.uint8, device=DEV)
        out_t = torch.empty((C, R), dtype=torch.uint8, device=DEV)
        db = torch.full((C,), float("nan"), dtype=torch.float32, device=DEV)
        F.fp8_dbias_cast_transpose(bf16_dev(dyh), scalar(1.0), F.E5M2, out, out_t, db, ws)
        torch.cuda.synchronize()
        assert np.all(np.abs(db.cpu().numpy().astype(np.float64) - oracle.dbias(dyh)) <= _dbias_bound(dyh)), k
        assert not torch.any(ws[:COUNTER_BYTES]), k


def test_empty_inputs_launch_nothing():
    x = torch.empty((0,), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((0,), dtype=torch.uint8, device=DEV)
    sinv = scalar(-1.0)
    F.fp8_cast_amax(x, scalar(1.0), F.E4M3, out, sinv, None)
    x2 = torch.empty((0, 5), dtype=torch.bfloat16, device=DEV)
    F.fp8_cast_transpose(x2, scalar(1.0), F.E4M3, torch.empty((0, 5), dtype=torch.uint8, device=DEV),
                         torch.empty((5, 0), dtype=torch.uint8, device=DEV), sinv, None)
    db = torch.full((5,), 3.0, dtype=torch.float32, device=DEV)
    F.fp8_dbias_cast_transpose(x2, scalar(1.0), F.E5M2, None, None, db, None)
    torch.cuda.synchronize()
    assert sinv.item() == -1.0 and torch.all(db == 0.0)


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2])
def test_cast_exhaustive_bf16_patterns_times_scales(fmt):
    """All 65536 bfloat16 bit patterns (every sign, exponent and mantissa, subnormals, +-0,
    +-inf and NaNs) times 40 scales from 2^-30 to 2^30 plus odd values: the cast's whole input
    domain for each scale, through both the 1-D cast and the cast+transpose, bit-exact."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    scales = [float(v) for v in 2.0 ** np.linspace(-30, 30, 33)] + [1.0, 3.0, 0.1, 112.0, 448.0, 57344.0, 1e-38]
    x2 = bf16_dev(allb.reshape(256, 256))
    x1 = bf16_dev(allb)
    for sc in scales:
        out = torch.empty(65536, dtype=torch.uint8, device=DEV)
        F.fp8_cast_amax(x1, scalar(sc), fmt, out)
        q = torch.empty((256, 256), dtype=torch.uint8, device=DEV)
        qt = torch.empty((256, 256), dtype=torch.uint8, device=DEV)
        F.fp8_cast_transpose(x2, scalar(sc), fmt, q, qt)
        torch.cuda.synchronize()
        ref, _, _ = oracle.cast_amax(allb, sc, fmt)
        got = u8_host(out)
        assert np.array_equal(got, ref), (sc, np.nonzero(got != ref)[0][:5])
        assert np.array_equal(u8_host(q).reshape(-1), ref), sc
        assert np.array_equal(u8_host(qt), ref.reshape(256, 256).T), sc
