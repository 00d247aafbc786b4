"""Seeded random shapes through the size-dependent code paths: cast+transpose (64 x 64 tiles below
128 tiles of 256 x 256, else 256 x 256; the 16-byte path and the element-wise path), dbias + cast
+ transpose (the one-launch strip form for tensors of whole tiles with at most two tiles per CU,
or three or four evenly, else the tile kernel + reduction), and the forward of a layer (one launch for small layers,
else the cast launch + GEMM), and the GEMM (both MFMA families, small-problem and 256 x 256
kernels, all format pairs, bfloat16 and float32 output).  Every code, transpose, amax and
inverse scale against the oracle bit for bit; dbias, y and D within their bounds."""
import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, bf16_dev, f32_bits, gemm_close, kernel_names, scalar, to_f64, u8_host

pytestmark = pytest.mark.gpu


def _draw(seed, k, lo, hi):
    """k seeded integers in [lo, hi]."""
    return [lo + int(u * (hi - lo + 1)) for u in S.uniform(seed, 0, k)]


def _ct_shapes():
    rows = _draw(S.seed_for(10, 0), 8, 1, 6000) + _draw(S.seed_for(10, 14), 4, 3000, 9000)
    cols = _draw(S.seed_for(10, 1), 8, 1, 6000) + _draw(S.seed_for(10, 15), 4, 3000, 9000)
    # every other shape rounded to the 16-byte path's multiples
    return [(r - r % 16 or 16, c - c % 8 or 8) if i % 2 else (r, c) for i, (r, c) in enumerate(zip(rows, cols))]


@pytest.mark.parametrize("shape", _ct_shapes())
def test_cast_transpose_random_shapes(shape):
    R, C = shape
    print(f"cast_transpose random shape {shape}", flush=True)
    xh = S.outlier_bf16(S.seed_for(10, 2 + R % 7), shape, 1.0)
    x = bf16_dev(xh)
    out = torch.full((R, C), 0xAB, dtype=torch.uint8, device=DEV)
    out_t = torch.full((C, R), 0xCD, dtype=torch.uint8, device=DEV)
    sinv, slot = scalar(-1.0), scalar(0.0)
    F.fp8_cast_transpose(x, scalar(3.0), F.E4M3, out, out_t, sinv, slot)
    torch.cuda.synchronize()
    rq, rqt, ra, rs = oracle.cast_transpose(xh, 3.0, F.E4M3)
    assert np.array_equal(u8_host(out), rq) and np.array_equal(u8_host(out_t), rqt)
    assert f32_bits(slot.item()) == f32_bits(ra) and f32_bits(sinv.item()) == f32_bits(rs)


def _dbias_shapes():
    # whole-tile shapes: tiles_r in [1, 32], tiles_c in [1, 40], some with at most 512 tiles and
    # two tiles per CU (strip form), some beyond (tile kernel); whole-tile shapes with three or
    # four tiles per CU, even (strip form) and uneven or with few strips (tile kernel); plus
    # ragged shapes
    tr = _draw(S.seed_for(10, 3), 6, 1, 32)
    tc = _draw(S.seed_for(10, 4), 6, 1, 40)
    whole = [(256 * a, 256 * b) for a, b in zip(tr, tc)]
    deep = [(8192, 8192), (12288, 4096), (1024, 65536), (8192, 6144), (32768, 2048), (768, 65536)]
    ragged = list(zip(_draw(S.seed_for(10, 5), 3, 1, 5000), _draw(S.seed_for(10, 6), 3, 1, 3000)))
    return whole + deep + ragged


@pytest.mark.parametrize("shape", _dbias_shapes())
def test_dbias_random_shapes(shape):
    R, C = shape
    print(f"dbias random shape {shape}", flush=True)
    dyh = S.normal_bf16(S.seed_for(10, 7 + R % 5), shape, 0.01)
    dy = bf16_dev(dyh)
    out = torch.full((R, C), 0xAB, dtype=torch.uint8, device=DEV)
    out_t = torch.full((C, R), 0xCD, dtype=torch.uint8, device=DEV)
    db = torch.full((C,), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), dtype=torch.uint8, device=DEV)
    sinv, slot = scalar(-1.0), scalar(0.0)
    rq, rqt, ra, rs, rdb = oracle.dbias_cast_transpose(dyh, 2048.0, F.E5M2)
    for rep in range(2):                      # the second call reuses the workspace as left
        F.fp8_dbias_cast_transpose(dy, scalar(2048.0), F.E5M2, out, out_t, db, ws, sinv, slot)
        torch.cuda.synchronize()
        assert np.array_equal(u8_host(out), rq) and np.array_equal(u8_host(out_t), rqt), rep
        assert f32_bits(slot.item()) == f32_bits(ra) and f32_bits(sinv.item()) == f32_bits(rs), rep
        bound = 1e-5 * np.abs(S.bf16_bits_to_f64(dyh)).sum(axis=0) + 1e-30
        assert np.all(np.abs(db.cpu().numpy().astype(np.float64) - rdb) <= bound), rep
        assert not torch.any(ws[:1024]), rep


@pytest.mark.parametrize("shape, strips", [((8192, 4096), True), ((8192, 8192), True), ((12288, 4096), True),
                                           ((768, 65536), True), ((8192, 6144), False), ((32768, 2048), False),
                                           ((4096, 12288), False), ((8448, 4096), False)])
def test_dbias_dispatch_rule_launches(shape, strips):
    """Whole-tile tensors with at most two tiles per CU, or three or four per CU for every CU
    with at least 16 tile columns, run as the single k_dbias_strips launch; the others as the
    tile kernel + k_dbias_reduce (the same codes either way; this checks which one ran)."""
    R, C = shape
    dy = bf16_dev(S.normal_bf16(S.seed_for(10, 30), shape, 0.01))
    out = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    out_t = torch.empty((C, R), dtype=torch.uint8, device=DEV)
    db = torch.empty((C,), dtype=torch.float32, device=DEV)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), dtype=torch.uint8, device=DEV)
    sinv, slot, sc = scalar(0.0), scalar(0.0), scalar(2048.0)
    call = lambda: F.fp8_dbias_cast_transpose(dy, sc, F.E5M2, out, out_t, db, ws, sinv, slot)
    call()
    names = kernel_names(call)
    if names is None:
        pytest.skip("the profiler recorded no GPU kernels on this build")
    fp8 = [n for n in names if "fp8ds" in n]
    print(f"dbias dispatch {shape}: {fp8}", flush=True)
    if strips:
        assert len(fp8) == 1 and "k_dbias_strips" in fp8[0]
    else:
        assert len(fp8) == 2 and not any("k_dbias_strips" in n for n in fp8)
        assert "k_dbias_reduce" in fp8[1]
    assert not torch.any(ws[:1024])


def _fwd_shapes():
    ms = _draw(S.seed_for(10, 8), 6, 1, 3000)
    ns = [16 * n for n in _draw(S.seed_for(10, 9), 6, 1, 80)]
    ks = [256 * k for k in _draw(S.seed_for(10, 10), 6, 1, 8)]
    return list(zip(ms, ns, ks))


@pytest.mark.parametrize("shape", _fwd_shapes())
def test_linear_fwd_random_shapes(shape):
    M, N, K = shape
    print(f"linear fwd random shape {shape}", flush=True)
    xh = S.normal_bf16(S.seed_for(10, 11), (M, K), 1.0)
    wh = S.normal_bf16(S.seed_for(10, 12), (N, K), 0.5)
    bh = S.normal_bf16(S.seed_for(10, 13), (N,), 0.1)
    u8 = dict(dtype=torch.uint8, device=DEV)
    x8, w8, w8t = torch.empty((M, K), **u8), torch.empty((N, K), **u8), torch.empty((K, N), **u8)
    am, si = torch.zeros(2, device=DEV), torch.zeros(2, device=DEV)
    sc = torch.tensor([2.0, 30.0], device=DEV)
    y = torch.empty((M, N), device=DEV, dtype=torch.bfloat16)
    F.fp8_linear_fwd(bf16_dev(xh), bf16_dev(wh), bf16_dev(bh), sc[0:1], am[0:1], x8, None, si[0:1], sc[1:2], am[1:2],
                     w8, w8t, si[1:2], None, y)
    torch.cuda.synchronize()
    fw = oracle.linear_fwd(xh, wh, bh, 2.0, 30.0, want_x_t=False)
    assert np.array_equal(u8_host(x8), fw["x8"])
    assert np.array_equal(u8_host(w8), fw["w8"]) and np.array_equal(u8_host(w8t), fw["w8t"])
    assert np.array_equal(f32_bits(am.cpu().numpy()), f32_bits(np.array([fw["x_amax"], fw["w_amax"]], np.float32)))
    assert np.array_equal(f32_bits(si.cpu().numpy()), f32_bits(np.array([fw["x_sinv"], fw["w_sinv"]], np.float32)))
    gemm_close(to_f64(y), fw["y"], bf16_out=True)


def _gemm_cases():
    ms = _draw(S.seed_for(10, 16), 10, 1, 3000)
    ns = _draw(S.seed_for(10, 17), 10, 1, 3000)
    # K: five multiples of 16 (the 32 x 32 x 64 family unless K % 256 == 0), five of 256
    ks = [16 * k for k in _draw(S.seed_for(10, 18), 5, 1, 160)] + [256 * k for k in _draw(S.seed_for(10, 19), 5, 1, 10)]
    pairs = _draw(S.seed_for(10, 20), 10, 0, 3)   # (A format, B format) = (p >> 1, p & 1)
    outs = _draw(S.seed_for(10, 21), 10, 0, 1)    # bfloat16 or float32 output
    return list(zip(ms, ns, ks, pairs, outs))


@pytest.mark.parametrize("case", _gemm_cases())
def test_gemm_random_shapes(case):
    """Seeded random GEMM shapes, format pairs and output dtypes (small-problem and 256 x 256
    kernels of both MFMA families, ragged M, N and K): full sampled rows and columns against the
    float64 oracle."""
    M, N, K, p, od = case
    fa, fb = p >> 1, p & 1
    print(f"gemm random M={M} N={N} K={K} fa={fa} fb={fb} out={od}", flush=True)
    A8 = oracle.cast_amax(S.normal_bf16(S.seed_for(10, 22), (M, K), 2.0), 1.0, fa)[0]
    B8 = oracle.cast_amax(S.normal_bf16(S.seed_for(10, 23), (N, K), 2.0), 1.0, fb)[0]
    bias = S.normal_bf16(S.seed_for(10, 24), (N,), 0.1)
    D = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16 if od == 0 else torch.float32)
    F.fp8_gemm_bias(torch.from_numpy(A8).to(DEV), fa, scalar(0.5), torch.from_numpy(B8).to(DEV), fb, scalar(0.25),
                    bf16_dev(bias), D)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], (S.uniform(S.seed_for(10, 25), 0, 30) * M).astype(np.int64)]))
    cols = np.unique(np.concatenate([[0, N - 1], (S.uniform(S.seed_for(10, 26), 0, 30) * N).astype(np.int64)]))
    R_rows, R_cols = oracle.gemm_bias_sampled(A8, fa, 0.5, B8, fb, 0.25, bias, rows, cols)
    gemm_close(to_f64(D[torch.from_numpy(rows).to(DEV)]), R_rows, bf16_out=(od == 0))
    gemm_close(to_f64(D[:, torch.from_numpy(cols).to(DEV)]), R_cols, bf16_out=(od == 0))


@pytest.mark.parametrize("shape", [(1, 1, 65536), (3, 5, 65520), (17, 33, 16448), (40, 24, 32768)])
def test_gemm_long_k_few_outputs(shape):
    """Long K with a handful of outputs (hundreds of K steps in one wave; K % 256 == 0, K % 64 ==
    0 and K % 16 == 0 only): every output against the float64 oracle."""
    M, N, K = shape
    print(f"gemm long K M={M} N={N} K={K}", flush=True)
    A8 = oracle.cast_amax(S.normal_bf16(S.seed_for(10, 27), (M, K), 1.0), 1.0, F.E4M3)[0]
    B8 = oracle.cast_amax(S.normal_bf16(S.seed_for(10, 28), (N, K), 1.0), 1.0, F.E5M2)[0]
    bias = S.normal_bf16(S.seed_for(10, 29), (N,), 0.1)
    for od in (0, 1):
        D = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16 if od == 0 else torch.float32)
        F.fp8_gemm_bias(torch.from_numpy(A8).to(DEV), F.E4M3, scalar(0.5), torch.from_numpy(B8).to(DEV), F.E5M2,
                        scalar(0.25), bf16_dev(bias), D)
        torch.cuda.synchronize()
        gemm_close(to_f64(D), oracle.gemm_bias(A8, F.E4M3, 0.5, B8, F.E5M2, 0.25, bias), bf16_out=(od == 0))
