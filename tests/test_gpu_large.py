"""Tensors of more than 2^31 elements (and one of more than 2^32): every offset past the 32-bit
range is 64-bit in the kernels, and these tests check it on outputs placed there.

The large inputs are a small seeded block tiled over the tensor (block sides of prime length, so
that an offset wrapped modulo 2^31 or 2^32 lands on a different block position and shows up as
a different value), with marker values planted at the far end and near the 2^31 / 2^32
boundaries.  Expected values come from the oracle applied to the block, to reconstructed rows
and columns, and to the markers; the tiling identities (a column of a row-tiled tensor is the
block column repeated) hold at any size."""
import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, f32_bits, gemm_close, scalar, to_f64, u8_host

pytestmark = pytest.mark.gpu

U8 = dict(dtype=torch.uint8, device=DEV)
TWO31, TWO32 = 1 << 31, 1 << 32
# 2-D shapes past 2^31 elements: 192 row tiles + 16 rows, 176 column tiles + 8 columns
R2, C2 = 49168, 45064
BR, BC = 251, 263                  # block sides (prime)


def _dev_bits(a: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).view(dtype)


def _tile2(block: torch.Tensor, R: int, C: int) -> torch.Tensor:
    br, bc = block.shape
    return block.repeat(-(-R // br), -(-C // bc))[:R, :C].contiguous()


def _row(block: np.ndarray, i: int, C: int) -> np.ndarray:
    return block[i % block.shape[0], np.arange(C) % block.shape[1]]


def _col(block: np.ndarray, j: int, R: int) -> np.ndarray:
    return block[np.arange(R) % block.shape[0], j % block.shape[1]]


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_cast_amax_past_2_32_elements():
    """n = 2^32 + 4109: the grid-stride part of the launch, the 13-element remainder, a marker
    holding the amax at n - 1 and distinct markers just past 2^31 and 2^32."""
    n = TWO32 + 4109
    B = 65537
    blk = S.normal_bf16(S.seed_for(30, 0), (B,), 1.0)
    markers = {n - 1: 0x4A12, TWO31 + 5: 0xC3A1, TWO32 + 3: 0x4321, TWO31 - 1: 0x3F11}  # 2.39e6, -322, 161, 0.57
    print(f"cast_amax n={n}", flush=True)
    x = _dev_bits(blk.view(np.int16), torch.bfloat16).repeat(-(-n // B))[:n]
    for i, v in markers.items():
        x.view(torch.int16)[i] = int(np.uint16(v).view(np.int16))
    out = torch.full((n,), 0xAB, **U8)
    sinv, slot = scalar(-1.0), scalar(0.0)
    F.fp8_cast_amax(x, scalar(3.0), F.E4M3, out, sinv, slot)
    torch.cuda.synchronize()

    def host_x(lo, hi):
        v = blk[np.arange(lo, hi) % B].copy()
        for i, m in markers.items():
            if lo <= i < hi:
                v[i - lo] = m
        return v

    for lo, hi in [(0, 4096), (TWO31 - 2048, TWO31 + 2048), (TWO32 - 2048, TWO32 + 2048), (n - 8192, n)]:
        q, _, _ = oracle.cast_amax(host_x(lo, hi), 3.0, F.E4M3)
        assert np.array_equal(u8_host(out[lo:hi]), q), (lo, hi)
    every = np.concatenate([blk, np.array(list(markers.values()), dtype=np.uint16)])
    _, am, si = oracle.cast_amax(every, 3.0, F.E4M3)
    assert f32_bits(slot.item()) == f32_bits(am) and f32_bits(sinv.item()) == f32_bits(si)
    del x, out
    _free()


def _markers_2d(R, C):
    # (row, col) -> bfloat16 bits; the largest magnitude sits in the last element
    return {(R - 1, C - 1): 0x49F4, (R - 3, 7): 0xC2F0, (5, C - 2): 0x42C8, (R // 2, C // 2): 0xC1A0}


def _plant(x: torch.Tensor, markers):
    xi = x.view(torch.int16)
    for (i, j), v in markers.items():
        xi[i, j] = int(np.uint16(v).view(np.int16))


def _host_row(blk, markers, i, C):
    v = _row(blk, i, C).copy()
    for (a, b), m in markers.items():
        if a == i:
            v[b] = m
    return v


def _host_col(blk, markers, j, R):
    v = _col(blk, j, R).copy()
    for (a, b), m in markers.items():
        if b == j:
            v[a] = m
    return v


def _sample_rows_cols(R, C, seed):
    rows = sorted({0, 5, R // 2, R - 3, R - 1, *(S.uniform(seed, 0, 6) * R).astype(np.int64).tolist()})
    cols = sorted({0, 7, C // 2, C - 2, C - 1, *(S.uniform(seed, 8, 6) * C).astype(np.int64).tolist()})
    return rows, cols


@pytest.mark.parametrize("fmt", [F.E4M3, F.E5M2])
def test_cast_transpose_past_2_31_elements(fmt):
    """[49168, 45064] (2.2e9 elements, ragged row and column tiles): sampled rows of the codes
    and sampled rows of the transpose (columns of x) against the oracle, markers included."""
    R, C = R2, C2
    scale = 3.0 if fmt == F.E4M3 else 2048.0
    blk = S.normal_bf16(S.seed_for(30, 1), (BR, BC), 1.0 if fmt == F.E4M3 else 0.01)
    mk = _markers_2d(R, C)
    print(f"cast_transpose [{R},{C}] fmt {fmt}", flush=True)
    x = _tile2(_dev_bits(blk.view(np.int16), torch.bfloat16), R, C)
    _plant(x, mk)
    out = torch.full((R, C), 0xAB, **U8)
    out_t = torch.full((C, R), 0xCD, **U8)
    sinv, slot = scalar(-1.0), scalar(0.0)
    F.fp8_cast_transpose(x, scalar(scale), fmt, out, out_t, sinv, slot)
    torch.cuda.synchronize()
    del x
    rows, cols = _sample_rows_cols(R, C, S.seed_for(30, 2))
    for i in rows:
        q, _, _ = oracle.cast_amax(_host_row(blk, mk, i, C), scale, fmt)
        assert np.array_equal(u8_host(out[i]), q), ("row", i)
    for j in cols:
        q, _, _ = oracle.cast_amax(_host_col(blk, mk, j, R), scale, fmt)
        assert np.array_equal(u8_host(out_t[j]), q), ("transposed row", j)
    every = np.concatenate([blk.reshape(-1), np.array(list(mk.values()), dtype=np.uint16)])
    _, am, si = oracle.cast_amax(every, scale, fmt)
    assert f32_bits(slot.item()) == f32_bits(am) and f32_bits(sinv.item()) == f32_bits(si)
    del out, out_t
    _free()


def test_dbias_cast_transpose_past_2_31_elements():
    """dy [49168, 45064] E5M2 (the tile kernel + reduction form): sampled code rows and
    transposed rows bit for bit; every column sum within its bound, the expected sums from the
    oracle's column sums of the block (each column of dy is its block column repeated, plus
    the markers)."""
    R, C = R2, C2
    blk = S.normal_bf16(S.seed_for(30, 3), (BR, BC), 0.01)
    mk = {(R - 1, C - 1): 0x3F80, (R - 3, 7): 0xBF00, (5, C - 2): 0x3E80}
    print(f"dbias_cast_transpose [{R},{C}]", flush=True)
    dy = _tile2(_dev_bits(blk.view(np.int16), torch.bfloat16), R, C)
    _plant(dy, mk)
    out = torch.full((R, C), 0xAB, **U8)
    out_t = torch.full((C, R), 0xCD, **U8)
    db = torch.full((C,), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), **U8)
    sinv, slot = scalar(-1.0), scalar(0.0)
    F.fp8_dbias_cast_transpose(dy, scalar(2048.0), F.E5M2, out, out_t, db, ws, sinv, slot)
    torch.cuda.synchronize()
    del dy
    rows, cols = _sample_rows_cols(R, C, S.seed_for(30, 4))
    for i in rows:
        q, _, _ = oracle.cast_amax(_host_row(blk, mk, i, C), 2048.0, F.E5M2)
        assert np.array_equal(u8_host(out[i]), q), ("row", i)
    for j in cols:
        q, _, _ = oracle.cast_amax(_host_col(blk, mk, j, R), 2048.0, F.E5M2)
        assert np.array_equal(u8_host(out_t[j]), q), ("transposed row", j)
    # column sums: full repeats of the block, the remaining rows, then the markers' changes
    full, rem = R // BR, R % BR
    bsum = oracle.dbias(blk)
    rsum = oracle.dbias(blk[:rem])
    babs = oracle.dbias(blk & np.uint16(0x7FFF))
    rabs = oracle.dbias(blk[:rem] & np.uint16(0x7FFF))
    jb = np.arange(C) % BC
    ref = full * bsum[jb] + rsum[jb]
    mag = full * babs[jb] + rabs[jb]
    for (i, j), v in mk.items():
        old = blk[i % BR, j % BC]
        ref[j] += S.bf16_bits_to_f64(np.uint16(v)) - S.bf16_bits_to_f64(old)
        mag[j] += abs(S.bf16_bits_to_f64(np.uint16(v))) - abs(S.bf16_bits_to_f64(old))
    got = db.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 1e-5 * mag + 1e-30)
    assert not torch.any(ws[:1024])
    del out, out_t, ws
    _free()


def test_fp8_transpose_past_2_31_elements():
    """FP8 -> FP8 transpose of a [49168, 45064] code tensor: sampled transposed rows equal the
    reconstructed columns, byte for byte."""
    R, C = R2, C2
    blk = S.random_bytes(S.seed_for(30, 5), (BR, BC))
    mk = {(R - 1, C - 1): 0x11, (R - 3, 7): 0x22, (5, C - 2): 0x33}
    print(f"fp8_transpose [{R},{C}]", flush=True)
    x8 = _tile2(torch.from_numpy(blk).to(DEV), R, C)
    for (i, j), v in mk.items():
        x8[i, j] = v
    out_t = torch.full((C, R), 0xCD, **U8)
    F.fp8_transpose(x8, out_t)
    torch.cuda.synchronize()
    del x8
    _, cols = _sample_rows_cols(R, C, S.seed_for(30, 6))
    for j in cols:
        col = _col(blk, j, R).copy()
        for (a, b), v in mk.items():
            if b == j:
                col[a] = v
        assert np.array_equal(u8_host(out_t[j]), col), j
    del out_t
    _free()


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_output_past_2_31_elements(out_dtype):
    """[47104, 256] x [47104, 256]^T -> 2.2e9 outputs (the last rows start past 2^31 elements):
    sampled full rows and full columns against the float64 oracle."""
    M = N = 47104
    K = 256
    print(f"gemm M=N={M} K={K} out={out_dtype}", flush=True)
    ah = S.normal_bf16(S.seed_for(30, 7), (M, K), 1.0)
    bh = S.normal_bf16(S.seed_for(30, 8), (N, K), 1.0)
    biash = S.normal_bf16(S.seed_for(30, 9), (N,), 0.1)
    A, _, _ = oracle.cast_amax(ah, 16.0, F.E4M3)
    B, _, _ = oracle.cast_amax(bh, 16.0, F.E4M3)
    sa = sb = 1.0 / 16.0
    D = torch.empty((M, N), device=DEV, dtype=out_dtype)
    F.fp8_gemm_bias(torch.from_numpy(A).to(DEV), F.E4M3, scalar(sa), torch.from_numpy(B).to(DEV), F.E4M3, scalar(sb),
                    _dev_bits(biash.view(np.int16), torch.bfloat16), D)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, M // 2, M - 2, M - 1, *(S.uniform(S.seed_for(30, 10), 0, 11) * M).astype(np.int64)}))
    cols = np.array(sorted({0, 1, N // 2, N - 2, N - 1, *(S.uniform(S.seed_for(30, 11), 0, 11) * N).astype(np.int64)}))
    R_rows, R_cols = oracle.gemm_bias_sampled(A, F.E4M3, sa, B, F.E4M3, sb, biash, rows, cols)
    rt, ct = torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)
    bf = out_dtype == torch.bfloat16
    gemm_close(to_f64(D.index_select(0, rt)), R_rows, bf16_out=bf)
    gemm_close(to_f64(D.index_select(1, ct)), R_cols, bf16_out=bf)
    del D
    _free()
