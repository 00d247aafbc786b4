"""GPU parity of the FP8-output GEMM (output codes with their own scale, amax of the output,
its private inverse scale) against the oracle: bit-exact where the float32 accumulation is
exact, inside the GEMM tolerance window otherwise, and consistent with the float32-output
GEMM of the same operands."""
import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, GEMM_TOL, bf16_dev, f32_bits, scalar, to_f64, u8_host

pytestmark = pytest.mark.gpu

TORCH_FP8 = {F.E4M3: torch.float8_e4m3fn, F.E5M2: torch.float8_e5m2}


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _codes(seed, shape, fmt, std=1.0, scale=1.0):
    return oracle.cast_amax(S.normal_bf16(seed, shape, std), scale, fmt)[0]


def _run(A8, fa, sa, B8, fb, sb, bias_h, d_fmt, ds, amax_in=0.0, D=None):
    M, N = A8.shape[0], B8.shape[0]
    if D is None:
        D = torch.full((M, N), 0xEE, dtype=torch.uint8, device=DEV)
    amax = scalar(amax_in)
    sinv = scalar(-1.0)
    F.fp8_gemm_bias_fp8(_u8(A8), fa, scalar(sa), _u8(B8), fb, scalar(sb), None if bias_h is None else bf16_dev(bias_h),
                        D, d_fmt, scalar(ds), sinv, amax)
    torch.cuda.synchronize()
    return u8_host(D), amax.item(), sinv.item()


def _window_ok(q, R, ds, fmt, tol_abs):
    """The GPU code must be the encoding of some value within the GEMM tolerance of the float64
    result: encode is monotone, so its decoded value lies between the decoded encodings of the
    window's ends."""
    lo = ((R - tol_abs) * np.float64(ds)).astype(np.float32)
    hi = ((R + tol_abs) * np.float64(ds)).astype(np.float32)
    v = oracle.decode(q, fmt)
    vlo = oracle.decode(oracle.encode(lo, fmt), fmt)
    vhi = oracle.decode(oracle.encode(hi, fmt), fmt)
    bad = ~((vlo <= v) & (v <= vhi))
    if bad.any():
        i = np.unravel_index(np.argmax(bad), bad.shape)
        raise AssertionError(f"code {q[i]:#x} ({v[i]}) outside [{vlo[i]}, {vhi[i]}] at {i}, R={R[i]}")


EXACT_TAB = np.array([0x00, 0x30, 0x38, 0x40], np.uint8)   # E4M3 0, 0.5, 1, 2


def _exact_operands(seed, M, N, K):
    rng = np.random.default_rng(seed)
    A8 = EXACT_TAB[rng.integers(0, 4, (M, K))] | np.where(rng.random((M, K)) < 0.5, 0x80, 0).astype(np.uint8)
    B8 = EXACT_TAB[rng.integers(0, 4, (N, K))] | np.where(rng.random((N, K)) < 0.5, 0x80, 0).astype(np.uint8)
    # bias: multiples of 1/4 below 64 in magnitude (exact in bfloat16 and in every partial sum)
    bias_f = (rng.integers(-256, 256, N) / 4.0).astype(np.float32)
    bias = (bias_f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return A8, B8, bias


@pytest.mark.parametrize("d_fmt", [F.E4M3, F.E5M2])
# the 32 x 32 x 64 small kernel (K % 64 == 0), the general one, the 16 x 16 x 128 small kernel
@pytest.mark.parametrize("K", [192, 80, 256])
def test_gemm_fp8_out_exact_arithmetic(d_fmt, K):
    """Codes in {0, +-0.5, +-1, +-2}, power-of-two inverse scales and quarter-integer bias: every
    float32 partial sum is exact, so codes, amax and inverse scale must match the oracle bit
    for bit, for scales that saturate, round and underflow."""
    M, N = 300, 520
    A8, B8, bias = _exact_operands(11 + K, M, N, K)
    for ds in (1.0, 0.3, 7.0, 1e-3, 2.0 ** -20):
        print(f"fp8-out exact d_fmt={d_fmt} K={K} ds={ds}", flush=True)
        q, amax, sinv = _run(A8, F.E4M3, 0.5, B8, F.E4M3, 2.0, bias, d_fmt, ds)
        rq, ramax, rsinv, _ = oracle.gemm_bias_fp8(A8, F.E4M3, 0.5, B8, F.E4M3, 2.0, bias, d_fmt, ds)
        assert np.array_equal(q, rq), ds
        assert f32_bits(amax)[0] == f32_bits(ramax)[0] and f32_bits(sinv)[0] == f32_bits(rsinv)[0]


SHAPES = [(1, 1, 16), (37, 45, 48), (256, 256, 128), (300, 520, 272), (513, 257, 1040), (128, 256, 256)]


@pytest.mark.parametrize("fa,fb,d_fmt", [(0, 0, 0), (1, 0, 1), (1, 0, 0), (0, 1, 1)])
@pytest.mark.parametrize("shape", SHAPES)
def test_gemm_fp8_out_parity(fa, fb, d_fmt, shape):
    M, N, K = shape
    print(f"fp8-out fa={fa} fb={fb} d_fmt={d_fmt} M={M} N={N} K={K}", flush=True)
    A8 = _codes(S.seed_for(40, fa), (M, K), fa, 2.0)
    B8 = _codes(S.seed_for(41, fb), (N, K), fb, 2.0)
    bias = S.normal_bf16(S.seed_for(42, 0), (N,), 0.5)
    R = oracle.gemm_bias(A8, fa, 0.5, B8, fb, 0.25, bias)
    big = float(np.abs(R).max())
    ds = oracle.fp8_max(d_fmt) / big * 0.5 if big else 1.0
    q, amax, sinv = _run(A8, fa, 0.5, B8, fb, 0.25, bias, d_fmt, ds)
    _window_ok(q, R, ds, d_fmt, GEMM_TOL * big)
    assert abs(amax - big) <= GEMM_TOL * big
    assert f32_bits(sinv)[0] == f32_bits(oracle.scale_inv(ds))[0]


@pytest.mark.parametrize("shape", [(300, 520, 272), (513, 257, 1040), (600, 900, 208), (77, 1000, 64),
                                   (1100, 2300, 512), (1300, 2100, 320)])
@pytest.mark.parametrize("d_fmt", [F.E4M3, F.E5M2])
def test_gemm_fp8_out_equals_encoded_fp32_output(shape, d_fmt):
    """The FP8 output is the float32 output of the same GEMM encoded with the output scale
    (torch's own float8 conversion of the clamped value serves as the encoder here), and the
    amax is exactly max |float32 output|, ragged tiles included."""
    M, N, K = shape
    A8 = _codes(S.seed_for(43, 0), (M, K), F.E5M2, 1.0)
    B8 = _codes(S.seed_for(43, 1), (N, K), F.E4M3, 1.0)
    bias = S.normal_bf16(S.seed_for(43, 2), (N,), 2.0)
    D32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    F.fp8_gemm_bias(_u8(A8), F.E5M2, scalar(0.5), _u8(B8), F.E4M3, scalar(1.5), bf16_dev(bias), D32)
    torch.cuda.synchronize()
    d = D32.cpu()
    for ds in (1.0, 37.0, 1e-2):
        q, amax, _ = _run(A8, F.E5M2, 0.5, B8, F.E4M3, 1.5, bias, d_fmt, ds)
        mx = oracle.fp8_max(d_fmt)
        y = torch.clamp(d * torch.tensor(ds, dtype=torch.float32), -mx, mx)
        ref = y.to(TORCH_FP8[d_fmt]).view(torch.uint8).numpy()
        assert np.array_equal(q, ref), ds
        assert amax == float(d.abs().max())


def test_gemm_fp8_out_k_zero_empty_and_amax_fold():
    N = 40
    bias = S.normal_bf16(S.seed_for(44, 0), (N,), 3.0)
    z = lambda r, c: np.zeros((r, c), np.uint8)
    # K == 0: D is the encoded bias
    q, amax, sinv = _run(z(7, 0), 0, 1.0, z(N, 0), 0, 1.0, bias, F.E4M3, 5.0)
    rq, ramax, rsinv, _ = oracle.gemm_bias_fp8(z(7, 0), 0, 1.0, z(N, 0), 0, 1.0, bias, F.E4M3, 5.0)
    assert np.array_equal(q, rq) and amax == ramax and sinv == rsinv
    # a larger amax already in the slot stays; a smaller one is raised
    q2, amax2, _ = _run(z(7, 0), 0, 1.0, z(N, 0), 0, 1.0, bias, F.E4M3, 5.0, amax_in=1e6)
    assert amax2 == 1e6 and np.array_equal(q2, rq)
    # M == 0: only the inverse scale is written
    D = torch.empty((0, N), dtype=torch.uint8, device=DEV)
    _, amax3, sinv3 = _run(z(0, 16), 0, 1.0, z(N, 16), 0, 1.0, bias, F.E5M2, 4.0, D=D)
    assert amax3 == 0.0 and sinv3 == 0.25


def test_gemm_fp8_out_strided_and_unaligned_output():
    """Output rows with a stride that is not a multiple of 16, at an odd address: the element
    path writes exactly the same codes and nothing outside the [M, N] view."""
    M, N, K = 300, 200, 128
    A8 = _codes(S.seed_for(45, 0), (M, K), 0, 1.0)
    B8 = _codes(S.seed_for(45, 1), (N, K), 0, 1.0)
    bias = S.normal_bf16(S.seed_for(45, 2), (N,), 1.0)
    q, amax, _ = _run(A8, 0, 1.0, B8, 0, 0.125, bias, F.E4M3, 3.0)
    ld = 211
    buf = torch.full((M * ld + 1,), 0xEE, dtype=torch.uint8, device=DEV)
    D = buf[1:].view(M, ld)[:, :N]
    q2, amax2, _ = _run(A8, 0, 1.0, B8, 0, 0.125, bias, F.E4M3, 3.0, D=D)
    assert np.array_equal(q, q2) and amax == amax2
    full = u8_host(buf[1:].view(M, ld))
    assert np.all(full[:, N:] == 0xEE) and u8_host(buf[:1])[0] == 0xEE


def test_gemm_fp8_out_full_size_dgrad():
    """dgrad of the QKV projection at one TP=2 rank's share (M=8192, K=18432 -> N=12288) written
    straight into an E5M2 tensor: 64 seeded full rows and 64 full columns inside the tolerance
    window of the float64 oracle, and the whole output equal to the encoded float32 output of
    the same GEMM with amax = max |float32 output|."""
    M, N, K = 8192, 12288, 18432
    print(f"fp8-out full-size dgrad M={M} N={N} K={K}", flush=True)
    A8 = _codes(S.seed_for(4, 10), (M, K), F.E5M2, 1.0)
    B8 = _codes(S.seed_for(4, 11), (N, K), F.E4M3, 0.02, 64.0)
    sb = 1.0 / 64.0
    ds = 512.0
    q, amax, sinv = _run(A8, F.E5M2, 1.0, B8, F.E4M3, sb, None, F.E5M2, ds)
    rows = (S.uniform(S.seed_for(4, 15), 0, 64) * M).astype(np.int64)
    cols = (S.uniform(S.seed_for(4, 16), 0, 64) * N).astype(np.int64)
    Rr, Rc = oracle.gemm_bias_sampled(A8, F.E5M2, 1.0, B8, F.E4M3, sb, None, rows, cols)
    big = max(float(np.abs(Rr).max()), float(np.abs(Rc).max()))
    _window_ok(q[rows], Rr, ds, F.E5M2, GEMM_TOL * big)
    _window_ok(q[:, cols], Rc, ds, F.E5M2, GEMM_TOL * big)
    D32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    F.fp8_gemm_bias(_u8(A8), F.E5M2, scalar(1.0), _u8(B8), F.E4M3, scalar(sb), None, D32)
    torch.cuda.synchronize()
    assert amax == float(D32.abs().max())
    d = D32.cpu()
    ref = torch.clamp(d * torch.tensor(ds, dtype=torch.float32), -57344.0, 57344.0).to(torch.float8_e5m2)
    assert np.array_equal(q, ref.view(torch.uint8).numpy())
    assert sinv == 1.0 / 512.0
