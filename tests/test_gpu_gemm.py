"""GPU parity of the FP8 GEMM with dequantisation and bias against the float64 oracle, the
N-chunked variant (bit-identical to the unchunked call, also as a replayed graph) and
determinism."""
import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, bf16_dev, gemm_close, scalar, to_f64

pytestmark = pytest.mark.gpu


def _codes(seed, shape, fmt, std=1.0, scale=1.0):
    """Seeded FP8 operands: cast of seeded bfloat16 by the oracle (host)."""
    return oracle.cast_amax(S.normal_bf16(seed, shape, std), scale, fmt)[0]


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _run(A8, fa, sa, B8, fb, sb, bias_h, out_dtype):
    M, N = A8.shape[0], B8.shape[0]
    D = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16 if out_dtype == 0 else torch.float32)
    F.fp8_gemm_bias(_u8(A8), fa, scalar(sa), _u8(B8), fb, scalar(sb), None if bias_h is None else bf16_dev(bias_h), D)
    torch.cuda.synchronize()
    return D


SHAPES = [(1, 1, 16), (37, 45, 48), (256, 256, 128), (300, 520, 272), (513, 257, 1040), (128, 256, 256),
          (1, 1, 256), (37, 45, 512), (300, 520, 1024)]


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("shape", SHAPES)
def test_gemm_parity_small(fa, fb, shape):
    M, N, K = shape
    print(f"gemm fa={fa} fb={fb} M={M} N={N} K={K}", flush=True)
    A8 = _codes(S.seed_for(20, fa), (M, K), fa, 2.0)
    B8 = _codes(S.seed_for(21, fb), (N, K), fb, 2.0)
    bias = S.normal_bf16(S.seed_for(22, 0), (N,), 0.1)
    R = oracle.gemm_bias(A8, fa, 0.5, B8, fb, 0.25, bias)
    for out_dtype in (0, 1):
        D = _run(A8, fa, 0.5, B8, fb, 0.25, bias, out_dtype)
        gemm_close(to_f64(D), R, bf16_out=(out_dtype == 0))
    D = _run(A8, fa, 0.5, B8, fb, 0.25, None, 1)
    gemm_close(to_f64(D), oracle.gemm_bias(A8, fa, 0.5, B8, fb, 0.25, None), bf16_out=False)


def test_gemm_exact_integer_products():
    """Small-integer codes: every partial sum is an integer below 2^24, so the float32
    accumulation is exact and the result must equal the oracle exactly."""
    M, N, K = 300, 280, 512
    rng = np.random.default_rng(5)
    tab = np.array([0x00, 0x38, 0x40, 0x44, 0x48], np.uint8)   # 0 1 2 3 4 in E4M3
    A8 = tab[rng.integers(0, 5, (M, K))] | np.where(rng.random((M, K)) < 0.5, 0x80, 0).astype(np.uint8)
    B8 = tab[rng.integers(0, 5, (N, K))]
    D = _run(A8, 0, 1.0, B8, 0, 1.0, None, 1)
    assert np.array_equal(to_f64(D), oracle.gemm_bias(A8, 0, 1.0, B8, 0, 1.0))


def test_gemm_k_zero_gives_bias_and_empty_mn():
    bias = S.normal_bf16(3, (40,), 1.0)
    D = torch.empty((7, 40), device=DEV, dtype=torch.float32)
    F.fp8_gemm_bias(torch.empty((7, 0), dtype=torch.uint8, device=DEV), 0, scalar(1.0),
                    torch.empty((40, 0), dtype=torch.uint8, device=DEV), 0, scalar(1.0), bf16_dev(bias), D)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(D), np.tile(S.bf16_bits_to_f64(bias), (7, 1)))
    D0 = torch.full((0, 5), 1.0, device=DEV)
    F.fp8_gemm_bias(torch.empty((0, 16), dtype=torch.uint8, device=DEV), 0, scalar(1.0),
                    torch.empty((5, 16), dtype=torch.uint8, device=DEV), 0, scalar(1.0), None, D0)


def test_gemm_strided_operands():
    """Leading dimensions larger than K (views into wider buffers)."""
    M, N, K = 200, 150, 96
    Aw = _codes(30, (M, 160), 0)
    Bw = _codes(31, (N, 128), 1)
    A8, B8 = Aw[:, :K], Bw[:, :K]
    Dw = torch.zeros((M, 168), device=DEV, dtype=torch.float32)
    D = Dw[:, :N]
    F.fp8_gemm_bias(_u8(Aw)[:, :K], 0, scalar(1.0), _u8(Bw)[:, :K], 1, scalar(1.0), None, D)
    torch.cuda.synchronize()
    gemm_close(to_f64(D), oracle.gemm_bias(A8, 0, 1.0, B8, 1, 1.0), bf16_out=False)
    assert torch.all(Dw[:, N:] == 0)


def test_gemm_deterministic():
    A8 = _codes(40, (1024, 2048), 0)
    B8 = _codes(41, (768, 2048), 0)
    D1 = _run(A8, 0, 1.0, B8, 0, 1.0, None, 1)
    D2 = _run(A8, 0, 1.0, B8, 0, 1.0, None, 1)
    assert torch.equal(D1.view(torch.int32), D2.view(torch.int32))


def _full_config(M, N, K, fa, fb, seed_base, stdA, stdB, scaleA, scaleB):
    A8 = _codes(seed_base, (M, K), fa, stdA, scaleA)
    B8 = _codes(seed_base + 1, (N, K), fb, stdB, scaleB)
    return A8, B8


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_gemm_full_size_qkv_sampled(which):
    """The GPT-175B QKV projection at one TP=2 rank's share (M=8192, K=12288, N=18432) in the
    launch configuration the benchmark times, checked on 64 seeded full rows and 64 seeded full
    columns of the output against the float64 oracle."""
    M, K, N = 8192, 12288, 18432
    if which == "fwd":
        shapes = (M, N, K, 0, 0)          # x8 [M,K] . W8 [N,K]
    elif which == "dgrad":
        shapes = (M, K, N, 1, 0)          # dy8 [M,N] . W8t [K,N]
    else:
        shapes = (N, K, M, 1, 0)          # dy8t [N,M] . x8t [K,M]
    m, n, k, fa, fb = shapes
    print(f"full-size {which}: M={m} N={n} K={k}", flush=True)
    A8 = _codes(S.seed_for(4, 10), (m, k), fa, 1.0, 1.0 if fa == 0 else 1.0)
    B8 = _codes(S.seed_for(4, 11), (n, k), fb, 0.02, 64.0)
    bias = S.normal_bf16(S.seed_for(4, 12), (n,), 0.1) if which == "fwd" else None
    D = torch.empty((m, n), device=DEV, dtype=torch.bfloat16)
    F.fp8_gemm_bias(_u8(A8), fa, scalar(1.0), _u8(B8), fb, scalar(1.0 / 64.0), None if bias is None else bf16_dev(bias), D)
    torch.cuda.synchronize()
    rows = (S.uniform(S.seed_for(4, 13), 0, 64) * m).astype(np.int64)
    cols = (S.uniform(S.seed_for(4, 14), 0, 64) * n).astype(np.int64)
    Rr, Rc = oracle.gemm_bias_sampled(A8, fa, 1.0, B8, fb, 1.0 / 64.0, bias, rows, cols)
    Dh = to_f64(D)
    big = max(float(np.abs(Rr).max()), float(np.abs(Rc).max()))
    gemm_close(Dh[rows], Rr, bf16_out=True, scale_ref=big)
    gemm_close(Dh[:, cols], Rc, bf16_out=True, scale_ref=big)


@pytest.mark.parametrize("n_chunks", [4, 8])
def test_chunked_equals_unchunked_and_graph(n_chunks):
    """N-chunked GEMM+bias (M=8192, K=N=12288), one stream per chunk with its own bias offset,
    is bit-identical to the unchunked call, eagerly and as a captured, replayed graph."""
    M, K, N = 8192, 12288, 12288
    print(f"chunked n_chunks={n_chunks}", flush=True)
    A8 = _u8(_codes(S.seed_for(5, 0), (M, K), 0, 1.0))
    B8 = _u8(_codes(S.seed_for(5, 1), (N, K), 0, 0.02, 64.0))
    bias = bf16_dev(S.normal_bf16(S.seed_for(5, 2), (N,), 0.1))
    sa, sb = scalar(1.0), scalar(1.0 / 64)
    ref = torch.empty((M, N), device=DEV, dtype=torch.bfloat16)
    F.fp8_gemm_bias(A8, 0, sa, B8, 0, sb, bias, ref)
    streams = [torch.cuda.Stream() for _ in range(n_chunks)]
    D = torch.zeros((M, N), device=DEV, dtype=torch.bfloat16)
    F.fp8_gemm_bias_chunked(A8, 0, sa, B8, 0, sb, bias, D, n_chunks, streams)
    torch.cuda.synchronize()
    assert torch.equal(D.view(torch.int16), ref.view(torch.int16))
    # graph capture of the whole fork/join sequence, replayed several times
    G = torch.zeros((M, N), device=DEV, dtype=torch.bfloat16)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        F.fp8_gemm_bias_chunked(A8, 0, sa, B8, 0, sb, bias, G, n_chunks, streams, stream=cap)
    for _ in range(3):
        G.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(G.view(torch.int16), ref.view(torch.int16))
    # sampled oracle check of the chunked output: 64 full rows and 64 full columns, the columns
    # drawn across every chunk
    rows = (S.uniform(S.seed_for(5, 3), 0, 64) * M).astype(np.int64)
    cols = (S.uniform(S.seed_for(5, 4), 0, 64) * N).astype(np.int64)
    Rr, Rc = oracle.gemm_bias_sampled(A8.cpu().numpy(), 0, 1.0, B8.cpu().numpy(), 0, 1.0 / 64,
                                      S.normal_bf16(S.seed_for(5, 2), (N,), 0.1), rows, cols)
    Gh = to_f64(G)
    big = max(float(np.abs(Rr).max()), float(np.abs(Rc).max()))
    gemm_close(Gh[rows], Rr, bf16_out=True, scale_ref=big)
    gemm_close(Gh[:, cols], Rc, bf16_out=True, scale_ref=big)


def test_chunked_single_stream_and_ragged_chunks():
    M, K, N = 300, 256, 1000
    A8 = _codes(60, (M, K), 1)
    B8 = _codes(61, (N, K), 0)
    bias = S.normal_bf16(62, (N,), 0.5)
    ref = _run(A8, 1, 1.0, B8, 0, 1.0, bias, 1)
    for n_chunks in (1, 3, 7, 16):
        D = torch.zeros((M, N), device=DEV, dtype=torch.float32)
        F.fp8_gemm_bias_chunked(_u8(A8), 1, scalar(1.0), _u8(B8), 0, scalar(1.0), bf16_dev(bias), D, n_chunks, None)
        torch.cuda.synchronize()
        assert torch.equal(D.view(torch.int32), ref.view(torch.int32)), n_chunks


def test_chunked_from_several_host_threads():
    """Four host threads each enqueue chunked GEMMs on their own streams at the same time (the
    ctypes calls release the interpreter lock); the shared fork / join events must keep every
    call's chunks ordered after its own inputs and joined into its own stream."""
    import threading
    M, N, K = 512, 3072, 512
    A8 = _u8(_codes(S.seed_for(25, 0), (M, K), 0, 1.0))
    B8 = _u8(_codes(S.seed_for(25, 1), (N, K), 0, 1.0))
    bias = bf16_dev(S.normal_bf16(S.seed_for(25, 2), (N,), 0.2))
    sa, sb = scalar(0.5), scalar(0.5)
    ref = torch.empty((M, N), device=DEV, dtype=torch.float32)
    F.fp8_gemm_bias(A8, 0, sa, B8, 0, sb, bias, ref)
    torch.cuda.synchronize()
    nthreads, ncalls = 4, 6
    outs = [[torch.full((M, N), float("nan"), device=DEV) for _ in range(ncalls)] for _ in range(nthreads)]
    errors = []

    def worker(t):
        try:
            main = torch.cuda.Stream()
            streams = [torch.cuda.Stream() for _ in range(4)]
            for c in range(ncalls):
                # the output is cleared on the caller's stream just before the call, so a chunk that
                # is not ordered after that clear can be overwritten by it
                with torch.cuda.stream(main):
                    outs[t][c].zero_()
                F.fp8_gemm_bias_chunked(A8, 0, sa, B8, 0, sb, bias, outs[t][c], 4, streams, stream=main)
            main.synchronize()
        except Exception as e:   # reported below
            errors.append(e)

    th = [threading.Thread(target=worker, args=(t,)) for t in range(nthreads)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(nthreads):
        for c in range(ncalls):
            assert torch.equal(outs[t][c].view(torch.int32), ref.view(torch.int32)), (t, c)


@pytest.mark.parametrize("out_dtype", [0, 1])
@pytest.mark.parametrize("shape", [(256, 16384, 512), (300, 16384, 320), (2048, 2048, 1024)])
def test_small_problem_kernel_matches_large_tile_kernel(shape, out_dtype):
    """A GEMM of few 256 x 256 tiles runs a one-wave 64 x 64 tile kernel.  These outputs have 64
    or more large tiles (large-tile kernel at their K); each of their 8 N-chunks has 8 or 16 (small
    kernel).  The MFMA sequence per element is the same, so the chunked output must equal the
    unchunked one bit for bit, ragged rows included."""
    M, N, K = shape
    print(f"small vs large kernel M={M} N={N} K={K} out={out_dtype}", flush=True)
    A8 = _codes(S.seed_for(24, 0), (M, K), 1, 1.0)
    B8 = _codes(S.seed_for(24, 1), (N, K), 0, 0.5)
    bias = S.normal_bf16(S.seed_for(24, 2), (N,), 0.3)
    ref = _run(A8, 1, 0.5, B8, 0, 0.25, bias, out_dtype)
    D = torch.zeros_like(ref)
    F.fp8_gemm_bias_chunked(_u8(A8), 1, scalar(0.5), _u8(B8), 0, scalar(0.25), bf16_dev(bias), D, 8, None)
    torch.cuda.synchronize()
    w = torch.int16 if out_dtype == 0 else torch.int32
    assert torch.equal(D.view(w), ref.view(w))
    rows = (S.uniform(S.seed_for(24, 3), 0, 8) * M).astype(np.int64)
    Rr, _ = oracle.gemm_bias_sampled(A8, 1, 0.5, B8, 0, 0.25, bias, rows, [0])
    gemm_close(to_f64(D)[rows], Rr, bf16_out=(out_dtype == 0))


@pytest.mark.parametrize("shape", [(1, 1, 64), (100, 300, 128), (257, 513, 192), (256, 256, 448), (300, 700, 512),
                                   (513, 1000, 576)])
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0)])
def test_gemm_pipelined_path_shapes(shape, fa, fb):
    """K a multiple of 64 (1 to 9 slices of 64 bytes; these few-tile shapes run the register-fed
    small-problem kernels), ragged M and N, against the oracle.  With K % 256 != 0 the 32 x 32 x 64
    family runs, whose output must equal the general kernel's bit for bit (checked through a
    K-padded call that the general kernel handles); K % 256 == 0 runs the 16 x 16 x 128 family,
    whose MFMAs sum 128 products at once, so there only the oracle tolerance applies."""
    M, N, K = shape
    print(f"gemm pipe fa={fa} fb={fb} M={M} N={N} K={K}", flush=True)
    A8 = _codes(S.seed_for(23, fa), (M, K), fa, 2.0)
    B8 = _codes(S.seed_for(24, fb), (N, K), fb, 2.0)
    bias = S.normal_bf16(S.seed_for(25, 0), (N,), 0.1)
    R = oracle.gemm_bias(A8, fa, 0.5, B8, fb, 0.25, bias)
    D = _run(A8, fa, 0.5, B8, fb, 0.25, bias, 1)
    gemm_close(to_f64(D), R, bf16_out=False)
    Db = _run(A8, fa, 0.5, B8, fb, 0.25, bias, 0)
    gemm_close(to_f64(Db), R, bf16_out=True)
    # K + 16 zero columns: same products, general kernel (K % 64 != 0) -> identical bits
    pad = np.zeros((M, 16), np.uint8), np.zeros((N, 16), np.uint8)
    Dg = _run(np.hstack([A8, pad[0]]), fa, 0.5, np.hstack([B8, pad[1]]), fb, 0.25, bias, 1)
    gemm_close(to_f64(Dg), R, bf16_out=False)
    if K % 256 != 0:
        assert torch.equal(D.view(torch.int32), Dg.view(torch.int32))


@pytest.mark.parametrize("shape", [(1100, 4100, 256), (1500, 2600, 512), (2304, 1041, 1280), (4097, 700, 768),
                                   (100, 17000, 256)])
@pytest.mark.parametrize("fa,fb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_gemm_fam16_large_tile_kernel(shape, fa, fb):
    """K % 256 == 0 with more 256 x 256 tiles than the small-problem kernel takes at that K (over
    64 at K = 256, over 48 at K <= 1024, over 32 beyond) runs the 16 x 16 x 128 pipelined kernel:
    2 to 10 K steps of 128 bytes, ragged M and N (partial tiles at both edges), every format pair,
    float32 and bfloat16 output against the oracle on sampled rows (the ragged last rows
    included); the same GEMM cut into four N-chunks (few tiles each) runs the small-problem
    kernel of the same family and must give the same bits."""
    M, N, K = shape
    print(f"gemm fam16 fa={fa} fb={fb} M={M} N={N} K={K}", flush=True)
    A8 = _codes(S.seed_for(26, fa), (M, K), fa, 2.0)
    B8 = _codes(S.seed_for(27, fb), (N, K), fb, 2.0)
    bias = S.normal_bf16(S.seed_for(28, 0), (N,), 0.1)
    rows = np.unique(np.concatenate([(S.uniform(S.seed_for(28, 1), 0, 48) * M).astype(np.int64),
                                     np.arange(M - 3, M)]))
    Rr, _ = oracle.gemm_bias_sampled(A8, fa, 0.5, B8, fb, 0.25, bias, rows, [0])
    D = _run(A8, fa, 0.5, B8, fb, 0.25, bias, 1)
    gemm_close(to_f64(D)[rows], Rr, bf16_out=False)
    Db = _run(A8, fa, 0.5, B8, fb, 0.25, bias, 0)
    gemm_close(to_f64(Db)[rows], Rr, bf16_out=True)
    Dc = torch.zeros_like(D)
    F.fp8_gemm_bias_chunked(_u8(A8), fa, scalar(0.5), _u8(B8), fb, scalar(0.25), bf16_dev(bias), Dc, 4, None)
    torch.cuda.synchronize()
    assert torch.equal(Dc.view(torch.int32), D.view(torch.int32))


@pytest.mark.parametrize("sa,sb", [(1.2345678, 1.0), (1.01171875, 1.0), (0.70710677, 2.0 ** -120), (1.9, 2.0 ** 110)])
@pytest.mark.parametrize("shape", [(256, 64, 64), (1280, 2048, 64), (300, 200, 48), (256, 64, 256), (1280, 2048, 256)],
                         ids=["small-kernel", "pipelined-kernel", "general-kernel", "small16-kernel", "pipe16-kernel"])
def test_bf16_output_rounding_is_exact(shape, sa, sb):
    """One nonzero product per output (row code times column code, every E4M3 code on both
    sides), so the float32 value before the bfloat16 store is known exactly: the stored bits
    must be its round-to-nearest-even bfloat16, through ties, float32 and bfloat16 subnormals
    (sb = 2^-120), overflow to infinity (sb = 2^110), signed zeros and NaN codes."""
    M, N, K = shape
    print(f"gemm bf16 rounding M={M} N={N} K={K} sa={sa} sb={sb}", flush=True)
    A8 = np.zeros((M, K), np.uint8)
    B8 = np.zeros((N, K), np.uint8)
    A8[:, 0] = np.arange(M) % 256
    B8[:, 0] = (np.arange(N) * 37 + 11) % 256
    sa32, sb32 = np.float32(sa), np.float32(sb)
    prod = np.outer(oracle.decode(A8[:, 0], F.E4M3), oracle.decode(B8[:, 0], F.E4M3))
    with np.errstate(over="ignore", invalid="ignore"):
        t = (prod * np.float64(sa32)).astype(np.float32)                  # acc * a_scale_inv
        v = (t.astype(np.float64) * np.float64(sb32) + 0.0).astype(np.float32)   # * b_scale_inv + 0
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    D = _run(A8, 0, float(sa32), B8, 0, float(sb32), None, 0)
    got = D.cpu().view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(v)
    assert nan.any() and np.isinf(v).any() == (sb > 1e30)
    assert np.all((got[nan] & 0x7FFF) > 0x7F80), "NaN products must store a NaN"
    assert np.array_equal(got[~nan], want[~nan])


def test_gemm_banded_tile_order_covers_every_tile():
    """Operands over 256 MiB (here 270 MB) make the 256 x 256 kernels take the tile-rows in bands of
    8; with M = 8492 (34 tile-rows: bands of 8, 8, 8, 8 and 2) every output element must still be
    written exactly as the oracle says: the output starts as NaN, none may remain, and sampled
    rows from every band (the ragged last rows included) match the oracle."""
    M, N, K = 8492, 8000, 16384
    assert M * K + N * K > 256 << 20
    print(f"gemm banded M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(S.seed_for(29, 0))
    A8 = (rng.integers(0, 0x7F, (M, K), dtype=np.uint8) | (rng.integers(0, 2, (M, K), dtype=np.uint8) << 7))
    B8 = (rng.integers(0, 0x7F, (N, K), dtype=np.uint8) | (rng.integers(0, 2, (N, K), dtype=np.uint8) << 7))
    bias = S.normal_bf16(S.seed_for(29, 1), (N,), 1.0)
    D = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    F.fp8_gemm_bias(_u8(A8), 0, scalar(2.0 ** -10), _u8(B8), 0, scalar(2.0 ** -8), bf16_dev(bias), D)
    torch.cuda.synchronize()
    assert not torch.isnan(D).any().item()
    rows = np.array([0, 1, 2047, 2048, 4100, 6143, 6200, 8191, 8192, 8300, M - 2, M - 1])
    Rr, _ = oracle.gemm_bias_sampled(A8, 0, 2.0 ** -10, B8, 0, 2.0 ** -8, bias, rows, [0])
    gemm_close(to_f64(D)[rows], Rr, bf16_out=False)
