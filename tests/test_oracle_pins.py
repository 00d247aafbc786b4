"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one oracle function against hand-worked values (tests/golden/), a closed
form, an invariant, a library routine (torch's float8 dtypes, numpy) or brute force, chosen
so that a plausible slip (a dropped term, a wrong sign or index, a transposed operand, a
wrong rounding or roll direction) fails at least one of them.  CPU only.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")
FMT = {"E4M3": oracle.E4M3, "E5M2": oracle.E5M2}
TORCH_FP8 = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


def _rows(name):
    out = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def _f32(bits):
    return np.array([int(bits, 16)], dtype=np.uint32).view(np.float32)


def _bits(x):
    return int(np.asarray(x, dtype=np.float32).reshape(1).view(np.uint32)[0])


# ----------------------------------------------------------------------------- formats

def test_encode_golden():
    rows = _rows("fp8_encode.txt")
    assert len(rows) >= 35
    for fmt, fbits, code, *_ in rows:
        got = oracle.encode(_f32(fbits), FMT[fmt])[0]
        assert got == int(code, 16), (fmt, fbits, hex(got), code)


def test_decode_golden():
    for fmt, code, val in _rows("fp8_decode.txt"):
        got = oracle.decode(np.array([int(code, 16)], dtype=np.uint8), FMT[fmt])[0]
        if val == "nan":
            assert np.isnan(got), (fmt, code)
        else:
            assert got == float(val) and np.signbit(got) == np.signbit(float(val)), (fmt, code, got)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_matches_torch_float8(fmt):
    """All 256 codes decode as torch's OCP float8 dtypes do (a library routine)."""
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode(codes, fmt)
    ref = torch.from_numpy(codes.copy()).view(TORCH_FP8[fmt]).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    m = ~np.isnan(ours)
    assert np.array_equal(ours[m], ref[m])
    assert np.array_equal(np.signbit(ours[m]), np.signbit(ref[m]))


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_format_counts_and_max(fmt):
    """Structure fixed by the definitions: E4M3 has 2 NaN codes and no inf; E5M2 has 6 NaN
    codes and 2 infinities; the largest finite values are 448 and 57344."""
    v = oracle.decode(np.arange(256, dtype=np.uint8), fmt)
    if fmt == oracle.E4M3:
        assert np.isnan(v).sum() == 2 and np.isinf(v).sum() == 0
        assert oracle.fp8_max(fmt) == 448.0
    else:
        assert np.isnan(v).sum() == 6 and np.isinf(v).sum() == 2
        assert oracle.fp8_max(fmt) == 57344.0
    fin = v[np.isfinite(v)]
    assert fin.max() == oracle.fp8_max(fmt)
    # positive finite codes are strictly increasing in value
    pos = v[:128][np.isfinite(v[:128])]
    assert np.all(np.diff(pos) > 0)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_decode_roundtrip(fmt):
    codes = np.arange(256, dtype=np.uint8)
    v = oracle.decode(codes, fmt)
    keep = np.isfinite(v)
    back = oracle.encode(v[keep].astype(np.float32), fmt)
    assert np.array_equal(back, codes[keep])


def _midpoints(fmt):
    """Every midpoint between adjacent finite non-negative codes, and its float32 neighbours."""
    v = oracle.decode(np.arange(128, dtype=np.uint8), fmt)
    v = v[np.isfinite(v)]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    mids = np.concatenate([mids, [np.float32((v[-1] + v[-1] * (1 + 2.0 ** -(3 if fmt == 0 else 2))) / 2)]])
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    x = np.concatenate([mids, up, dn, v.astype(np.float32)])
    return np.concatenate([x, -x]).astype(np.float32)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_agrees_with_search_encoder(fmt):
    """The grid-rounding encoder equals the independent nearest-code search on: all bfloat16
    patterns times several scales, every midpoint and its neighbours, and random float32 bits
    (NaN, inf and subnormals included)."""
    bf = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    xs = [bf.view(np.float32)]
    for s in (112.0, 2.0 ** -10, 3.0):
        with np.errstate(all="ignore"):
            xs.append((bf.view(np.float32) * np.float32(s)).astype(np.float32))
    xs.append(_midpoints(fmt))
    xs.append(S.splitmix64(12345 + fmt, 0, 300000).astype(np.uint32).view(np.float32))
    x = np.concatenate(xs)
    assert np.array_equal(oracle.encode(x, fmt), oracle.encode_search(x, fmt))


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_encode_matches_torch_float8_in_range(fmt):
    """Within [-max, max] the saturating encoder is plain round-to-nearest-even, which is what
    torch's float32 -> float8 conversion computes; outside, clamping first makes it so."""
    mx = np.float32(oracle.fp8_max(fmt))
    bf = (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(np.float32)
    rnd = S.splitmix64(999 + fmt, 0, 200000).astype(np.uint32).view(np.float32)
    x = np.concatenate([bf, rnd, _midpoints(fmt)])
    x = x[~np.isnan(x)]
    with np.errstate(invalid="ignore"):
        xc = np.clip(x, -mx, mx).astype(np.float32)
    ref = torch.from_numpy(xc).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode(x, fmt), ref)


# ----------------------------------------------------------------------------- cast, amax, transpose

@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("scale", [1.0, 112.0, 0.3, 2.0 ** -20, 5000.0])
def test_cast_matches_torch_and_amax(fmt, scale):
    """cast = one float32 product x*scale, then saturating RNE; amax = max |x| (numpy)."""
    x = S.outlier_bf16(S.seed_for(9, fmt), (97, 131), 1.0)
    q, amax, sinv = oracle.cast_amax(x, scale, fmt)
    xf = S.bf16_bits_to_f64(x).astype(np.float32)
    y = (xf * np.float32(scale)).astype(np.float32)
    mx = np.float32(oracle.fp8_max(fmt))
    ref = torch.from_numpy(np.clip(y, -mx, mx)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    assert amax == np.float32(np.abs(S.bf16_bits_to_f64(x)).max())
    assert sinv == np.float32(1.0 / np.float64(np.float32(scale)))


def test_cast_amax_folds_into_slot():
    x = S.normal_bf16(3, (64,), 1.0)
    _, a0, _ = oracle.cast_amax(x, 1.0, oracle.E4M3)
    _, a1, _ = oracle.cast_amax(x, 1.0, oracle.E4M3, amax_in=1e9)
    _, a2, _ = oracle.cast_amax(x, 1.0, oracle.E4M3, amax_in=0.25 * float(a0))
    assert a1 == np.float32(1e9) and a2 == a0


def test_amax_special_tensors():
    z = np.zeros((64, 64), dtype=np.uint16)
    assert oracle.cast_amax(z, 1.0, oracle.E4M3)[1] == 0.0
    t = S.tiny_bf16(S.seed_for(2, 5), (1024, 1024))
    q, amax, _ = oracle.cast_amax(t, 1.0, oracle.E4M3)
    assert _bits(amax) == 0x00010000          # 2^-133, the bfloat16 0x0001 pattern widened
    # 2^-133 * 1 encodes to a signed zero
    neg = (t & 0x8000) != 0
    assert np.all(q[neg] == 0x80) and np.all(q[~neg] == 0x00)
    # NaN input makes the amax NaN
    n = np.array([0x3F80, 0x7FC0, 0x4000], dtype=np.uint16)
    assert np.isnan(oracle.cast_amax(n, 1.0, oracle.E4M3)[1])


def test_transpose_worked_4x4():
    # values that are exact in E4M3: code(k) for the integers below
    vals = np.array([[1, 2, 3, 4], [-1, -2, -3, -4], [0.5, 0.25, 8, 16], [448, -448, 0, 6]], dtype=np.float32)
    x = (vals.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    q, qt, amax, _ = oracle.cast_transpose(x, 1.0, oracle.E4M3)
    # hand-worked codes: 1=0x38 2=0x40 3=0x44 4=0x48 0.5=0x30 0.25=0x28 8=0x50 16=0x58 448=0x7e 6=0x4c
    want = np.array([[0x38, 0x40, 0x44, 0x48], [0xB8, 0xC0, 0xC4, 0xC8],
                     [0x30, 0x28, 0x50, 0x58], [0x7E, 0xFE, 0x00, 0x4C]], dtype=np.uint8)
    assert np.array_equal(q, want)
    assert np.array_equal(qt, want.T)
    assert amax == 448.0


@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (64, 33), (130, 257)])
def test_transpose_involution(shape):
    x = S.normal_bf16(S.seed_for(8, shape[0]), shape, 2.0)
    q, qt, _, _ = oracle.cast_transpose(x, 3.0, oracle.E5M2)
    assert qt.shape == (shape[1], shape[0])
    assert np.array_equal(qt.T, q)
    # transposing the transpose's source gives back the row-major codes
    q2, q2t, _, _ = oracle.cast_transpose(np.ascontiguousarray(x.T), 3.0, oracle.E5M2)
    assert np.array_equal(q2, qt) and np.array_equal(q2t, q)


# ----------------------------------------------------------------------------- dbias

def test_dbias_closed_forms():
    R, C = 8192, 8
    x = np.zeros((R, C), dtype=np.float32)
    x[:, 0] = 0.5                                      # 0.5 * 8192 = 4096
    x[:, 1] = np.where(np.arange(R) % 2 == 0, 3.0, -3.0)   # cancels to 0
    x[:, 2] = -2.0 ** -10                              # -8
    x[:, 3] = np.arange(R) % 4                         # 0+1+2+3 per 4 rows: 6 * 2048
    x[5, 4] = 7.0                                      # a single entry
    b = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    db = oracle.dbias(b)
    assert list(db[:5]) == [4096.0, 0.0, -8.0, 12288.0, 7.0]
    assert np.all(db[5:] == 0.0)


def test_dbias_matches_numpy_sum():
    dy = S.normal_bf16(S.seed_for(3, 0), (513, 77), 0.01)
    ref = S.bf16_bits_to_f64(dy).sum(axis=0)
    assert np.allclose(oracle.dbias(dy), ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- scale update

def test_scale_update_golden():
    for fmt, abits, margin, prev, ws, wsi, *_ in _rows("scale_update.txt"):
        L, T = 4, 1
        h = np.zeros((L, T), dtype=np.float32)
        h[0, 0] = _f32(abits)[0]
        s0 = _f32(prev)
        h2, s, si = oracle.scale_update(h, s0, 1.0 / s0, [FMT[fmt]], int(margin))
        assert _bits(s[0]) == int(ws, 16), (abits, margin, hex(_bits(s[0])))
        assert _bits(si[0]) == int(wsi, 16), (abits, margin, hex(_bits(si[0])))


def test_scale_update_window_golden():
    """Hand-worked whole windows: a NaN in any row (not only row 0) keeps the previous scale,
    the max may sit in any row, and the roll moves every row one place towards row 0."""
    for fmt, margin, prev, hist, ws, wsi, rolled, *_ in _rows("scale_update_window.txt"):
        h = np.array([int(v, 16) for v in hist.split(",")], np.uint32).view(np.float32).reshape(-1, 1)
        s0 = _f32(prev)
        h2, s, si = oracle.scale_update(h, s0, 1.0 / s0, [FMT[fmt]], int(margin))
        assert _bits(s[0]) == int(ws, 16), (hist, hex(_bits(s[0])))
        assert _bits(si[0]) == int(wsi, 16), (hist, hex(_bits(si[0])))
        want = [int(v, 16) for v in rolled.split(",")]
        assert [int(b) for b in np.asarray(h2, np.float32).reshape(-1).view(np.uint32)] == want, hist


def test_scale_update_l1_reduces_to_fp8max_over_amax():
    a = S.log_uniform_f32(77, 200, 1e-3, 1e3)
    for fmt in (oracle.E4M3, oracle.E5M2):
        h, s, si = oracle.scale_update(a.reshape(1, -1), np.ones(200, np.float32), np.ones(200, np.float32),
                                       [fmt] * 200, 0)
        want = (np.float32(oracle.fp8_max(fmt)) / a).astype(np.float32)
        assert np.array_equal(s, want)
        assert np.array_equal(si, (np.float32(1) / want).astype(np.float32))
        assert np.all(h == 0)


@pytest.mark.parametrize("L", [1, 2, 5, 16])
def test_scale_update_sliding_window_brute_force(L):
    """3L iterations: each writes its amax into row 0, then updates.  The scale must equal
    fp8_max over the max of the last L amaxes (current included), computed by brute force
    over the list of all amaxes; the previous scale survives an all-zero window."""
    T = 3
    fmts = [oracle.E4M3, oracle.E4M3, oracle.E5M2]
    steps = 3 * L + 2
    am = S.log_uniform_f32(5 + L, steps * T, 1e-3, 1e3).reshape(steps, T)
    am[steps // 2: steps // 2 + L, 1] = 0.0            # a window of zeros for tensor 1
    h = np.zeros((L, T), np.float32)
    s = np.ones(T, np.float32)
    si = np.ones(T, np.float32)
    prev = s.copy()
    for k in range(steps):
        h[0] = am[k]
        h, s, si = oracle.scale_update(h, s, si, fmts, 0)
        for t in range(T):
            window = am[max(0, k - L + 1): k + 1, t]
            a = np.float32(window.max())
            if a == 0:
                want = prev[t]
            else:
                want = np.float32(np.float32(oracle.fp8_max(fmts[t])) / a)
            assert s[t] == want, (L, k, t)
        prev = s.copy()
        # history keeps the last L-1 amaxes in rows L-1 (newest) .. 1 (oldest); row 0 is clear
        assert np.all(h[0] == 0)
        for j in range(1, L):
            idx = k - (L - 1 - j)
            want_row = am[idx] if idx >= 0 else np.zeros(T, np.float32)
            assert np.array_equal(h[j], want_row), (L, k, j)


# ----------------------------------------------------------------------------- GEMM

def _e4m3_int_codes(vals):
    """E4M3 codes of small integers, hand-worked: 0=0x00 1=0x38 2=0x40 3=0x44 4=0x48 5=0x4a 6=0x4c."""
    tab = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C}
    v = np.asarray(vals)
    return np.vectorize(lambda z: tab[abs(int(z))] | (0x80 if z < 0 else 0))(v).astype(np.uint8)


def test_gemm_4x4_brute_force_integers():
    rng = np.random.default_rng(0)
    Ai = rng.integers(-6, 7, size=(4, 4))
    Bi = rng.integers(-6, 7, size=(4, 4))
    A, B = _e4m3_int_codes(Ai), _e4m3_int_codes(Bi)
    want = (Ai @ Bi.T).astype(np.float64)         # integer matmul: exact
    assert np.array_equal(oracle.gemm_bias(A, 0, 1.0, B, 0, 1.0), want)
    assert np.array_equal(oracle.gemm_bias_scalar(A, 0, 1.0, B, 0, 1.0), want)
    # hand-worked element: row 0 of A with row 2 of B
    assert want[0, 2] == sum(Ai[0, k] * Bi[2, k] for k in range(4))


def test_gemm_nonsquare_integer_matmul_and_scales():
    rng = np.random.default_rng(1)
    M, N, K = 5, 3, 7
    Ai = rng.integers(-6, 7, size=(M, K))
    Bi = rng.integers(-6, 7, size=(N, K))
    bias = np.array([0x3F80, 0xC000, 0x3E80], dtype=np.uint16)   # 1.0, -2.0, 0.25
    R = oracle.gemm_bias(_e4m3_int_codes(Ai), 0, 0.5, _e4m3_int_codes(Bi), 0, 0.25, bias)
    want = (Ai @ Bi.T) * 0.125 + np.array([1.0, -2.0, 0.25])[None, :]
    assert R.shape == (M, N)
    assert np.array_equal(R, want)


def test_gemm_identity_returns_dequantised_a():
    A = S.normal_bf16(11, (6, 16), 3.0)
    A8, _, _ = oracle.cast_amax(A, 1.0, oracle.E5M2)
    I = np.where(np.eye(16, dtype=bool), 0x38, 0x00).astype(np.uint8)    # E4M3 1.0 on the diagonal
    R = oracle.gemm_bias(A8, oracle.E5M2, 1.0, I, oracle.E4M3, 1.0)
    assert np.array_equal(R, oracle.decode(A8, oracle.E5M2))
    # identity on the left gives B itself (rows of R = rows of the identity times B^T)
    R2 = oracle.gemm_bias(I, oracle.E4M3, 1.0, A8, oracle.E5M2, 1.0)
    assert np.array_equal(R2, oracle.decode(A8, oracle.E5M2).T)


def test_gemm_k1_outer_product_and_zero_a_bias():
    a = np.array([[0x38], [0x40], [0xC4]], dtype=np.uint8)   # 1, 2, -3
    b = np.array([[0x48], [0x30]], dtype=np.uint8)           # 4, 0.5
    assert np.array_equal(oracle.gemm_bias(a, 0, 1.0, b, 0, 1.0), np.outer([1, 2, -3], [4, 0.5]))
    bias = S.normal_bf16(12, (9,), 0.1)
    R = oracle.gemm_bias(np.zeros((4, 32), np.uint8), 0, 1.0, S.splitmix64(4, 0, 9 * 32).astype(np.uint8).reshape(9, 32) & 0x77,
                         0, 1.0, bias)
    assert np.array_equal(R, np.tile(S.bf16_bits_to_f64(bias), (4, 1)))


def test_gemm_matches_torch_float8_matmul():
    """Random codes, all four format pairs: the dequantise-then-matmul path equals torch's
    float8 decode and a float64 torch matmul, and the scalar C triple loop."""
    M, N, K = 17, 23, 48
    for fa in (0, 1):
        for fb in (0, 1):
            A = S.normal_bf16(20 + fa, (M, K), 2.0)
            B = S.normal_bf16(30 + fb, (N, K), 2.0)
            A8 = oracle.cast_amax(A, 1.0, fa)[0]
            B8 = oracle.cast_amax(B, 1.0, fb)[0]
            bias = S.normal_bf16(40, (N,), 0.1)
            R = oracle.gemm_bias(A8, fa, 0.75, B8, fb, 1.5, bias)
            ta = torch.from_numpy(A8.copy()).view(TORCH_FP8[fa]).to(torch.float64)
            tb = torch.from_numpy(B8.copy()).view(TORCH_FP8[fb]).to(torch.float64)
            ref = (ta @ tb.T) * 0.75 * 1.5 + torch.from_numpy(S.bf16_bits_to_f64(bias))[None, :]
            assert np.allclose(R, ref.numpy(), rtol=1e-13, atol=1e-13)
            assert np.allclose(R, oracle.gemm_bias_scalar(A8, fa, 0.75, B8, fb, 1.5, bias), rtol=1e-13, atol=1e-13)


def test_gemm_chunked_equals_unchunked():
    """Each N-chunk with its own bias offset ("Userbuffers support in operation-based API",
    the bias-offset fix) reproduces the columns of the unchunked GEMM exactly."""
    M, N, K = 9, 24, 32
    A8 = oracle.cast_amax(S.normal_bf16(50, (M, K), 1.0), 1.0, 0)[0]
    B8 = oracle.cast_amax(S.normal_bf16(51, (N, K), 1.0), 1.0, 0)[0]
    bias = S.normal_bf16(52, (N,), 0.5)
    full = oracle.gemm_bias(A8, 0, 1.0, B8, 0, 1.0, bias)
    for chunks in (2, 3, 4):
        nc = N // chunks
        parts = [oracle.gemm_bias(A8, 0, 1.0, B8[c * nc:(c + 1) * nc], 0, 1.0, bias[c * nc:(c + 1) * nc])
                 for c in range(chunks)]
        assert np.array_equal(np.concatenate(parts, axis=1), full)


def test_gemm_sampled_rows_cols_match_full():
    M, N, K = 40, 30, 64
    A8 = oracle.cast_amax(S.normal_bf16(60, (M, K), 1.0), 1.0, 1)[0]
    B8 = oracle.cast_amax(S.normal_bf16(61, (N, K), 1.0), 1.0, 0)[0]
    bias = S.normal_bf16(62, (N,), 0.5)
    full = oracle.gemm_bias(A8, 1, 2.0, B8, 0, 0.5, bias)
    rr, rc = oracle.gemm_bias_sampled(A8, 1, 2.0, B8, 0, 0.5, bias, [0, 7, 39], [1, 29])
    assert np.array_equal(rr, full[[0, 7, 39]])
    assert np.array_equal(rc, full[:, [1, 29]])


# ----------------------------------------------------------------------------- composition

def test_linear_fwd_bwd_shapes_and_definitions():
    M, N, K = 32, 48, 64
    x = S.normal_bf16(70, (M, K), 1.0)
    w = S.normal_bf16(71, (N, K), 0.02)
    b = S.normal_bf16(72, (N,), 0.1)
    dy = S.normal_bf16(73, (M, N), 0.01)
    f = oracle.linear_fwd(x, w, b, 1.0, 64.0)
    assert f["y"].shape == (M, N) and f["x8t"].shape == (K, M) and f["w8t"].shape == (K, N)
    # y against the float64 product of the dequantised operands, by torch
    xd = torch.from_numpy(f["x8"].copy()).view(torch.float8_e4m3fn).to(torch.float64) * float(f["x_sinv"])
    wd = torch.from_numpy(f["w8"].copy()).view(torch.float8_e4m3fn).to(torch.float64) * float(f["w_sinv"])
    ref = xd @ wd.T + torch.from_numpy(S.bf16_bits_to_f64(b))
    assert np.allclose(f["y"], ref.numpy(), rtol=1e-12, atol=1e-12)
    g = oracle.linear_bwd(dy, 4096.0, f["x8t"], f["x_sinv"], f["w8t"], f["w_sinv"])
    assert g["dx"].shape == (M, K) and g["dw"].shape == (N, K) and g["dbias"].shape == (N,)
    dyd = torch.from_numpy(g["dy8"].copy()).view(torch.float8_e5m2).to(torch.float64) * float(g["dy_sinv"])
    assert np.allclose(g["dx"], (dyd @ wd).numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dw"], (dyd.T @ xd).numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dbias"], S.bf16_bits_to_f64(dy).sum(0), atol=1e-12)


# ----------------------------------------------------------------------------- FP8 transpose

def _hex_block(rows):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=np.uint8)


def test_fp8_transpose_golden():
    rows = _rows("fp8_transpose.txt")
    cut = [r[0] for r in rows].index("out_t")
    src, want = _hex_block(rows[1:cut]), _hex_block(rows[cut + 1:])
    assert src.shape == (3, 5) and want.shape == (5, 3)
    assert np.array_equal(oracle.fp8_transpose(src), want)


@pytest.mark.parametrize("shape", [(1, 1), (1, 7), (9, 1), (17, 33), (64, 48)])
def test_fp8_transpose_brute_force_and_involution(shape):
    R, C = shape
    rng = np.random.default_rng(R * 1000 + C)
    x = rng.integers(0, 256, size=shape, dtype=np.uint8)
    t = oracle.fp8_transpose(x)
    assert t.shape == (C, R)
    for i in range(R):
        for j in range(C):
            assert t[j, i] == x[i, j]
    assert np.array_equal(oracle.fp8_transpose(t), x)


def test_fp8_transpose_empty_and_noop():
    assert oracle.fp8_transpose(np.zeros((0, 5), np.uint8)).shape == (5, 0)
    x = np.arange(12, dtype=np.uint8).reshape(3, 4)
    stale = np.full((4, 3), 0xAB, dtype=np.uint8)
    assert np.array_equal(oracle.fp8_transpose(x, noop=True, out_t_prev=stale), stale)
    with pytest.raises(ValueError):
        oracle.fp8_transpose(x, noop=True)


def test_cast_transpose_is_cast_then_transpose():
    x = S.normal_bf16(S.seed_for(9, 0), (40, 24), 1.0)
    q, qt, _, _ = oracle.cast_transpose(x, 3.0, oracle.E4M3)
    assert np.array_equal(oracle.fp8_transpose(q), qt)


# ----------------------------------------------------------------------------- FP8-output GEMM

def test_cast_f32_amax_matches_bf16_cast_on_bf16_values():
    # float32 inputs that are exactly bfloat16 values (every pattern, incl. inf, NaN, -0) must
    # cast exactly like the bfloat16 cast, whose encoder and amax are pinned above.
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xf = (allb.astype(np.uint32) << np.uint32(16)).view(np.float32)
    for fmt in (oracle.E4M3, oracle.E5M2):
        for s in (1.0, 0.0625, 3.0, 1e-30):
            q1, a1, si1 = oracle.cast_amax(allb, s, fmt)
            q2, a2, si2 = oracle.cast_f32_amax(xf, s, fmt)
            assert np.array_equal(q1, q2)
            assert _bits(a1) == _bits(a2) and _bits(si1) == _bits(si2)
    finite = xf[np.isfinite(xf)]
    _, a, _ = oracle.cast_f32_amax(finite, 1.0, oracle.E4M3)
    assert a == np.abs(finite).max()


def test_gemm_fp8_output_golden():
    A = np.full((2, 64), 0x38, dtype=np.uint8)
    B = np.full((4, 64), 0x38, dtype=np.uint8)
    bias = np.array([0x0000, 0x3F00, 0xC1A0, 0x4396], dtype=np.uint16)
    rows = _rows("fp8_gemm_fp8out.txt")
    assert len(rows) == 5
    for fmt, sbits, abits, c0, c1, c2, c3, amax_bits, sinv_bits in rows:
        codes, amax, sinv, D = oracle.gemm_bias_fp8(A, oracle.E4M3, 0.5, B, oracle.E4M3, 0.25, bias, FMT[fmt],
                                                    _f32(sbits)[0], _f32(abits)[0])
        assert np.array_equal(D, np.tile(np.array([8, 8.5, -12, 308], np.float32), (2, 1)))
        want = np.array([int(c, 16) for c in (c0, c1, c2, c3)], dtype=np.uint8)
        assert np.array_equal(codes, np.tile(want, (2, 1))), (fmt, sbits, codes)
        assert _bits(amax) == int(amax_bits, 16) and _bits(sinv) == int(sinv_bits, 16)


@pytest.mark.parametrize("fmt_out", [oracle.E4M3, oracle.E5M2])
def test_gemm_fp8_output_identity_weight(fmt_out):
    # B = identity (code 1.0 on the diagonal): D = dec(A) * sa * sb + bias exactly, with the
    # A operand's row/column roles visible (A is not square).  Reference built from the pinned
    # decode and the independent nearest-code search encoder.
    M, K = 24, 32
    rng = np.random.default_rng(7)
    A = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x3C                      # no NaN codes
    B = np.zeros((K, K), dtype=np.uint8)
    np.fill_diagonal(B, 0x38)
    bias = S.normal_bf16(S.seed_for(9, 1), (K,), 0.5)
    sa, sb, ds = np.float32(0.75), np.float32(2.0), np.float32(0.3)
    codes, amax, sinv, D = oracle.gemm_bias_fp8(A, oracle.E4M3, sa, B, oracle.E4M3, sb, bias, fmt_out, ds)
    bias_f = (bias.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    ref = (oracle.decode(A, oracle.E4M3) * np.float64(sa) * np.float64(sb) + bias_f[None, :]).astype(np.float32)
    assert np.array_equal(D, ref)
    assert np.array_equal(codes, oracle.encode_search(ref * ds, fmt_out))
    assert amax == np.abs(ref).max()
    assert _bits(sinv) == _bits(np.float32(1) / ds)
