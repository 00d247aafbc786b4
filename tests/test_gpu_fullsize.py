"""Full-size parity of the training step the benchmark times: the GPT-175B QKV projection at
one TP=2 rank's share (M = 8192 tokens, K = 12288, N = 18432), forward and backward through
fp8_linear_fwd / fp8_linear_bwd, the GPU casts feeding the GPU GEMMs.

Bit for bit against the oracle: x8 / x8^T / W8 / W8^T (E4M3), dy8 / dy8^T (E5M2), the three
amaxes and the private inverse scales.  Within the gates: y (bfloat16) and dx (bfloat16) on 64
seeded full rows and 64 seeded full columns, dW (float32: the 2e-3 normwise gate alone) the same
way, dbias within its summation bound.  The oracle's GEMMs take the oracle's own codes, which
must equal the GPU's, so the GEMM check covers the GPU GEMMs on the GPU-made operands.

Inputs as the benchmark's: x ~ N(0,1), W ~ N(0,0.02), bias ~ N(0,0.1), dy ~ N(0,0.01) (seeded
bfloat16).  Scales fixed at powers of two near the steady state (x 64, W 4096, dy 2^20: a few
dy values saturate at the E5M2 maximum)."""
import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, bf16_dev, bf16_host, f32_bits, gemm_close, oracle_cast_transpose_rows, to_f64, u8_host

pytestmark = pytest.mark.gpu

M, K, N = 8192, 12288, 18432
SX, SW, SDY = 64.0, 4096.0, 2.0 ** 20


@pytest.fixture(scope="module")
def step():
    print("full-size QKV step: generating inputs", flush=True)
    xh = S.normal_bf16(S.seed_for(4, 0), (M, K), 1.0)
    wh = S.normal_bf16(S.seed_for(4, 1), (N, K), 0.02)
    bh = S.normal_bf16(S.seed_for(4, 2), (N,), 0.1)
    dyh = S.normal_bf16(S.seed_for(4, 3), (M, N), 0.01)
    u8 = dict(device=DEV, dtype=torch.uint8)
    f32 = dict(device=DEV, dtype=torch.float32)
    scale = torch.tensor([SX, SW, SDY], **f32)
    hist = torch.zeros((4, 3), **f32)
    sinv = torch.zeros(3, **f32)
    x8, x8t = torch.empty((M, K), **u8), torch.empty((K, M), **u8)
    w8, w8t = torch.empty((N, K), **u8), torch.empty((K, N), **u8)
    dy8, dy8t = torch.empty((M, N), **u8), torch.empty((N, M), **u8)
    y = torch.empty((M, N), device=DEV, dtype=torch.bfloat16)
    dx = torch.empty((M, K), device=DEV, dtype=torch.bfloat16)
    dw = torch.empty((N, K), **f32)
    db = torch.empty(N, **f32)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(M, N), **u8)
    print("full-size QKV step: fwd + bwd on the GPU", flush=True)
    F.fp8_linear_fwd(bf16_dev(xh), bf16_dev(wh), bf16_dev(bh), scale[0:1], hist[0, 0:1], x8, x8t, sinv[0:1],
                     scale[1:2], hist[0, 1:2], w8, w8t, sinv[1:2], None, y)
    F.fp8_linear_bwd(bf16_dev(dyh), K, scale[2:3], hist[0, 2:3], dy8, dy8t, sinv[2:3], db, ws, x8t, sinv[0:1], w8t,
                     sinv[1:2], dx, dw)
    torch.cuda.synchronize()
    g = dict(x8=u8_host(x8), x8t=u8_host(x8t), w8=u8_host(w8), w8t=u8_host(w8t), dy8=u8_host(dy8),
             dy8t=u8_host(dy8t), amax=hist[0].cpu().numpy(), sinv=sinv.cpu().numpy(), y=to_f64(y), dx=to_f64(dx),
             dw=to_f64(dw), db=db.cpu().numpy().astype(np.float64))
    del x8, x8t, w8, w8t, dy8, dy8t, y, dx, dw, ws
    torch.cuda.empty_cache()
    print("full-size QKV step: oracle casts", flush=True)
    r = {}
    r["x8"], r["x8t"], r["x_amax"], r["x_sinv"], _ = oracle_cast_transpose_rows(oracle, xh, SX, oracle.E4M3)
    r["w8"], r["w8t"], r["w_amax"], r["w_sinv"], _ = oracle_cast_transpose_rows(oracle, wh, SW, oracle.E4M3)
    r["dy8"], r["dy8t"], r["dy_amax"], r["dy_sinv"], r["db"] = oracle_cast_transpose_rows(
        oracle, dyh, SDY, oracle.E5M2, with_dbias=True)
    r["bias"] = bh
    r["dy_abs_colsum"] = np.abs(S.bf16_bits_to_f64(dyh)).sum(axis=0)
    return g, r


def test_fullsize_forward_casts(step):
    g, r = step
    assert np.array_equal(g["x8"], r["x8"]) and np.array_equal(g["x8t"], r["x8t"])
    assert np.array_equal(g["w8"], r["w8"]) and np.array_equal(g["w8t"], r["w8t"])
    assert f32_bits(g["amax"][0]) == f32_bits(r["x_amax"]) and f32_bits(g["amax"][1]) == f32_bits(r["w_amax"])
    assert f32_bits(g["sinv"][0]) == f32_bits(r["x_sinv"]) and f32_bits(g["sinv"][1]) == f32_bits(r["w_sinv"])


def test_fullsize_backward_casts_and_dbias(step):
    g, r = step
    assert np.array_equal(g["dy8"], r["dy8"]) and np.array_equal(g["dy8t"], r["dy8t"])
    assert f32_bits(g["amax"][2]) == f32_bits(r["dy_amax"]) and f32_bits(g["sinv"][2]) == f32_bits(r["dy_sinv"])
    assert np.all(np.abs(g["db"] - r["db"]) <= 1e-5 * r["dy_abs_colsum"] + 1e-30)


def _sampled(which, g, r):
    rows_n = {"y": M, "dx": M, "dw": N}[which]
    cols_n = {"y": N, "dx": K, "dw": K}[which]
    rows = (S.uniform(S.seed_for(4, 20), 0, 64) * rows_n).astype(np.int64)
    cols = (S.uniform(S.seed_for(4, 21), 0, 64) * cols_n).astype(np.int64)
    if which == "y":
        args = (r["x8"], oracle.E4M3, r["x_sinv"], r["w8"], oracle.E4M3, r["w_sinv"], r["bias"])
    elif which == "dx":
        args = (r["dy8"], oracle.E5M2, r["dy_sinv"], r["w8t"], oracle.E4M3, r["w_sinv"], None)
    else:
        args = (r["dy8t"], oracle.E5M2, r["dy_sinv"], r["x8t"], oracle.E4M3, r["x_sinv"], None)
    print(f"full-size {which}: oracle on 64 rows + 64 columns", flush=True)
    Rr, Rc = oracle.gemm_bias_sampled(*args, rows, cols)
    big = max(float(np.abs(Rr).max()), float(np.abs(Rc).max()))
    D = g[which]
    e1 = gemm_close(D[rows], Rr, bf16_out=which != "dw", scale_ref=big)
    e2 = gemm_close(D[:, cols], Rc, bf16_out=which != "dw", scale_ref=big)
    return max(e1, e2)


@pytest.mark.parametrize("which", ["y", "dx", "dw"])
def test_fullsize_gemms_sampled(step, which):
    """Forward y = x8 W8^T + bias (bf16), dgrad dx = dy8 (W8^T)^T (bf16) and wgrad
    dW = dy8^T (x8^T)^T (float32) on 64 seeded full rows and 64 seeded full columns."""
    err = _sampled(which, *step)
    print(f"full-size {which}: normwise error {err:.3e}", flush=True)
