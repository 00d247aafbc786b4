"""CPU oracle of per-tensor FP8 delayed scaling: plain, slow and obviously correct.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the HIP library under
``fp8_delayed_scaling_amd/`` and never imports it.

The element-wise arithmetic (FP8 encode/decode, cast, amax, transpose, dbias, the scale
update) lives in ``fp8_oracle.c`` (scalar C, float64 where the definition allows it); this
module marshals numpy arrays into it and composes the steps.  The GEMM is the plain
definition: dequantise each FP8 code by the format's closed form (C), then one float64
matrix product (numpy), then the two inverse scales and the bias in float64.

Sources (cited by page title and section):
  * "[PyTorch] Refactor FP8 workspaces in linear modules" (TransformerEngine PR 820),
    Motivations: the FP8 scale-update kernel, the too-tiny-amax guard, the private
    scale-inverse copy a Float8Tensor keeps; "grown in scope": the transpose cache.
  * "[PyTorch] cuda graph support" (PR 575), feature list (amax reduction per iteration,
    persistent transposes) and the transpose-cache thread (DbiasCastTranspose,
    Float8Tensor.to_float8, fp8_gemm in FP8Linear.backward).
  * "[PyTorch] Userbuffers support in operation-based API" (PR 1142): each output chunk of
    a chunked GEMM adds its own chunk of the bias.
  * The OCP "8-bit Floating Point Specification (OFP8)" for the E4M3 / E5M2 bit formats,
    which the pages do not state.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

E4M3 = 0
E5M2 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile ``fp8_oracle.c`` into ``liboracle.so`` with gcc (no fast-math, no FTZ)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        f32 = ctypes.c_float
        L.orc_fp8_decode.argtypes = [ctypes.c_uint8, i32]
        L.orc_fp8_decode.restype = ctypes.c_double
        L.orc_fp8_encode.argtypes = [f32, i32]
        L.orc_fp8_encode.restype = ctypes.c_uint8
        L.orc_fp8_encode_search.argtypes = [f32, i32]
        L.orc_fp8_encode_search.restype = ctypes.c_uint8
        L.orc_fp8_max.argtypes = [i32]
        L.orc_fp8_max.restype = ctypes.c_double
        L.orc_fp8_encode_n.argtypes = [P, i64, i32, P]
        L.orc_fp8_encode_search_n.argtypes = [P, i64, i32, P]
        L.orc_fp8_decode_n.argtypes = [P, i64, i32, P]
        L.orc_cast_amax.argtypes = [P, i64, f32, i32, P, P]
        L.orc_cast_transpose.argtypes = [P, i64, i64, f32, i32, P, P, P]
        L.orc_dbias.argtypes = [P, i64, i64, P]
        L.orc_fp8_transpose.argtypes = [P, i64, i64, P]
        L.orc_cast_f32_amax.argtypes = [P, i64, f32, i32, P, P]
        L.orc_scale_inv.argtypes = [f32]
        L.orc_scale_inv.restype = f32
        L.orc_scale_update.argtypes = [P, i64, i64, P, P, P, ctypes.c_int32]
        L.orc_dequant.argtypes = [P, i64, i64, i64, i32, P]
        L.orc_gemm_bias_scalar.argtypes = [P, i32, f32, i64, P, i32, f32, i64, P, i64, i64, i64, P, i64]
        for fn in ("orc_fp8_encode_n", "orc_fp8_encode_search_n", "orc_fp8_decode_n", "orc_cast_amax",
                   "orc_cast_transpose", "orc_dbias", "orc_scale_update", "orc_dequant",
                   "orc_gemm_bias_scalar", "orc_fp8_transpose", "orc_cast_f32_amax"):
            getattr(L, fn).restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


# ----------------------------------------------------------------------------- format

def fp8_max(fmt: int) -> float:
    """Largest finite magnitude of the format (448 for E4M3, 57344 for E5M2)."""
    return lib().orc_fp8_max(fmt)


def decode(codes, fmt: int) -> np.ndarray:
    """float64 values of FP8 codes (closed form of the OCP bit fields)."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().orc_fp8_decode_n(_p(c), c.size, fmt, _p(out))
    return out


def encode(x, fmt: int) -> np.ndarray:
    """Saturating round-to-nearest-even FP8 codes of float32 values."""
    f = _c(x, np.float32)
    out = np.empty(f.shape, dtype=np.uint8)
    lib().orc_fp8_encode_n(_p(f), f.size, fmt, _p(out))
    return out


def encode_search(x, fmt: int) -> np.ndarray:
    """The independent nearest-code search encoder (cross-check of ``encode``)."""
    f = _c(x, np.float32)
    out = np.empty(f.shape, dtype=np.uint8)
    lib().orc_fp8_encode_search_n(_p(f), f.size, fmt, _p(out))
    return out


def scale_inv(scale: float) -> np.float32:
    """The private inverse scale a cast records: float32 1/scale."""
    return np.float32(lib().orc_scale_inv(np.float32(scale)))


# ----------------------------------------------------------------------------- casts

def cast_amax(x_bf16, scale: float, fmt: int, amax_in: float = 0.0):
    """FP8 codes of ``x * scale`` and the amax folded into ``amax_in``.

    Returns ``(codes, amax, scale_inv)`` with ``amax`` a float32.
    """
    x = _c(x_bf16, np.uint16)
    out = np.empty(x.shape, dtype=np.uint8)
    amax = np.array([amax_in], dtype=np.float32)
    lib().orc_cast_amax(_p(x), x.size, np.float32(scale), fmt, _p(out), _p(amax))
    return out, amax[0], scale_inv(scale)


def cast_transpose(x_bf16, scale: float, fmt: int, amax_in: float = 0.0):
    """``(codes [R,C], codes_t [C,R], amax, scale_inv)`` of a 2-D bfloat16 tensor."""
    x = _c(x_bf16, np.uint16)
    if x.ndim != 2:
        raise ValueError("cast_transpose takes a 2-D tensor")
    R, C = x.shape
    out = np.empty((R, C), dtype=np.uint8)
    out_t = np.empty((C, R), dtype=np.uint8)
    amax = np.array([amax_in], dtype=np.float32)
    lib().orc_cast_transpose(_p(x), R, C, np.float32(scale), fmt, _p(out), _p(out_t), _p(amax))
    return out, out_t, amax[0], scale_inv(scale)


def fp8_transpose(codes, noop: bool = False, out_t_prev=None) -> np.ndarray:
    """Transpose cache of an existing 2-D FP8 tensor: ``[C, R]`` codes, moved not re-encoded.

    With ``noop`` set the cache is left as it was: ``out_t_prev`` is returned unchanged (the
    weight-caching flag of [CG], "noop_flag in transpose").
    """
    c = _c(codes, np.uint8)
    if c.ndim != 2:
        raise ValueError("fp8_transpose takes a 2-D tensor")
    R, C = c.shape
    if noop:
        if out_t_prev is None:
            raise ValueError("noop needs the previous cache")
        return np.array(out_t_prev, copy=True)
    out_t = np.empty((C, R), dtype=np.uint8)
    lib().orc_fp8_transpose(_p(c), R, C, _p(out_t))
    return out_t


def cast_f32_amax(x_f32, scale: float, fmt: int, amax_in: float = 0.0):
    """``(codes, amax, scale_inv)`` of a float32 tensor cast with ``scale`` (amax of |x|)."""
    x = _c(x_f32, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    amax = np.array([amax_in], dtype=np.float32)
    lib().orc_cast_f32_amax(_p(x), x.size, np.float32(scale), fmt, _p(out), _p(amax))
    return out, amax[0], scale_inv(scale)


def dbias(dy_bf16) -> np.ndarray:
    """float64 column sums of a 2-D bfloat16 tensor."""
    x = _c(dy_bf16, np.uint16)
    R, C = x.shape
    out = np.empty(C, dtype=np.float64)
    lib().orc_dbias(_p(x), R, C, _p(out))
    return out


def dbias_cast_transpose(dy_bf16, scale: float, fmt: int, amax_in: float = 0.0):
    """``(codes, codes_t, amax, scale_inv, dbias_f64)``: dbias of the bfloat16 dy, then its cast+transpose."""
    db = dbias(dy_bf16)
    q, qt, amax, sinv = cast_transpose(dy_bf16, scale, fmt, amax_in)
    return q, qt, amax, sinv, db


# ----------------------------------------------------------------------------- recipe

def scale_update(hist, scale, scale_inv_, fmts, margin: int = 0):
    """One delayed-scaling update; returns new ``(hist [L,T], scale [T], scale_inv [T])``."""
    h = np.array(_c(hist, np.float32), copy=True)
    if h.ndim != 2:
        raise ValueError("history is [L, T]")
    L, T = h.shape
    s = np.array(_c(scale, np.float32), copy=True)
    si = np.array(_c(scale_inv_, np.float32), copy=True)
    f = np.ascontiguousarray(np.asarray(fmts, dtype=np.int32))
    if s.shape != (T,) or si.shape != (T,) or f.shape != (T,):
        raise ValueError("scale, scale_inv and fmts are [T]")
    lib().orc_scale_update(_p(h), L, T, _p(s), _p(si), _p(f), int(margin))
    return h, s, si


# ----------------------------------------------------------------------------- GEMM

def dequant(codes, fmt: int) -> np.ndarray:
    """float64 values of a 2-D FP8 operand (closed-form decode per code)."""
    c = _c(codes, np.uint8)
    if c.ndim != 2:
        raise ValueError("dequant takes a 2-D operand")
    out = np.empty(c.shape, dtype=np.float64)
    lib().orc_dequant(_p(c), c.shape[0], c.shape[1], c.shape[1], fmt, _p(out))
    return out


def _bias_f64(bias_bf16, n):
    if bias_bf16 is None:
        return np.zeros(n, dtype=np.float64)
    b = _c(bias_bf16, np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def gemm_bias(A, fa: int, a_sinv: float, B, fb: int, b_sinv: float, bias_bf16=None) -> np.ndarray:
    """R[m,n] = (sum_k dec(A[m,k]) dec(B[n,k])) * a_sinv * b_sinv + bias[n], in float64.

    A is [M, K] and B is [N, K] FP8 codes (both K-contiguous); bias is bfloat16 [N] or None.
    """
    Ad = dequant(A, fa)
    Bd = dequant(B, fb)
    if Ad.shape[1] != Bd.shape[1]:
        raise ValueError("A and B must share K")
    acc = Ad @ Bd.T
    return acc * np.float64(np.float32(a_sinv)) * np.float64(np.float32(b_sinv)) + _bias_f64(bias_bf16, Bd.shape[0])[None, :]


def gemm_bias_fp8(A, fa: int, a_sinv: float, B, fb: int, b_sinv: float, bias_bf16, d_fmt: int,
                  d_scale: float, amax_in: float = 0.0):
    """FP8-output GEMM ([CG] transpose-cache thread: fp8_gemm(..., out=dx._data)).

    The output value D is the plain GEMM+bias rounded once to float32 (the GEMM's accumulate
    and epilogue type); D is then cast like any float32 tensor with the output's own scale:
    ``codes = enc(D * d_scale)``, ``amax = max |D|`` folded into ``amax_in``, and the output's
    private inverse scale 1/d_scale.  Returns ``(codes, amax, scale_inv, D_f32)``.
    """
    D = gemm_bias(A, fa, a_sinv, B, fb, b_sinv, bias_bf16).astype(np.float32)
    codes, amax, sinv = cast_f32_amax(D, d_scale, d_fmt, amax_in)
    return codes, amax, sinv, D


def gemm_bias_scalar(A, fa, a_sinv, B, fb, b_sinv, bias_bf16=None) -> np.ndarray:
    """The same GEMM as three nested scalar loops in C (small shapes only)."""
    A = _c(A, np.uint8)
    B = _c(B, np.uint8)
    M, K = A.shape
    N = B.shape[0]
    R = np.empty((M, N), dtype=np.float64)
    bp = None
    if bias_bf16 is not None:
        bias = _c(bias_bf16, np.uint16)
        bp = _p(bias)
    lib().orc_gemm_bias_scalar(_p(A), fa, np.float32(a_sinv), K, _p(B), fb, np.float32(b_sinv), K,
                               bp, M, N, K, _p(R), N)
    return R


def gemm_bias_sampled(A, fa, a_sinv, B, fb, b_sinv, bias_bf16, rows, cols):
    """Full output rows ``rows`` and full output columns ``cols`` of ``gemm_bias``.

    Returns ``(R_rows [len(rows), N], R_cols [M, len(cols)])``.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    b = None if bias_bf16 is None else np.asarray(bias_bf16)
    R_rows = gemm_bias(np.asarray(A)[rows], fa, a_sinv, B, fb, b_sinv, b)
    R_cols = gemm_bias(A, fa, a_sinv, np.asarray(B)[cols], fb, b_sinv, None if b is None else b[cols])
    return R_rows, R_cols


# ----------------------------------------------------------------------------- linear layer

def linear_fwd(x, w, bias, x_scale, w_scale, want_x_t=True):
    """Forward of the FP8 linear layer: cast x (E4M3), cast+transpose W (E4M3), then
    y = gemm_bias(x8, W8) with the private inverse scales.

    Returns a dict with the FP8 tensors, amaxes, inverse scales and the float64 output.
    """
    if want_x_t:
        x8, x8t, x_amax, x_sinv = cast_transpose(x, x_scale, E4M3)
    else:
        x8, x_amax, x_sinv = cast_amax(x, x_scale, E4M3)
        x8t = None
    w8, w8t, w_amax, w_sinv = cast_transpose(w, w_scale, E4M3)
    y = gemm_bias(x8, E4M3, x_sinv, w8, E4M3, w_sinv, bias)
    return dict(x8=x8, x8t=x8t, x_amax=x_amax, x_sinv=x_sinv, w8=w8, w8t=w8t, w_amax=w_amax,
                w_sinv=w_sinv, y=y)


def linear_bwd(dy, dy_scale, x8t, x_sinv, w8t, w_sinv):
    """Backward of the FP8 linear layer ([CG] transpose-cache thread, FP8Linear.backward and
    DbiasCastTranspose.backward): dbias + cast + transpose of dy (E5M2), then
    dgrad dx[M,K] = gemm(dy8 [M,N], W8^T [K,N]) and wgrad dW[N,K] = gemm(dy8^T [N,M], x8^T [K,M]).
    """
    dy8, dy8t, dy_amax, dy_sinv, db = dbias_cast_transpose(dy, dy_scale, E5M2)
    dx = gemm_bias(dy8, E5M2, dy_sinv, w8t, E4M3, w_sinv, None)
    dw = gemm_bias(dy8t, E5M2, dy_sinv, x8t, E4M3, x_sinv, None)
    return dict(dy8=dy8, dy8t=dy8t, dy_amax=dy_amax, dy_sinv=dy_sinv, dbias=db, dx=dx, dw=dw)
