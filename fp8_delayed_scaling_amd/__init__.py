"""fp8_delayed_scaling_amd -- FP8 per-tensor delayed scaling on AMD MI355X (gfx950).

A thin ctypes binding of ``libfp8ds.so`` (the HIP kernels behind the C ABI of
``include/fp8ds.h``).  Every function here has the name of its C entry point and only
marshals arguments: it reads sizes, strides and pointers off torch tensors, picks the
stream, calls the library and turns a non-zero status into an exception.  All arithmetic
runs in the library's kernels; PyTorch only supplies device memory and streams.

The library must be built (``__graft_entry__.build()`` or ``python -m
fp8_delayed_scaling_amd.build``); importing this package without it raises immediately,
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence

import torch

__all__ = [
    "E4M3", "E5M2", "OUT_BF16", "OUT_FP32", "Fp8dsError", "lib", "library_path",
    "fp8ds_status_string", "fp8ds_version",
    "fp8_cast_amax", "fp8_cast_transpose", "fp8_dbias_workspace_bytes", "fp8_dbias_cast_transpose",
    "fp8_dbias_cast_transpose_noalloc", "fp8_scale_update", "fp8_gemm_bias", "fp8_gemm_bias_chunked", "fp8_gemm_bias_fp8", "fp8_transpose",
    "fp8_linear_fwd", "fp8_linear_bwd", "prepare", "Prepared",
]

E4M3 = 0
E5M2 = 1
OUT_BF16 = 0
OUT_FP32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libfp8ds.so")


class Fp8dsError(RuntimeError):
    """A libfp8ds call returned a non-zero status."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None
P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int32
INT = ctypes.c_int
SZ = ctypes.c_size_t

_SIGS = {
    "fp8ds_status_string": ([INT], ctypes.c_char_p),
    "fp8ds_version": ([], INT),
    "fp8_cast_amax": ([P, I64, P, INT, P, P, P, P, P], INT),
    "fp8_cast_transpose": ([P, I64, I64, P, INT, P, P, P, P, P, P], INT),
    "fp8_dbias_workspace_bytes": ([I64, I64], SZ),
    "fp8_dbias_cast_transpose": ([P, I64, I64, P, INT, P, P, P, P, P, P, SZ, P], INT),
    "fp8_dbias_cast_transpose_noalloc": ([P, I64, I64, P, INT, P, P, P, P, P, P], INT),
    "fp8_scale_update": ([P, I64, I64, P, P, P, I32, P], INT),
    "fp8_gemm_bias": ([P, INT, P, I64, P, INT, P, I64, P, P, I64, INT, I64, I64, I64, P], INT),
    "fp8_gemm_bias_chunked": ([P, INT, P, I64, P, INT, P, I64, P, P, I64, INT, I64, I64, I64, INT, P, P], INT),
    "fp8_gemm_bias_fp8": ([P, INT, P, I64, P, INT, P, I64, P, P, I64, INT, P, P, P, I64, I64, I64, P], INT),
    "fp8_transpose": ([P, I64, I64, P, P, P], INT),
    "fp8_linear_fwd": ([P, P, P, I64, I64, I64, P, P, P, P, P, P, P, P, P, P, P, P, P], INT),
    "fp8_linear_bwd": ([P, I64, I64, I64, P, P, P, P, P, P, P, SZ, P, P, P, P, P, P, INT, P], INT),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                "(the FP8 path has no fallback)")
        L = ctypes.CDLL(library_path)
        for name, (argtypes, restype) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = restype
        _lib = L
    return _lib


def fp8ds_status_string(status: int) -> str:
    return lib().fp8ds_status_string(int(status)).decode()


def fp8ds_version() -> int:
    return int(lib().fp8ds_version())


# ----------------------------------------------------------------------------- marshalling

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live on the GPU")
    return t.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int):
    if status != 0:
        raise Fp8dsError(status, fp8ds_status_string(status))


_tls = threading.local()   # .rec: the list prepare() records into, on this thread only


def _invoke(name: str, *cargs):
    """Call entry point ``name`` with marshalled arguments, or hand them to prepare()."""
    rec = getattr(_tls, "rec", None)
    if rec is not None:
        rec.append((name, cargs))
        return
    _check(getattr(lib(), name)(*cargs))


class Prepared:
    """One entry-point call whose checks and marshalling ran once, in prepare(): calling it
    repeats only the C call, with the same device pointers, sizes and stream (or ``stream``).
    It keeps the tensors it was prepared with alive; they must keep their storage (no resize,
    no set_) for as long as it is used."""

    def __init__(self, name: str, cargs, keep):
        self.name = name
        self._fn = getattr(lib(), name)
        self._args = tuple(cargs)
        self._keep = keep

    def __call__(self, stream=None):
        a = self._args if stream is None else self._args[:-1] + (_stream(stream),)
        status = self._fn(*a)
        if status != 0:
            raise Fp8dsError(status, fp8ds_status_string(status))


def prepare(fn, *args, **kwargs) -> Prepared:
    """Run the binding ``fn`` (one of the entry points above) on these arguments up to the C call
    and return that call, ready to repeat: for layers small enough that the binding's per-call
    checks cost more host time than the launch itself.  The stream is the one ``fn`` would have
    used (the current stream unless ``stream=`` is given) unless the call passes another."""
    rec = []
    _tls.rec = rec
    try:
        fn(*args, **kwargs)
    finally:
        _tls.rec = None
    if len(rec) != 1:
        raise ValueError(f"{getattr(fn, '__name__', fn)} is not a single library call")
    name, cargs = rec[0]
    return Prepared(name, cargs, (args, kwargs))


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


_F32 = (torch.float32,)
_U8 = (torch.uint8,)


def _want(t, dtypes, name, contiguous=True, shape=None, min_numel=None, required=False):
    """Check a tensor argument before its pointer goes to the library, which cannot see sizes:
    dtype, density, and the exact ``shape`` or at least ``min_numel`` elements.  A plain int is
    a raw device pointer and is passed through unchecked."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if isinstance(t, int):
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, got {t.numel()}")


def _workspace_bytes(workspace) -> int:
    """Size of a dbias workspace tensor in bytes (0 for None); it must be one dense block."""
    if workspace is None:
        return 0
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace.numel() * workspace.element_size()


def _scalars(**kw):
    """float32 device scalars (scale, inverse scale, amax slot, noop flag): one element each."""
    for name, t in kw.items():
        _want(t, _F32, name, min_numel=1)


# ----------------------------------------------------------------------------- entry points

def fp8_cast_amax(x, scale, fmt, out, scale_inv_out=None, amax_slot=None, noop=None, stream=None):
    """Cast bfloat16 ``x`` to FP8 codes ``out`` with amax capture (see include/fp8ds.h)."""
    _want(x, _BF16, "x", required=True)
    _want(out, _U8, "out", required=True)
    if out.numel() != x.numel():
        raise ValueError("out must have x's number of elements")
    _scalars(scale=scale, scale_inv_out=scale_inv_out, amax_slot=amax_slot, noop=noop)
    _invoke("fp8_cast_amax", _ptr(x), x.numel(), _ptr(scale), int(fmt), _ptr(out), _ptr(scale_inv_out),
                               _ptr(amax_slot), _ptr(noop), _stream(stream))


def fp8_cast_transpose(x, scale, fmt, out, out_t, scale_inv_out=None, amax_slot=None, noop=None, stream=None):
    """Cast a 2-D bfloat16 ``x`` [R, C] to ``out`` [R, C] and its transpose ``out_t`` [C, R]."""
    _want(x, _BF16, "x", required=True)
    R, C = x.shape
    _want(out, _U8, "out", shape=(R, C), required=True)
    _want(out_t, _U8, "out_t", shape=(C, R), required=True)
    _scalars(scale=scale, scale_inv_out=scale_inv_out, amax_slot=amax_slot, noop=noop)
    _invoke("fp8_cast_transpose", _ptr(x), R, C, _ptr(scale), int(fmt), _ptr(out), _ptr(out_t),
                                    _ptr(scale_inv_out), _ptr(amax_slot), _ptr(noop), _stream(stream))


def fp8_dbias_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().fp8_dbias_workspace_bytes(int(rows), int(cols)))


def fp8_dbias_cast_transpose(dy, scale, fmt, out, out_t, dbias, workspace, scale_inv_out=None, amax_slot=None,
                             stream=None):
    """dbias = column sums of ``dy`` plus its cast+transpose (see include/fp8ds.h).

    ``workspace``: at least ``fp8_dbias_workspace_bytes(rows, cols)`` bytes, zero-filled before
    its first use (``torch.zeros``); every call leaves its counter bytes zero again."""
    _want(dy, _BF16, "dy", required=True)
    R, C = dy.shape
    _want(dbias, _F32, "dbias", shape=(C,), required=True)
    _want(out, _U8, "out", shape=(R, C))
    _want(out_t, _U8, "out_t", shape=(C, R))
    ws_bytes = _workspace_bytes(workspace)
    _scalars(scale=scale, scale_inv_out=scale_inv_out, amax_slot=amax_slot)
    _invoke("fp8_dbias_cast_transpose", _ptr(dy), R, C, _ptr(scale), int(fmt), _ptr(out), _ptr(out_t),
                                          _ptr(scale_inv_out), _ptr(amax_slot), _ptr(dbias), _ptr(workspace),
                                          ws_bytes, _stream(stream))


def fp8_dbias_cast_transpose_noalloc(dy, scale, fmt, out, out_t, dbias, scale_inv_out=None, amax_slot=None,
                                     stream=None):
    """fp8_dbias_cast_transpose without a workspace: the partial sums go to the library's static
    per-GPU scratch (no allocation; calls overlapping on one GPU race; see include/fp8ds.h)."""
    _want(dy, _BF16, "dy", required=True)
    R, C = dy.shape
    _want(dbias, _F32, "dbias", shape=(C,), required=True)
    _want(out, _U8, "out", shape=(R, C))
    _want(out_t, _U8, "out_t", shape=(C, R))
    _scalars(scale=scale, scale_inv_out=scale_inv_out, amax_slot=amax_slot)
    _invoke("fp8_dbias_cast_transpose_noalloc", _ptr(dy), R, C, _ptr(scale), int(fmt), _ptr(out), _ptr(out_t),
                                                  _ptr(scale_inv_out), _ptr(amax_slot), _ptr(dbias),
                                                  _stream(stream))


def fp8_scale_update(amax_history, scale, scale_inv, fmts: Sequence[int], margin: int = 0, stream=None):
    """One delayed-scaling step for the T tensors of ``amax_history`` [L, T]."""
    _want(amax_history, _F32, "amax_history", required=True)
    L, T = amax_history.shape
    _want(scale, _F32, "scale", min_numel=T, required=True)
    _want(scale_inv, _F32, "scale_inv", min_numel=T, required=True)
    if len(fmts) != T:
        raise ValueError("one format per tensor")
    f = (ctypes.c_int32 * T)(*[int(v) for v in fmts])
    _invoke("fp8_scale_update", _ptr(amax_history), L, T, _ptr(scale), _ptr(scale_inv),
                                  ctypes.cast(f, ctypes.c_void_p), int(margin), _stream(stream))


def _out_dtype(D):
    if D.dtype == torch.bfloat16:
        return OUT_BF16
    if D.dtype == torch.float32:
        return OUT_FP32
    raise TypeError("D must be bfloat16 or float32")


def _gemm_args(A, fa, a_scale_inv, B, fb, b_scale_inv, bias, D):
    _want(A, _U8, "A", contiguous=False, required=True)
    _want(B, _U8, "B", contiguous=False, required=True)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("A and B must share K")
    _want(bias, _BF16, "bias", shape=(N,))
    if tuple(D.shape) != (M, N):
        raise ValueError("D must be [M, N]")
    for t, nm in ((A, "A"), (B, "B"), (D, "D")):
        if t.numel() and t.stride(1) != 1:
            raise ValueError(f"{nm} rows must be contiguous")
    _scalars(a_scale_inv=a_scale_inv, b_scale_inv=b_scale_inv)
    return (_ptr(A), int(fa), _ptr(a_scale_inv), A.stride(0), _ptr(B), int(fb), _ptr(b_scale_inv), B.stride(0),
            _ptr(bias), _ptr(D), D.stride(0), _out_dtype(D), M, N, K)


def fp8_gemm_bias(A, fa, a_scale_inv, B, fb, b_scale_inv, bias, D, stream=None):
    """D = (A B^T) * a_scale_inv * b_scale_inv + bias, A [M, K] and B [N, K] FP8 codes."""
    _invoke("fp8_gemm_bias", *_gemm_args(A, fa, a_scale_inv, B, fb, b_scale_inv, bias, D), _stream(stream))


def fp8_gemm_bias_fp8(A, fa, a_scale_inv, B, fb, b_scale_inv, bias, D, d_fmt, d_scale, d_scale_inv_out=None,
                      d_amax_slot=None, stream=None):
    """FP8-output GEMM: D = codes of ((A B^T) * a_scale_inv * b_scale_inv + bias) * d_scale, with the
    output's amax folded into ``d_amax_slot`` and 1/d_scale written to ``d_scale_inv_out``."""
    _want(D, _U8, "D", contiguous=False, required=True)
    _want(A, _U8, "A", contiguous=False, required=True)
    _want(B, _U8, "B", contiguous=False, required=True)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("A and B must share K")
    _want(bias, _BF16, "bias", shape=(N,))
    _scalars(a_scale_inv=a_scale_inv, b_scale_inv=b_scale_inv, d_scale=d_scale, d_scale_inv_out=d_scale_inv_out,
             d_amax_slot=d_amax_slot)
    if tuple(D.shape) != (M, N):
        raise ValueError("D must be [M, N]")
    for t, nm in ((A, "A"), (B, "B"), (D, "D")):
        if t.numel() and t.stride(1) != 1:
            raise ValueError(f"{nm} rows must be contiguous")
    _invoke("fp8_gemm_bias_fp8", _ptr(A), int(fa), _ptr(a_scale_inv), A.stride(0), _ptr(B), int(fb),
                                   _ptr(b_scale_inv), B.stride(0), _ptr(bias), _ptr(D), D.stride(0), int(d_fmt),
                                   _ptr(d_scale), _ptr(d_scale_inv_out), _ptr(d_amax_slot), M, N, K,
                                   _stream(stream))


def fp8_transpose(x8, out_t, noop=None, stream=None):
    """Transpose cache of an existing FP8 tensor: out_t [C, R] = x8 [R, C]^T (codes copied)."""
    _want(x8, _U8, "x8", required=True)
    R, C = x8.shape
    _want(out_t, _U8, "out_t", shape=(C, R), required=True)
    _scalars(noop=noop)
    _invoke("fp8_transpose", _ptr(x8), R, C, _ptr(out_t), _ptr(noop), _stream(stream))


def fp8_gemm_bias_chunked(A, fa, a_scale_inv, B, fb, b_scale_inv, bias, D, n_chunks: int,
                          chunk_streams=None, stream=None):
    """The N-chunked GEMM: chunk c on ``chunk_streams[c]`` with its own bias offset."""
    arr = None
    if chunk_streams is not None:
        if len(chunk_streams) < n_chunks:
            raise ValueError("one stream per chunk")
        arr = (ctypes.c_void_p * n_chunks)(*[_stream(s) for s in chunk_streams[:n_chunks]])
    _invoke("fp8_gemm_bias_chunked", *_gemm_args(A, fa, a_scale_inv, B, fb, b_scale_inv, bias, D),
                                       int(n_chunks), None if arr is None else ctypes.cast(arr, ctypes.c_void_p),
                                       _stream(stream))


def fp8_linear_fwd(x, w, bias, x_scale, x_amax, x8, x8_t, x_scale_inv, w_scale, w_amax, w8, w8_t, w_scale_inv,
                   w_noop, y, stream=None):
    """Forward of the FP8 linear layer: casts of x and W, then y = x8 W8^T + bias."""
    _want(x, _BF16, "x", required=True)
    _want(w, _BF16, "w", required=True)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("x [M, K] and w [N, K] must share K")
    _want(y, (torch.bfloat16,), "y", shape=(M, N), required=True)
    _want(bias, _BF16, "bias", shape=(N,))
    _want(x8, _U8, "x8", shape=(M, K), required=True)
    _want(x8_t, _U8, "x8_t", shape=(K, M))
    _want(w8, _U8, "w8", shape=(N, K), required=True)
    _want(w8_t, _U8, "w8_t", shape=(K, N), required=True)
    _scalars(x_scale=x_scale, x_amax=x_amax, x_scale_inv=x_scale_inv, w_scale=w_scale, w_amax=w_amax,
             w_scale_inv=w_scale_inv, w_noop=w_noop)
    _invoke("fp8_linear_fwd", _ptr(x), _ptr(w), _ptr(bias), M, N, K, _ptr(x_scale), _ptr(x_amax), _ptr(x8),
                                _ptr(x8_t), _ptr(x_scale_inv), _ptr(w_scale), _ptr(w_amax), _ptr(w8), _ptr(w8_t),
                                _ptr(w_scale_inv), _ptr(w_noop), _ptr(y), _stream(stream))


def fp8_linear_bwd(dy, K, dy_scale, dy_amax, dy8, dy8_t, dy_scale_inv, dbias, workspace, x8_t, x_scale_inv, w8_t,
                   w_scale_inv, dx, dw, stream=None):
    """Backward of the FP8 linear layer: dbias + cast+transpose of dy, dgrad and wgrad GEMMs.

    ``workspace`` (with ``dbias``): zero-filled before its first use, as for
    ``fp8_dbias_cast_transpose``."""
    _want(dy, _BF16, "dy", required=True)
    M, N = dy.shape
    K = int(K)
    _want(dy8, _U8, "dy8", shape=(M, N), required=True)
    _want(dy8_t, _U8, "dy8_t", shape=(N, M), required=True)
    _want(dbias, _F32, "dbias", shape=(N,))
    _want(x8_t, _U8, "x8_t", shape=(K, M), required=True)
    _want(w8_t, _U8, "w8_t", shape=(K, N), required=True)
    _want(dx, (torch.bfloat16,), "dx", shape=(M, K), required=True)
    _want(dw, (torch.bfloat16, torch.float32), "dw", shape=(N, K), required=True)
    ws_bytes = _workspace_bytes(workspace)
    _scalars(dy_scale=dy_scale, dy_amax=dy_amax, dy_scale_inv=dy_scale_inv, x_scale_inv=x_scale_inv,
             w_scale_inv=w_scale_inv)
    _invoke("fp8_linear_bwd", _ptr(dy), M, N, int(K), _ptr(dy_scale), _ptr(dy_amax), _ptr(dy8), _ptr(dy8_t),
                                _ptr(dy_scale_inv), _ptr(dbias), _ptr(workspace), ws_bytes, _ptr(x8_t),
                                _ptr(x_scale_inv), _ptr(w8_t), _ptr(w_scale_inv), _ptr(dx), _ptr(dw),
                                _out_dtype(dw), _stream(stream))
