"""The C ABI on the CPU: the library loads, exports every function include/fp8ds.h declares,
and rejects bad arguments on the host (before any HIP call, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import fp8_delayed_scaling_amd as F

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fp8ds.h")


def _declared():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fp8\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_hot_path():
    names = _declared()
    for n in ("fp8_cast_amax", "fp8_cast_transpose", "fp8_dbias_cast_transpose", "fp8_dbias_workspace_bytes",
              "fp8_scale_update", "fp8_gemm_bias", "fp8_gemm_bias_chunked", "fp8_gemm_bias_fp8", "fp8_transpose",
              "fp8_linear_fwd", "fp8_linear_bwd", "fp8ds_status_string", "fp8ds_version",
              "fp8_dbias_cast_transpose_noalloc"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = F.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert F.fp8ds_version() >= 100


def test_status_strings():
    for code in range(0, -9, -1):
        s = F.fp8ds_status_string(code)
        assert s.startswith("FP8DS")
    assert "unknown" in F.fp8ds_status_string(-99)


A16 = 1 << 20        # a fake 16-byte aligned address: never dereferenced, validation fails first


def test_cast_validation():
    L = F.lib()
    assert L.fp8_cast_amax(None, 10, A16, 0, A16, None, None, None, None) == -1     # NULL x
    assert L.fp8_cast_amax(A16, -1, A16, 0, A16, None, None, None, None) == -2      # negative size
    assert L.fp8_cast_amax(A16, 10, A16, 5, A16, None, None, None, None) == -4      # bad format
    assert L.fp8_cast_amax(A16 + 2, 10, A16, 0, A16, None, None, None, None) == -3  # misaligned x
    assert L.fp8_cast_amax(None, 0, None, 0, None, None, None, None, None) == 0     # empty: nothing
    assert L.fp8_cast_transpose(A16, 4, 4, A16, 0, A16, None, None, None, None, None) == -1   # NULL out_t
    assert L.fp8_cast_transpose(A16, 4, -4, A16, 0, A16, A16, None, None, None, None) == -2
    assert L.fp8_cast_transpose(A16, 4, 4, A16, 0, A16, A16 + 8, None, None, None, None) == -3
    # 2^40 elements in one row: 2^32 tiles of 256 x 256, more than a launch numbers
    assert L.fp8_cast_transpose(A16, 1, 1 << 40, A16, 0, A16, A16, None, None, None, None) == -2
    assert L.fp8_dbias_cast_transpose(A16, 1, 1 << 40, A16, 1, A16, A16, None, None, A16, A16, 1 << 50, None) == -2


def test_dbias_validation():
    L = F.lib()
    need = F.fp8_dbias_workspace_bytes(300, 100)
    assert need == 1024 + 2 * 100 * 4       # strip counters, then one float per (256-row block, column)
    assert F.fp8_dbias_workspace_bytes(0, 100) == 0
    assert L.fp8_dbias_cast_transpose(A16, 300, 100, A16, 1, A16, A16, None, None, A16, None, 0, None) == -5
    assert L.fp8_dbias_cast_transpose(A16, 300, 100, A16, 1, A16, A16, None, None, A16, A16, need - 4, None) == -5
    assert L.fp8_dbias_cast_transpose(A16, 300, 100, A16, 1, A16, A16, None, None, None, A16, need, None) == -1


def test_dbias_noalloc_rejects_sizes_beyond_its_scratch():
    L = F.lib()
    f = L.fp8_dbias_cast_transpose_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    # 32 row blocks x 80000 columns x 4 bytes = 10.24 MB of partials > 8 MiB: rejected, nothing launched
    assert F.fp8_dbias_workspace_bytes(8192, 80000) > 8 << 20
    # the limit: 1 KiB of strip counters + 32 x cols x 4 bytes <= 8 MiB, so 8192 rows fit up to 65528 columns
    assert F.fp8_dbias_workspace_bytes(8192, 65528) == 8 << 20
    assert F.fp8_dbias_workspace_bytes(8192, 65536) > 8 << 20
    assert f(A16, 8192, 65536, A16, 1, A16, A16, None, None, A16, None) == -8
    assert f(A16, 8192, 80000, A16, 1, A16, A16, None, None, A16, None) == -8
    assert f(A16, -1, 100, A16, 1, A16, A16, None, None, A16, None) == -2


def test_scale_update_validation():
    L = F.lib()
    fm = (ctypes.c_int32 * 3)(0, 0, 1)
    bad = (ctypes.c_int32 * 3)(0, 2, 1)
    p = ctypes.cast(fm, ctypes.c_void_p)
    assert L.fp8_scale_update(A16, 0, 3, A16, A16, p, 0, None) == -2          # L < 1
    assert L.fp8_scale_update(A16, 4, 4097, A16, A16, p, 0, None) == -2       # T > 4096
    assert L.fp8_scale_update(A16, 4, 3, A16, A16, p, 127, None) == -7        # margin range
    assert L.fp8_scale_update(A16, 4, 3, None, A16, p, 0, None) == -1
    assert L.fp8_scale_update(A16, 4, 3, A16, A16, ctypes.cast(bad, ctypes.c_void_p), 0, None) == -4


def test_gemm_validation():
    L = F.lib()
    g = L.fp8_gemm_bias
    ok = dict(A=A16, fa=0, sa=A16, lda=64, B=A16, fb=1, sb=A16, ldb=64, bias=None, D=A16, ldd=64, dt=0,
              M=32, N=64, K=64)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["A"], a["fa"], a["sa"], a["lda"], a["B"], a["fb"], a["sb"], a["ldb"], a["bias"], a["D"], a["ldd"],
                 a["dt"], a["M"], a["N"], a["K"], None)

    assert call(K=40) == -2                 # K % 16
    assert call(lda=32) == -2               # lda < K
    assert call(ldd=60) == -2               # ldd < N
    assert call(D=A16 + 1) == -3            # D not aligned to its element size
    assert call(A=None) == -1
    assert call(D=None) == -1
    assert call(fa=3) == -4
    assert call(dt=2) == -4
    assert call(B=A16 + 4) == -3
    assert call(M=-1) == -2
    assert call(M=0) == 0                   # empty output: nothing launched
    assert L.fp8_gemm_bias_chunked(A16, 0, A16, 64, A16, 0, A16, 64, None, A16, 64, 0, 32, 64, 64, 0, None,
                                   None) == -7   # n_chunks out of range
    assert L.fp8_gemm_bias_chunked(A16, 0, A16, 64, A16, 0, A16, 64, None, A16, 64, 0, 32, 64, 64, 17, None,
                                   None) == -7


def test_linear_validation():
    L = F.lib()
    # K not a multiple of 16
    assert L.fp8_linear_fwd(A16, A16, None, 16, 16, 24, A16, None, A16, None, A16, A16, None, A16, A16, A16, None,
                            A16, None) == -2
    # backward needs M and N multiples of 16
    assert L.fp8_linear_bwd(A16, 24, 16, 16, A16, None, A16, A16, A16, None, None, 0, A16, A16, A16, A16, A16,
                            A16, 0, None) == -2


def test_gemm_fp8_out_validation():
    L = F.lib()
    g = L.fp8_gemm_bias_fp8
    ok = dict(A=A16, fa=0, sa=A16, lda=64, B=A16, fb=0, sb=A16, ldb=64, bias=None, D=A16, ldd=32, d_fmt=0,
              ds=A16, dsinv=None, damax=None, M=16, N=32, K=64)

    def call(**kw):
        a = dict(ok, **kw)
        return g(a["A"], a["fa"], a["sa"], a["lda"], a["B"], a["fb"], a["sb"], a["ldb"], a["bias"], a["D"], a["ldd"],
                 a["d_fmt"], a["ds"], a["dsinv"], a["damax"], a["M"], a["N"], a["K"], None)

    assert call(d_fmt=2) == -4                 # unknown output format
    assert call(fa=3) == -4
    assert call(ds=None) == -1                 # the output scale is required
    assert call(ds=A16 + 2) == -3
    assert call(damax=A16 + 1) == -3
    assert call(D=None) == -1
    assert call(K=40) == -2                    # K % 16
    assert call(ldd=31) == -2                  # ldd < N
    assert call(lda=48) == -2                  # lda < K
    assert call(A=A16 + 8) == -3
    assert call(M=0) == 0                      # empty output, no inverse scale asked: nothing launched


def test_fp8_out_dtype_codes_stay_private():
    """The plain GEMM accepts only the two public output dtypes."""
    L = F.lib()
    args = [A16, 0, A16, 64, A16, 0, A16, 64, None, A16, 32]
    assert L.fp8_gemm_bias(*args, 2, 16, 32, 64, None) == -4
    assert L.fp8_gemm_bias(*args, 3, 16, 32, 64, None) == -4
    assert L.fp8_gemm_bias_chunked(*args, 2, 16, 32, 64, 2, None, None) == -4


def test_transpose_validation():
    L = F.lib()
    assert L.fp8_transpose(None, 4, 4, A16, None, None) == -1
    assert L.fp8_transpose(A16, 4, 4, None, None, None) == -1
    assert L.fp8_transpose(A16, -1, 4, A16, None, None) == -2
    assert L.fp8_transpose(A16, 4, 4, A16, A16 + 2, None) == -3      # misaligned noop flag
    assert L.fp8_transpose(None, 0, 4, None, None, None) == 0         # empty: nothing
    assert L.fp8_transpose(A16, 1, 1 << 40, A16, None, None) == -2    # too many tiles
