"""The Python binding rejects mis-sized buffers before it takes a single pointer.

The C ABI receives bare pointers and cannot see sizes, so a too-small or mis-shaped buffer
would become an out-of-bounds device write.  Each case below passes host tensors in which
exactly one argument is wrong: the binding must raise a ValueError or TypeError naming that
argument (a well-formed host-tensor call would only fail later, at the device-pointer step,
with a different message).  CPU only: nothing is launched."""
import pytest
import torch

import fp8_delayed_scaling_amd as F

u8 = dict(dtype=torch.uint8)
f32 = dict(dtype=torch.float32)
bf = dict(dtype=torch.bfloat16)


def _raises(name, fn, *a, **kw):
    with pytest.raises((ValueError, TypeError), match=name):
        fn(*a, **kw)


def _good_scalar():
    return torch.ones(1, **f32)


def test_cast_checks():
    x = torch.zeros((8, 16), **bf)
    s = _good_scalar()
    _raises("out", F.fp8_cast_amax, x, s, F.E4M3, torch.empty(100, **u8))
    _raises("scale", F.fp8_cast_amax, x, torch.ones(1, dtype=torch.float64), F.E4M3, torch.empty(128, **u8))
    _raises("amax_slot", F.fp8_cast_amax, x, s, F.E4M3, torch.empty(128, **u8), amax_slot=torch.empty(0, **f32))
    _raises("out_t", F.fp8_cast_transpose, x, s, F.E4M3, torch.empty((8, 16), **u8), torch.empty((8, 16), **u8))
    _raises("out", F.fp8_cast_transpose, x, s, F.E4M3, torch.empty((8, 15), **u8), torch.empty((16, 8), **u8))
    _raises("noop", F.fp8_cast_transpose, x, s, F.E4M3, torch.empty((8, 16), **u8), torch.empty((16, 8), **u8),
            noop=torch.zeros(1, dtype=torch.int32))
    _raises("out_t", F.fp8_transpose, torch.empty((8, 16), **u8), torch.empty((8, 16), **u8))


def test_dbias_checks():
    dy = torch.zeros((32, 16), **bf)
    s = _good_scalar()
    out, out_t = torch.empty((32, 16), **u8), torch.empty((16, 32), **u8)
    ws = torch.empty(4096, **u8)
    _raises("dbias", F.fp8_dbias_cast_transpose, dy, s, F.E5M2, out, out_t, torch.empty(8, **f32), ws)
    _raises("dbias", F.fp8_dbias_cast_transpose, dy, s, F.E5M2, out, out_t, torch.empty(16, dtype=torch.float16), ws)
    _raises("out_t", F.fp8_dbias_cast_transpose, dy, s, F.E5M2, out, torch.empty((32, 16), **u8),
            torch.empty(16, **f32), ws)
    _raises("workspace", F.fp8_dbias_cast_transpose, dy, s, F.E5M2, out, out_t, torch.empty(16, **f32),
            torch.empty((64, 128), **u8)[:, ::2])


def test_scale_update_checks():
    h = torch.zeros((4, 3), **f32)
    _raises("scale", F.fp8_scale_update, h, torch.ones(1, **f32), torch.ones(3, **f32), [0, 0, 1])
    _raises("scale_inv", F.fp8_scale_update, h, torch.ones(3, **f32), torch.ones(2, **f32), [0, 0, 1])
    _raises("one format", F.fp8_scale_update, h, torch.ones(3, **f32), torch.ones(3, **f32), [0, 1])
    _raises("amax_history", F.fp8_scale_update, h.t(), torch.ones(4, **f32), torch.ones(4, **f32), [0] * 4)


def test_gemm_checks():
    A, B = torch.empty((32, 64), **u8), torch.empty((48, 64), **u8)
    s = _good_scalar()
    D = torch.empty((32, 48), **bf)
    _raises("bias", F.fp8_gemm_bias, A, F.E4M3, s, B, F.E4M3, s, torch.zeros(16, **bf), D)
    _raises("D", F.fp8_gemm_bias, A, F.E4M3, s, B, F.E4M3, s, None, torch.empty((32, 47), **bf))
    _raises("b_scale_inv", F.fp8_gemm_bias, A, F.E4M3, s, B, F.E4M3, torch.empty(0, **f32), None, D)
    _raises("share K", F.fp8_gemm_bias, A, F.E4M3, s, torch.empty((48, 32), **u8), F.E4M3, s, None, D)
    _raises("d_amax_slot", F.fp8_gemm_bias_fp8, A, F.E4M3, s, B, F.E4M3, s, None, torch.empty((32, 48), **u8),
            F.E4M3, s, d_amax_slot=torch.empty(0, **f32))


def _fwd_args(M=32, N=48, K=64):
    s = _good_scalar
    return dict(x=torch.zeros((M, K), **bf), w=torch.zeros((N, K), **bf), bias=torch.zeros(N, **bf),
                x_scale=s(), x_amax=s(), x8=torch.empty((M, K), **u8), x8_t=torch.empty((K, M), **u8),
                x_scale_inv=s(), w_scale=s(), w_amax=s(), w8=torch.empty((N, K), **u8),
                w8_t=torch.empty((K, N), **u8), w_scale_inv=s(), w_noop=None, y=torch.empty((M, N), **bf))


@pytest.mark.parametrize("name,bad", [
    ("x8", torch.empty((32, 63), **u8)),
    ("x8_t", torch.empty((32, 64), **u8)),
    ("w8", torch.empty((47, 64), **u8)),
    ("w8_t", torch.empty((48, 64), **u8)),
    ("y", torch.empty((32, 47), **bf)),
    ("bias", torch.empty(47, **bf)),
    ("x_scale", torch.empty(0, **f32)),
    ("w_scale_inv", torch.empty(0, **f32)),
])
def test_linear_fwd_checks(name, bad):
    a = _fwd_args()
    a[name] = bad
    _raises(name, F.fp8_linear_fwd, **a)


def _bwd_args(M=32, N=48, K=64):
    s = _good_scalar
    return dict(dy=torch.zeros((M, N), **bf), K=K, dy_scale=s(), dy_amax=s(), dy8=torch.empty((M, N), **u8),
                dy8_t=torch.empty((N, M), **u8), dy_scale_inv=s(), dbias=torch.empty(N, **f32),
                workspace=torch.empty(1 << 16, **u8), x8_t=torch.empty((K, M), **u8), x_scale_inv=s(),
                w8_t=torch.empty((K, N), **u8), w_scale_inv=s(), dx=torch.empty((M, K), **bf),
                dw=torch.empty((N, K), **f32))


@pytest.mark.parametrize("name,bad", [
    ("dy8", torch.empty((32, 47), **u8)),
    ("dy8_t", torch.empty((32, 48), **u8)),
    ("dbias", torch.empty(47, **f32)),
    ("x8_t", torch.empty((63, 32), **u8)),
    ("w8_t", torch.empty((64, 47), **u8)),
    ("dx", torch.empty((32, 63), **bf)),
    ("dw", torch.empty((48, 63), **f32)),
    ("dw", torch.empty((48, 64), dtype=torch.float16)),
    ("dy_scale_inv", torch.empty(0, **f32)),
    ("workspace", torch.empty((256, 512), **u8)[:, ::2]),
])
def test_linear_bwd_checks(name, bad):
    a = _bwd_args()
    a[name] = bad
    _raises(name, F.fp8_linear_bwd, **a)


def test_well_formed_host_call_fails_only_at_the_pointer_step():
    """The same calls with every buffer right get past the checks and stop at the device
    pointer (host tensors are refused there), so the cases above fail for their one bad argument."""
    with pytest.raises(ValueError, match="must live on the GPU"):
        F.fp8_linear_fwd(**_fwd_args())
    with pytest.raises(ValueError, match="must live on the GPU"):
        F.fp8_linear_bwd(**_bwd_args())


def test_prepare_needs_one_library_call():
    """prepare() records exactly one C call; a function that makes none is refused, and a failed
    check inside it leaves the binding in its normal (calling) state."""
    with pytest.raises(ValueError, match="not a single library call"):
        F.prepare(lambda: None)
    with pytest.raises((ValueError, TypeError), match="out_t"):
        F.prepare(F.fp8_transpose, torch.empty((8, 16), **u8), torch.empty((8, 16), **u8))
    assert getattr(F._tls, "rec", None) is None
