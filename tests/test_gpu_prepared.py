"""Prepared calls (fp8_delayed_scaling_amd.prepare): the binding's checks and marshalling run
once, then each call repeats only the C call.  A prepared call must give exactly what the plain
binding call gives, on the stream it was prepared for or on another one: the small-layer
forward (one launch), a scale update (its formats array kept alive by the prepared call), an
N-chunked GEMM (its stream array likewise), and the backward."""
import pytest
import torch

import fp8_delayed_scaling_amd as F
import synthetic as S
from helpers import DEV, bf16_dev

pytestmark = pytest.mark.gpu

U8 = dict(device=DEV, dtype=torch.uint8)
F32 = dict(device=DEV, dtype=torch.float32)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.uint8)


def test_prepared_forward_equals_the_binding_call():
    M, N, K = 128, 256, 256
    print(f"prepared forward {M}x{N}x{K}", flush=True)
    x = bf16_dev(S.normal_bf16(S.seed_for(11, 0), (M, K), 1.0))
    w = bf16_dev(S.normal_bf16(S.seed_for(11, 1), (N, K), 1.0))
    b = bf16_dev(S.normal_bf16(S.seed_for(11, 2), (N,), 0.1))
    sc = torch.tensor([2.0, 16.0], **F32)
    am, si = torch.zeros(2, **F32), torch.zeros(2, **F32)
    x8, w8, w8t = torch.empty((M, K), **U8), torch.empty((N, K), **U8), torch.empty((K, N), **U8)
    y = torch.empty((M, N), device=DEV, dtype=torch.bfloat16)
    args = (x, w, b, sc[0:1], am[0:1], x8, None, si[0:1], sc[1:2], am[1:2], w8, w8t, si[1:2], None, y)
    F.fp8_linear_fwd(*args)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (x8, w8, w8t, am, si, y)]
    p = F.prepare(F.fp8_linear_fwd, *args)
    assert p.name == "fp8_linear_fwd"
    side = torch.cuda.Stream()
    for stream in (None, None, side):
        for t in (x8, w8, w8t, y):
            t.zero_()
        am.zero_()
        si.fill_(-1.0)
        torch.cuda.synchronize()
        p(stream=stream)
        torch.cuda.synchronize()
        for got, want in zip((x8, w8, w8t, am, si, y), ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else _bits(got),
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else _bits(want))


def test_prepared_scale_update_keeps_its_formats():
    L, T = 16, 3
    print("prepared scale update", flush=True)
    hist0 = torch.rand((L, T), generator=torch.Generator().manual_seed(5)).to(DEV) * 100
    fmts = [F.E4M3, F.E4M3, F.E5M2]
    h1, s1, si1 = hist0.clone(), torch.ones(T, **F32), torch.ones(T, **F32)
    F.fp8_scale_update(h1, s1, si1, fmts, 0)
    h2, s2, si2 = hist0.clone(), torch.ones(T, **F32), torch.ones(T, **F32)
    p = F.prepare(F.fp8_scale_update, h2, s2, si2, list(fmts), 0)
    import gc
    gc.collect()   # the formats array lives on in the prepared call, not in this frame
    p()
    torch.cuda.synchronize()
    for a, b_ in ((h1, h2), (s1, s2), (si1, si2)):
        assert torch.equal(_bits(a), _bits(b_))


def test_prepared_chunked_gemm_keeps_its_streams():
    M, N, K = 512, 1024, 512
    print(f"prepared chunked GEMM {M}x{N}x{K}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(7)
    A = torch.randint(0, 256, (M, K), generator=g, device=DEV, dtype=torch.uint8) & 0x77
    B = torch.randint(0, 256, (N, K), generator=g, device=DEV, dtype=torch.uint8) & 0x77
    one = torch.ones(1, **F32)
    bias = bf16_dev(S.normal_bf16(S.seed_for(11, 3), (N,), 0.1))
    D1 = torch.empty((M, N), device=DEV, dtype=torch.bfloat16)
    D2 = torch.full((M, N), float("nan"), device=DEV, dtype=torch.bfloat16)
    F.fp8_gemm_bias(A, F.E4M3, one, B, F.E4M3, one, bias, D1)
    streams = [torch.cuda.Stream() for _ in range(4)]
    p = F.prepare(F.fp8_gemm_bias_chunked, A, F.E4M3, one, B, F.E4M3, one, bias, D2, 4, streams)
    import gc
    gc.collect()
    p()
    torch.cuda.synchronize()
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))


def test_prepared_backward_equals_the_binding_call():
    M, N, K = 256, 512, 256
    print(f"prepared backward {M}x{N}x{K}", flush=True)
    dy = bf16_dev(S.normal_bf16(S.seed_for(11, 4), (M, N), 0.01))
    g = torch.Generator(device=DEV).manual_seed(9)
    x8t = torch.randint(0, 256, (K, M), generator=g, device=DEV, dtype=torch.uint8) & 0x77
    w8t = torch.randint(0, 256, (K, N), generator=g, device=DEV, dtype=torch.uint8) & 0x77
    one = torch.ones(1, **F32)

    def outs():
        return dict(dy_amax=torch.zeros(1, **F32), dy8=torch.empty((M, N), **U8), dy8_t=torch.empty((N, M), **U8),
                    dy_scale_inv=torch.zeros(1, **F32), dbias=torch.empty(N, **F32),
                    workspace=torch.zeros(F.fp8_dbias_workspace_bytes(M, N), **U8),
                    dx=torch.empty((M, K), device=DEV, dtype=torch.bfloat16), dw=torch.empty((N, K), **F32))

    o1, o2 = outs(), outs()
    kw = dict(K=K, dy_scale=torch.full((1,), 1024.0, **F32), x8_t=x8t, x_scale_inv=one, w8_t=w8t, w_scale_inv=one)
    F.fp8_linear_bwd(dy, **kw, **o1)
    p = F.prepare(F.fp8_linear_bwd, dy, **kw, **o2)
    p()
    p()   # twice: the workspace counters are left zero, the amax slot keeps its maximum
    torch.cuda.synchronize()
    for k in o1:
        if k == "workspace":
            continue
        a, b_ = o1[k], o2[k]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else _bits(a),
                           b_.view(torch.int16) if b_.dtype == torch.bfloat16 else _bits(b_)), k
