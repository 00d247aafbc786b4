"""GPU parity of the FP8 -> FP8 transpose (lazy transpose-cache fill) against the oracle: every
byte value, vector and byte-by-byte paths, ragged tiles, the full-size weight, the noop flag,
and replays of a captured graph with the flag flipped between them."""
import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, bf16_dev, scalar, u8_host

pytestmark = pytest.mark.gpu


def _bytes(seed, shape):
    """Seeded bytes covering all 256 codes (the transpose never looks at their values)."""
    return S.random_bytes(seed, shape)


def _run(xh, noop=None, prefill=0x5A):
    x = torch.from_numpy(xh).to(DEV)
    R, C = xh.shape
    out = torch.full((C, R), prefill, dtype=torch.uint8, device=DEV)
    F.fp8_transpose(x, out, noop=noop)
    torch.cuda.synchronize()
    return u8_host(out)


# (512, 4096), (1024, 256) and (2048, 768) are whole 512 x 256 tiles (the 512-row kernel)
@pytest.mark.parametrize("shape", [(16, 16), (256, 256), (272, 528), (512, 4096), (4112, 48), (1024, 256), (2048, 768),
                                   (1, 1), (17, 33), (300, 257), (1, 4000), (5000, 1), (255, 16), (768, 256)])
def test_transpose_parity(shape):
    print(f"fp8_transpose {shape}", flush=True)
    xh = _bytes(S.seed_for(30, shape[0] % 16), shape)
    assert np.array_equal(_run(xh), oracle.fp8_transpose(xh))


@pytest.mark.parametrize("shape", [(18432, 12288), (8192, 18432), (8192, 12288)])
def test_transpose_full_size(shape):
    """The weight of the QKV projection at one TP=2 rank's share, its dy and its x: the shapes
    whose transpose cache the backward needs."""
    print(f"fp8_transpose full {shape}", flush=True)
    xh = _bytes(S.seed_for(31, 0), shape)
    assert np.array_equal(_run(xh), oracle.fp8_transpose(xh))


def test_transpose_unaligned_buffers_take_the_byte_path():
    R, C = 96, 80
    xh = _bytes(S.seed_for(32, 0), (R, C))
    buf = torch.zeros(R * C + 1, dtype=torch.uint8, device=DEV)
    x = buf[1:].view(R, C)
    x.copy_(torch.from_numpy(xh).to(DEV))
    obuf = torch.full((C * R + 3,), 0x11, dtype=torch.uint8, device=DEV)
    out = obuf[3:].view(C, R)
    F.fp8_transpose(x, out)
    torch.cuda.synchronize()
    assert np.array_equal(u8_host(out), oracle.fp8_transpose(xh))
    assert np.all(u8_host(obuf[:3]) == 0x11)


def test_transpose_empty_is_a_no_op():
    out = torch.full((5, 0), 7, dtype=torch.uint8, device=DEV)
    F.fp8_transpose(torch.empty((0, 5), dtype=torch.uint8, device=DEV), out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [(272, 528), (512, 256)])
def test_transpose_noop_flag(shape):
    R, C = shape
    xh = _bytes(S.seed_for(33, 0), (R, C))
    stale = np.full((C, R), 0x5A, np.uint8)
    assert np.array_equal(_run(xh, noop=scalar(1.0)), oracle.fp8_transpose(xh, noop=True, out_t_prev=stale))
    assert np.array_equal(_run(xh, noop=scalar(0.0)), oracle.fp8_transpose(xh))
    assert np.array_equal(_run(xh, noop=scalar(0.5)), oracle.fp8_transpose(xh))   # only exactly 1.0 skips


def test_lazy_transpose_equals_cast_transpose():
    """Cast without the transpose, then fill the cache from the FP8 tensor: the same bytes as
    the fused cast+transpose (a transpose of codes, no re-encoding)."""
    R, C = 384, 272
    xh = S.normal_bf16(S.seed_for(34, 0), (R, C), 1.0)
    x = bf16_dev(xh)
    q = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    qt = torch.empty((C, R), dtype=torch.uint8, device=DEV)
    F.fp8_cast_amax(x, scalar(3.0), F.E4M3, q)
    F.fp8_transpose(q, qt)
    torch.cuda.synchronize()
    _, rqt, _, _ = oracle.cast_transpose(xh, 3.0, F.E4M3)
    assert np.array_equal(u8_host(qt), rqt)


def test_transpose_graph_replay_with_flag_flips():
    """The transpose captured in a graph with its noop flag: the host flips the device flag
    between replays (cached vs refreshed), and the source changes in place between them."""
    R, C = 512, 768
    src = torch.empty((R, C), dtype=torch.uint8, device=DEV)
    out = torch.zeros((C, R), dtype=torch.uint8, device=DEV)
    flag = torch.zeros(1, dtype=torch.float32, device=DEV)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        F.fp8_transpose(src, out, noop=flag, stream=cap)
    expect = np.zeros((C, R), np.uint8)
    for it, f in enumerate([0.0, 1.0, 1.0, 0.0, 1.0, 0.0]):
        xh = _bytes(S.seed_for(35, it), (R, C))
        src.copy_(torch.from_numpy(xh).to(DEV))
        flag.fill_(f)
        g.replay()
        torch.cuda.synchronize()
        expect = oracle.fp8_transpose(xh, noop=(f == 1.0), out_t_prev=expect)
        assert np.array_equal(u8_host(out), expect), (it, f)
