"""The no-allocation dbias + cast + transpose (fp8_dbias_cast_transpose_noalloc) against the
workspace entry point (fp8_dbias_cast_transpose) and the oracle, called through the C ABI.

Two calls in a row on the library's static scratch, the second with a smaller input (the
scratch then still holds the first call's partials), at the backward-prep shape [8192, 4096],
at shapes that give each CU four and three tiles in the one-launch form, and at ragged shapes; every output must equal the workspace entry point's bit for bit (same
kernels, same summation order), and the codes, amax and inverse scale the oracle's."""
import ctypes

import numpy as np
import pytest
import torch

import fp8_delayed_scaling_amd as F
import oracle
import synthetic as S
from helpers import DEV, bf16_dev, f32_bits, scalar, u8_host

pytestmark = pytest.mark.gpu


def _abi():
    f = F.lib().fp8_dbias_cast_transpose_noalloc
    P, I64, INT = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f.argtypes = [P, I64, I64, P, INT, P, P, P, P, P, P]
    f.restype = INT
    return f


def _outputs(R, C):
    return (torch.full((R, C), 0xA5, dtype=torch.uint8, device=DEV),
            torch.full((C, R), 0x5A, dtype=torch.uint8, device=DEV),
            torch.full((C,), float("nan"), dtype=torch.float32, device=DEV),
            scalar(0.0), scalar(0.0))


def _one(shape, seed):
    R, C = shape
    print(f"noalloc dbias {shape}", flush=True)
    dyh = S.normal_bf16(seed, shape, 0.01)
    dy = bf16_dev(dyh)
    scale = scalar(2048.0)
    stream = torch.cuda.current_stream().cuda_stream
    # the new entry point, straight through the C ABI
    out, out_t, db, slot, sinv = _outputs(R, C)
    st = _abi()(dy.data_ptr(), R, C, scale.data_ptr(), F.E5M2, out.data_ptr(), out_t.data_ptr(), sinv.data_ptr(),
                slot.data_ptr(), db.data_ptr(), stream)
    assert st == 0, F.fp8ds_status_string(st)
    # the existing entry point with its own workspace
    rout, rout_t, rdb, rslot, rsinv = _outputs(R, C)
    ws = torch.zeros(F.fp8_dbias_workspace_bytes(R, C), dtype=torch.uint8, device=DEV)
    F.fp8_dbias_cast_transpose(dy, scale, F.E5M2, rout, rout_t, rdb, ws, rsinv, rslot)
    torch.cuda.synchronize()
    assert torch.equal(out, rout) and torch.equal(out_t, rout_t)
    assert torch.equal(db.view(torch.int32), rdb.view(torch.int32))
    assert f32_bits(slot.item()) == f32_bits(rslot.item()) and f32_bits(sinv.item()) == f32_bits(rsinv.item())
    # and the oracle: codes, transpose, amax and inverse scale exact, dbias within its bound
    q, qt, a, s, dbr = oracle.dbias_cast_transpose(dyh, 2048.0, F.E5M2)
    assert np.array_equal(u8_host(out), q) and np.array_equal(u8_host(out_t), qt)
    assert f32_bits(slot.item()) == f32_bits(a) and f32_bits(sinv.item()) == f32_bits(s)
    bound = 1e-5 * np.abs(S.bf16_bits_to_f64(dyh)).sum(axis=0) + 1e-30
    assert np.all(np.abs(db.cpu().numpy().astype(np.float64) - dbr) <= bound)


@pytest.mark.parametrize("shapes", [((8192, 4096), (2048, 1024)), ((8192, 8192), (12288, 4096)), ((1300, 777), (260, 136))])
def test_noalloc_two_calls_second_smaller(shapes):
    big, small = shapes
    _one(big, S.seed_for(3, 12))
    _one(small, S.seed_for(3, 13))


def test_noalloc_rejects_beyond_scratch():
    R, C = 8192, 80000          # 10.24 MB of partials > the 8 MiB scratch
    dy = torch.zeros((R, 16), dtype=torch.bfloat16, device=DEV)   # never read: rejected first
    st = _abi()(dy.data_ptr(), R, C, dy.data_ptr(), F.E5M2, dy.data_ptr(), dy.data_ptr(), None, None,
                dy.data_ptr(), None)
    assert st == -8
