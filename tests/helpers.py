"""Shared helpers of the GPU parity tests: host <-> device copies of bit patterns and the
GEMM tolerance.  No arithmetic of the method lives here."""
import numpy as np
import torch

DEV = "cuda:0"


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    """bfloat16 bit patterns (uint16) -> a bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u8_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy()


def f32_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).reshape(-1).view(np.uint32)


def scalar(v: float) -> torch.Tensor:
    return torch.tensor([v], dtype=torch.float32, device=DEV)


def to_f64(D: torch.Tensor) -> np.ndarray:
    return D.detach().float().cpu().numpy().astype(np.float64)


GEMM_TOL = 2e-3          # normwise, float32 accumulation against the float64 oracle
BF16_HALF_ULP_REL = 2.0 ** -8   # bfloat16 rounding: |round(v) - v| <= 2^-8 |v|


def gemm_close(got: np.ndarray, ref: np.ndarray, bf16_out: bool, scale_ref: float = None):
    """Normwise check max|D - R| <= 2e-3 * max|R| (fp32 output); a bfloat16 output may also
    differ by its own rounding, at most 2^-8 |R| per element (plus the float32 part)."""
    ref = np.asarray(ref, dtype=np.float64)
    big = scale_ref if scale_ref is not None else float(np.abs(ref).max()) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = GEMM_TOL * big + (BF16_HALF_ULP_REL * (np.abs(ref) + GEMM_TOL * big) if bf16_out else 0.0)
    ok = err <= bound
    if not np.all(ok):
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"GEMM mismatch at {i}: got {got[i]} ref {ref[i]} err {err[i]} bound "
                             f"{np.broadcast_to(bound, err.shape)[i]} (max|R| {big})")
    return float(err.max() / big) if big else 0.0


def oracle_cast_transpose_rows(oracle, x, scale, fmt, nthreads=16, with_dbias=False):
    """The oracle's cast+transpose (and float64 dbias) of a large 2-D tensor, one row block per
    host thread (the oracle's C calls release the GIL): the blocks' codes stacked, their
    transposed codes side by side, the largest block amax, the sum of the blocks' column sums.
    Every element goes through the oracle's own per-element code; only the rows are split."""
    from concurrent.futures import ThreadPoolExecutor
    R = x.shape[0]
    n = max(1, min(nthreads, R // 256))
    edges = [R * k // n for k in range(n + 1)]

    def one(k):
        xb = x[edges[k]:edges[k + 1]]
        q, qt, a, si = oracle.cast_transpose(xb, scale, fmt)
        return q, qt, a, si, (oracle.dbias(xb) if with_dbias else None)

    with ThreadPoolExecutor(n) as ex:
        parts = list(ex.map(one, range(n)))
    q = np.concatenate([p[0] for p in parts], 0)
    qt = np.concatenate([p[1] for p in parts], 1)
    amax = max(np.float32(p[2]) for p in parts)
    db = sum(p[4] for p in parts) if with_dbias else None
    return q, qt, np.float32(amax), parts[0][3], db


def kernel_names(fn):
    """Names of the GPU kernels ``fn`` launches (torch's profiler), or None when it records none."""
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    names = [e.name for e in prof.events() if e.device_type == torch.autograd.DeviceType.CUDA]
    return names or None
