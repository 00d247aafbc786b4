"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This module only draws numbers: it holds none of the FP8 method's arithmetic (no FP8
encoding, no scaling, no amax).  Every tensor is returned as host ``numpy`` bit patterns
(bfloat16 as ``uint16``), so both sides of a parity test consume the very same bytes.

Generator (counter-based, so any element can be drawn independently of the others):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014): the i-th 64-bit word of stream ``seed`` is ``mix(seed + (i + 1) * gamma)``
  with ``gamma = 0x9E3779B97F4A7C15`` and ``mix`` the published finaliser.
* uniform: the top 53 bits of a word scaled by ``2**-53``, in ``[0, 1)``.
* normal: Box-Muller on word pairs ``(2j, 2j+1)`` in float64, times the standard deviation.
* bfloat16: float64 -> float32 (numpy round-to-nearest-even) -> bfloat16 by
  round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

BASE_SEED = 0xF8D50000

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the bulk generator ``gen.c`` (gcc, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _clib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.synth_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                        ctypes.c_void_p]
        L.synth_normal_bf16.restype = None
        L.synth_scale_at.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_double,
                                     ctypes.c_double, ctypes.c_void_p]
        L.synth_scale_at.restype = None
        L.synth_normal_at.argtypes = [ctypes.c_uint64, ctypes.c_int64]
        L.synth_normal_at.restype = ctypes.c_double
        _lib = L
    return _lib


def seed_for(config: int, tensor: int) -> int:
    """Fixed seed of tensor ``tensor`` in workload ``config`` (both small integers)."""
    return BASE_SEED + 16 * config + tensor


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of SplitMix64 stream ``seed`` (uint64)."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform(seed: int, start: int, count: int) -> np.ndarray:
    """float64 uniforms in [0, 1) from words ``start ..`` of stream ``seed``."""
    w = splitmix64(seed, start, count)
    return (w >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def random_bytes(seed: int, shape) -> np.ndarray:
    """Uniform random bytes of ``shape``: the little-endian bytes of stream ``seed``'s words."""
    n = int(np.prod(shape))
    w = splitmix64(seed, 0, (n + 7) // 8)
    return np.ascontiguousarray(w.astype("<u8").view(np.uint8)[:n]).reshape(shape)


def normal_f64(seed: int, n: int, std: float) -> np.ndarray:
    """``n`` float64 samples of N(0, std^2) by Box-Muller, drawn chunk by chunk."""
    out = np.empty(n, dtype=np.float64)
    pairs = (n + 1) // 2
    for p0 in range(0, pairs, _CHUNK):
        p1 = min(pairs, p0 + _CHUNK)
        u = uniform(seed, 2 * p0, 2 * (p1 - p0)).reshape(-1, 2)
        r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))
        t = (2.0 * np.pi) * u[:, 1]
        z = np.empty((p1 - p0, 2), dtype=np.float64)
        z[:, 0] = r * np.cos(t)
        z[:, 1] = r * np.sin(t)
        lo, hi = 2 * p0, min(n, 2 * p1)
        out[lo:hi] = z.reshape(-1)[: hi - lo] * std
    return out


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 bits (RNE on the bit pattern; inputs finite)."""
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns (test helper; no rounding involved)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def normal_bf16(seed: int, shape, std: float) -> np.ndarray:
    """bfloat16 bits of shape ``shape`` with N(0, std^2) values (bulk path in ``gen.c``)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    L = _clib()
    base = out.ctypes.data
    step = 1 << 22  # even

    def run(s0):
        cnt = min(step, n - s0)
        L.synth_normal_bf16(seed & 0xFFFFFFFFFFFFFFFF, s0, cnt, float(std), ctypes.c_void_p(base + 2 * s0))

    starts = list(range(0, n, step))
    if len(starts) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(run, starts))
    elif starts:
        run(0)
    return out.reshape(shape)


def distinct_positions(seed: int, n: int, k: int) -> np.ndarray:
    """``k`` distinct indices in [0, n), drawn in order from stream ``seed`` (duplicates skipped)."""
    if k > n:
        raise ValueError("k > n")
    chosen: dict[int, None] = {}
    start = 0
    while len(chosen) < k:
        need = max(64, 2 * (k - len(chosen)))
        cand = (uniform(seed, start, need) * n).astype(np.int64)
        start += need
        for c in cand.tolist():
            if c not in chosen:
                chosen[c] = None
                if len(chosen) == k:
                    break
    return np.fromiter(chosen.keys(), dtype=np.int64, count=k)


def outlier_bf16(seed: int, shape, std: float = 1.0, frac: float = 0.001, factor: float = 1e3) -> np.ndarray:
    """N(0, std^2) bfloat16 with exactly ``round(frac * numel)`` distinct entries drawn as
    ``factor`` times their own normal sample (the factor is applied in float64, before the
    bfloat16 rounding)."""
    n = int(np.prod(shape))
    out = normal_bf16(seed, (n,), std)
    k = int(round(frac * n))
    if k:
        pos = np.ascontiguousarray(distinct_positions(seed ^ 0x5A5A5A5A, n, k))
        _clib().synth_scale_at(seed & 0xFFFFFFFFFFFFFFFF, pos.ctypes.data_as(ctypes.c_void_p), k, float(std),
                               float(factor), out.ctypes.data_as(ctypes.c_void_p))
    return out.reshape(shape)


def _uniform_at(seed: int, idx: np.ndarray) -> np.ndarray:
    """Uniforms at arbitrary word indices ``idx`` of stream ``seed``."""
    with np.errstate(over="ignore"):
        i = np.asarray(idx, dtype=np.uint64) + np.uint64(1)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def tiny_bf16(seed: int, shape, frac: float = 0.001) -> np.ndarray:
    """Zeros with ``round(frac * numel)`` distinct entries set to +-2^-133, the smallest
    positive bfloat16 subnormal (bit pattern 0x0001), signs drawn from the stream."""
    n = int(np.prod(shape))
    out = np.zeros(n, dtype=np.uint16)
    k = int(round(frac * n))
    if k:
        pos = distinct_positions(seed, n, k)
        sgn = (_uniform_at(seed ^ 0x33, np.arange(k)) < 0.5)
        out[pos] = np.where(sgn, 0x8001, 0x0001).astype(np.uint16)
    return out.reshape(shape)


def log_uniform_f32(seed: int, n: int, lo: float, hi: float) -> np.ndarray:
    """float32 values log-uniform in [lo, hi]."""
    u = uniform(seed, 0, n)
    return np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).astype(np.float32)
