"""Counter-based seeded random numbers for the synthetic inputs.

Every random value is a pure function of (seed, stream name, element index), so
any slice of any tensor can be regenerated on its own, in any order, by any
number of threads, and always comes out the same.  The generator is the
splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) applied to ``key + (index + 1) * gamma``.

Normals use the Box-Muller transform on two uniforms per element (the sine
half is discarded so that each element depends only on its own index).

This module holds no part of the dequantize/multiply arithmetic.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
BASE_SEED = 1234


def _mix(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def _fnv1a64(text: str) -> int:
    h = 0xCBF29CE484222325
    for b in text.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def stream_key(seed: int, name: str) -> np.uint64:
    """64-bit key of the named stream under ``seed``."""
    z = np.array([(seed ^ _fnv1a64(name)) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(z + GAMMA)[0]


def bits(key: np.uint64, idx: np.ndarray) -> np.ndarray:
    """Raw 64-bit outputs for element indices ``idx`` (uint64 array)."""
    with np.errstate(over="ignore"):
        return _mix(key + (idx.astype(np.uint64) + np.uint64(1)) * GAMMA)


def uniform(key: np.uint64, idx: np.ndarray) -> np.ndarray:
    """Uniform doubles in the open interval (0, 1)."""
    b = bits(key, idx) >> np.uint64(11)
    return (b.astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal(key: np.uint64, idx: np.ndarray) -> np.ndarray:
    """Standard normal doubles, one per index."""
    i2 = idx.astype(np.uint64) * np.uint64(2)
    u1 = uniform(key, i2)
    u2 = uniform(key, i2 + np.uint64(1))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_matrix(seed: int, name: str, rows: int, cols: int, std: float = 1.0,
                  row0: int = 0, nrows: int | None = None) -> np.ndarray:
    """Rows ``row0 .. row0+nrows`` of a ``rows x cols`` matrix of N(0, std^2)
    doubles; element (r, c) uses index ``r * cols + c`` of stream ``name``."""
    nrows = rows - row0 if nrows is None else nrows
    key = stream_key(seed, name)
    out = np.empty((nrows, cols), dtype=np.float64)
    chunk = max(1, (1 << 22) // max(cols, 1))

    def work(r):
        r1 = min(nrows, r + chunk)
        idx = (np.arange((row0 + r) * cols, (row0 + r1) * cols, dtype=np.uint64))
        out[r:r1] = normal(key, idx).reshape(r1 - r, cols) * std

    starts = list(range(0, nrows, chunk))
    if len(starts) == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, starts))
    return out


def uniform_matrix(seed: int, name: str, rows: int, cols: int,
                   row0: int = 0, nrows: int | None = None) -> np.ndarray:
    nrows = rows - row0 if nrows is None else nrows
    key = stream_key(seed, name)
    idx = np.arange(row0 * cols, (row0 + nrows) * cols, dtype=np.uint64)
    return uniform(key, idx).reshape(nrows, cols)


def randint_bytes(seed: int, name: str, count: int, lo: int = 0, hi: int = 256) -> np.ndarray:
    """``count`` integers uniform in [lo, hi) as uint8 (hi <= 256)."""
    key = stream_key(seed, name)
    b = bits(key, np.arange(count, dtype=np.uint64)) >> np.uint64(32)
    return (lo + (b % np.uint64(hi - lo))).astype(np.uint8)
