"""Encoders that turn real-valued synthetic weights into packed codes.

These produce test and benchmark inputs only: the library and the oracle both
receive the packed bytes, never the real weights.  Each encoder rounds to the
nearest representable code, ties to the even code, and saturates at the
format's largest magnitude.  The rules are the plainest reading of the
"TurboEXL3" article, section 2.1 (block-scaled 4-bit formats), and of the
splash pull request #19 description (Q6_K's 6-bit codes with zero point 32):

* affine4_g64: scale = (max - min) / 15 and bias = min per 64 weights, both
  stored as float16; code = round((w - bias) / scale) clamped to 0..15.
* mxfp4: shared exponent E = floor(log2(amax)) - 2 per 32 weights (the E2M1
  maximum is 1.5 * 2^2), stored as E8M0 = E + 127; codes round w / 2^E onto
  the E2M1 grid.
* nvfp4: tensor multiplier g = amax_tensor / (448 * 6) in float32; block scale
  S = E4M3(amax_block / (6 g)) per 16 weights; codes round w / (S g).
* q6_k: per 16-weight sub-block sigma = amax / 31; per 256-weight super-block
  d = float16(max sigma / 127); sub-block scale sc = round(sigma / d) as int8;
  code q = round(w / (d sc)) + 32 clamped to 0..63.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import formats as F
from . import rng

# Decision points between neighbouring E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
# and whether a value exactly on the point moves up (the upper neighbour has
# the even index) or stays.
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_E2M1_TIE_UP = np.array([False, True, False, True, False, True, False])


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code (sign in bit 3) for each value; saturates at +-6.
    A magnitude that rounds to zero gets code 0 whatever its sign."""
    a = np.abs(v)
    idx = np.zeros(a.shape, np.uint8)
    for mid, up in zip(_E2M1_MID, _E2M1_TIE_UP):
        idx += (a >= mid) if up else (a > mid)
    sign = ((v < 0) & (idx > 0)).astype(np.uint8)
    return (sign << 3) | idx


def e4m3_round(v: np.ndarray):
    """Round non-negative values to E4M3 (bias 7, subnormals, largest finite
    448), to nearest, ties to even, saturating at 448.  Returns the code and
    the value it was rounded to."""
    v = np.asarray(v, np.float64)
    code = np.zeros(v.shape, np.int64)
    val = np.zeros(v.shape, np.float64)
    sub = v < 2.0 ** -6
    ms = np.rint(v[sub] / 2.0 ** -9)            # 8 steps of 2^-9 reach 2^-6
    code[sub] = ms.astype(np.int64)
    val[sub] = ms * 2.0 ** -9
    nrm = ~sub
    if nrm.any():
        m, ex = np.frexp(v[nrm])                # v = m * 2^ex, m in [0.5, 1)
        ex = ex - 1                              # v = (2m) * 2^ex
        mm = np.rint((2.0 * m - 1.0) * 8.0)
        carry = mm == 8
        ex = ex + carry
        mm = np.where(carry, 0.0, mm)
        code[nrm] = ((ex + 7) << 3) | mm.astype(np.int64)
        val[nrm] = (1.0 + mm / 8.0) * np.ldexp(1.0, ex)
    sat = code > 0x7E
    code[sat] = 0x7E
    val[sat] = 448.0
    return code.astype(np.uint8), val


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bfloat16 (round to nearest even), as uint16 bits."""
    u = np.asarray(a, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


# ---------------------------------------------------------------- encoders

def _affine(w: np.ndarray):
    n, k = w.shape
    g = w.reshape(n, k // 64, 64)
    mn = g.min(-1)
    mx = g.max(-1)
    s = ((mx - mn) / 15.0).astype(np.float16)
    b = mn.astype(np.float16)
    sd = s.astype(np.float64)[..., None]
    bd = b.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sd > 0, np.clip(np.rint((g - bd) / sd), 0, 15), 0)
    sc = np.stack([s, b], axis=-1)
    return F.pack_nibbles(q.reshape(n, k)), sc


def _mxfp4(w: np.ndarray):
    n, k = w.shape
    g = w.reshape(n, k // 32, 32)
    amax = np.abs(g).max(-1)
    _, ex = np.frexp(amax)
    e = np.where(amax > 0, np.clip(ex - 1 - 2 + 127, 0, 254), 0)
    scale = np.ldexp(1.0, (e - 127).astype(np.int64))[..., None]
    codes = np.where(amax[..., None] > 0, e2m1_encode(g / scale), 0).astype(np.uint8)
    return F.pack_nibbles(codes.reshape(n, k)), e.astype(np.uint8)


def _nvfp4(w: np.ndarray, g32: np.float32):
    n, k = w.shape
    gd = float(g32)
    blk = w.reshape(n, k // 16, 16)
    amax = np.abs(blk).max(-1)
    s, sv = e4m3_round(amax / (6.0 * gd))
    sv = sv[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        codes = np.where(sv > 0, e2m1_encode(blk / (sv * gd)), 0).astype(np.uint8)
    return F.pack_nibbles(codes.reshape(n, k)), s


def _q6k(w: np.ndarray):
    n, k = w.shape
    sb = w.reshape(n, k // 256, 16, 16)
    sigma = np.abs(sb).max(-1) / 31.0                      # [n, k/256, 16]
    d = (sigma.max(-1) / 127.0).astype(np.float16)         # [n, k/256]
    dd = d.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(dd > 0, np.clip(np.rint(sigma / dd), -128, 127), 0)
        den = (dd * sc)[..., None]
        q = np.where(den != 0, np.clip(np.rint(sb / den) + 32, 0, 63), 32)
    q = q.astype(np.uint8).reshape(n, k)
    return (F.pack_nibbles(q & 15), F.pack_crumbs(q >> 4),
            sc.astype(np.int8).reshape(n, k // 16), d)


def nvfp4_tensor_scale(amax: float) -> np.float32:
    return np.float32(amax / (448.0 * 6.0)) if amax > 0 else np.float32(1.0)


def quantize(fmt: int, w: np.ndarray, tensor_scale: np.float32 | None = None) -> F.Packed:
    """Quantize one real N x K matrix into a batch-1 ``Packed``."""
    n, k = w.shape
    p = F.empty(fmt, n, k, 1)
    _quantize_rows(p, 0, 0, w, tensor_scale)
    return p


def _quantize_rows(p: F.Packed, e: int, r0: int, w: np.ndarray, ts):
    r1 = r0 + w.shape[0]
    if p.fmt == F.AFFINE4_G64:
        c, s = _affine(w)
        p.codes[e, r0:r1] = c
        p.scales[e, r0:r1] = s
    elif p.fmt == F.MXFP4:
        c, s = _mxfp4(w)
        p.codes[e, r0:r1] = c
        p.scales[e, r0:r1] = s
    elif p.fmt == F.NVFP4:
        if ts is None:
            ts = nvfp4_tensor_scale(float(np.abs(w).max()))
        p.tensor_scale[e] = ts
        c, s = _nvfp4(w, np.float32(ts))
        p.codes[e, r0:r1] = c
        p.scales[e, r0:r1] = s
    elif p.fmt == F.Q6_K:
        c, h, s, d = _q6k(w)
        p.codes[e, r0:r1] = c
        p.codes_hi[e, r0:r1] = h
        p.scales[e, r0:r1] = s
        p.scales2[e, r0:r1] = d
    else:
        raise ValueError(p.fmt)


# ------------------------------------------------- seeded synthetic weights

def _weight_rows(seed, name, n, k, std, outlier_rate, outlier_mult, r0, r1):
    w = rng.normal_matrix(seed, name, n, k, std, row0=r0, nrows=r1 - r0)
    if outlier_rate > 0:
        u = rng.uniform_matrix(seed, name + "/outliers", n, k, row0=r0, nrows=r1 - r0)
        w = np.where(u < outlier_rate, w * outlier_mult, w)
    return w


def synthetic_weight(fmt: int, n: int, k: int, *, seed: int = rng.BASE_SEED,
                     name: str = "W", batch: int = 1, std: float = 0.02,
                     outlier_rate: float = 0.0, outlier_mult: float = 8.0,
                     rows_per_chunk: int | None = None) -> F.Packed:
    """A batch of N x K weights drawn N(0, std^2) (optionally with a fraction
    ``outlier_rate`` of them multiplied by ``outlier_mult``), quantized.
    Matrix e of the batch uses stream ``f"{name}[{e}]"``."""
    p = F.empty(fmt, n, k, batch)
    if rows_per_chunk is None:
        rows_per_chunk = max(1, (1 << 21) // k)
    jobs = [(e, r0, min(n, r0 + rows_per_chunk)) for e in range(batch)
            for r0 in range(0, n, rows_per_chunk)]

    if fmt == F.NVFP4 and rows_per_chunk >= n:
        # whole matrices per job: draw once, take the amax, quantize
        def whole_job(e):
            w = _weight_rows(seed, f"{name}[{e}]", n, k, std, outlier_rate, outlier_mult, 0, n)
            ts = nvfp4_tensor_scale(float(np.abs(w).max()))
            _quantize_rows(p, e, 0, w, ts)

        with ThreadPoolExecutor(_nthreads()) as ex:
            list(ex.map(whole_job, range(batch)))
        p.meta = dict(seed=seed, name=name, std=std, outlier_rate=outlier_rate)
        return p

    if fmt == F.NVFP4:
        # the tensor multiplier needs the whole matrix's amax first
        def amax_job(j):
            e, r0, r1 = j
            return e, float(np.abs(_weight_rows(seed, f"{name}[{e}]", n, k, std,
                                                outlier_rate, outlier_mult, r0, r1)).max())
        am = np.zeros(batch)
        with ThreadPoolExecutor(_nthreads()) as ex:
            for e, a in ex.map(amax_job, jobs):
                am[e] = max(am[e], a)
        p.tensor_scale[:] = [nvfp4_tensor_scale(a) for a in am]

    def job(j):
        e, r0, r1 = j
        w = _weight_rows(seed, f"{name}[{e}]", n, k, std, outlier_rate, outlier_mult, r0, r1)
        _quantize_rows(p, e, r0, w, None if fmt != F.NVFP4 else p.tensor_scale[e])

    if len(jobs) == 1:
        job(jobs[0])
    else:
        with ThreadPoolExecutor(_nthreads()) as ex:
            list(ex.map(job, jobs))
    p.meta = dict(seed=seed, name=name, std=std, outlier_rate=outlier_rate)
    return p


def synthetic_bf16(rows: int, cols: int, *, seed: int = rng.BASE_SEED, name: str = "x",
                   std: float = 1.0) -> np.ndarray:
    """N(0, std^2) activations rounded to bfloat16, as uint16 bits [rows][cols]."""
    return bf16_bits(rng.normal_matrix(seed, name, rows, cols, std))


def _nthreads() -> int:
    return max(1, min(16, os.cpu_count() or 1))
