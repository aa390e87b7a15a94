"""Plain CPU oracle for the dequantizing matrix multiplies, in float64.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP library
never calls it and shares no code with it; the two meet only through the
packed bytes produced by the ``synth`` input generators.

What it computes, and where the pages define it:

* Element decoders, one per stored number type:
  - E2M1 ("TurboEXL3", section 2.1, MXFP4 bullet): sign bit 3, magnitude index
    bits 0-2 into the list 0, 0.5, 1, 1.5, 2, 3, 4, 6.
  - E8M0 (same bullet, "8-bit power-of-two scale", OCP MX reference [3]):
    2^(e - 127); 0xFF is NaN.
  - E4M3 (same section, NVFP4 bullet, "8-bit floating-point scale"): sign,
    4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0,
    S.1111.111 is NaN (OCP FP8 E4M3).
  - float16 and bfloat16 by their IEEE-style bit fields.
* Dequantization of each weight to its exact real value:
  - affine4_g64 (section 2.1, MLX affine bullet: 16-bit scale and 16-bit bias
    per 64 weights; section 3.1: each weight costs a shift, a mask and one
    multiply-add):
    w = s * q + b.
  - mxfp4 (section 2.1): w = e2m1(c) * 2^(E - 127), one E per 32 weights.
  - nvfp4 (section 2.1: E4M3 scale per 16 weights plus one 32-bit scale per
    tensor): w = e2m1(c) * e4m3(S) * g.
  - q6_k (splash PR #19, "What changed": 6-bit codes with zero point 32, a
    per-16 scale and a per-256 float16 scale): w = d * sc * (q - 32), with
    q = low nibble | high 2 bits << 4.
  All four products are exact in float64.
* Products summed in float64 from the exact weights and the bfloat16 inputs
  taken exactly: y[m][n] = sum_k w[n][k] x[m][k] (+ r[m][n]).
* The MoE route step as plain counting: per-expert row counts, their
  exclusive prefix sums and the table of 128-row tiles ("TurboEXL3"
  section 4.1, steps 1 and 6).
* The MoE layer stage by stage ("TurboEXL3" section 4.1: gate and up in one
  GEMM, SwiGLU in 32-bit between them and the down projection, then the
  score-weighted sum of each token's ten expert outputs), rounding only where
  the library's contract rounds: h = bf16(silu(g) * u), y = sum_k w_k d_k
  (+ w_s d_shared).
* The MoE router ("TurboEXL3" section 4.2, the router's top-k and softmax;
  the model description: 10 of 512 experts per token): the k largest logits
  (equal logits in ascending expert id, -0 equal to +0), in descending order,
  weighted by the softmax over those k, in float64.
* W4A4 ("TurboEXL3" section 2.2, the W4A4 bullet: the activations are also
  quantized to a 4-bit format on the fly, with a scale per block, so both
  operands of the multiply are FP4).  Here the block-scaled format of the
  activations is MXFP4 (section 2.1: E2M1 values with one E8M0 power-of-two
  scale per 32), the format the MI355X matrix cores multiply natively.  Each
  row of x is cut into blocks of 32 along K; a block's shared exponent is
  E = floor(log2(amax)) - 2 (the largest E2M1 magnitude is 6 = 1.5 * 2^2; OCP
  MX conversion, reference [3]), stored as E8M0 = E + 127 (raised to 0 where
  that is negative; 0 with all codes 0 for an all-zero block); every value is
  divided by 2^E and rounded to the nearest E2M1 value, ties to the even
  code, magnitudes past 6 saturating to 6, a value that rounds to zero taking
  code 0.  The product is then the exact sum of the dequantized weights times
  the dequantized activation codes.
* The EXL3 rotation stages ("TurboEXL3" section 3.1, prepare and finish;
  section 2.3: sign-randomized Hadamard transforms in blocks of 128, with one
  16-bit scale per input and per output channel as the only scales), on
  their own: prepare(x) = bf16(H (s_in * x)) and finish(y) = s_out * (H y),
  block by block of 128 values, H the orthonormal 128-point Hadamard matrix
  H_128 / sqrt(128) built by Sylvester's doubling (H_1 = [1], H_2n = [[H_n,
  H_n], [H_n, -H_n]]), the random signs carried by the sign bits of the
  float16 channel scales.
* Alongside every output, its magnitude sum sum_k |w||x| (+ |r|), which sets the
  tolerance |y - y_ref| <= 2e-3 * magnitude.

Everything is vectorised numpy; no blocking, fusion or reordering beyond the
definitions above.
"""

from __future__ import annotations

import numpy as np

AFFINE4_G64, MXFP4, NVFP4, Q6_K = 1, 2, 3, 4

# E2M1 magnitudes as listed in "TurboEXL3", section 2.1.
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


# ------------------------------------------------------------ element types

def e2m1(code) -> np.ndarray:
    c = np.asarray(code).astype(np.int64) & 0xF
    mag = np.asarray(E2M1_MAGNITUDES)[c & 7]
    return np.where(c & 8, -1.0, 1.0) * mag


def e8m0(e) -> np.ndarray:
    e = np.asarray(e).astype(np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))


def e4m3(b) -> np.ndarray:
    b = np.asarray(b).astype(np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    ex = (b >> 3) & 0xF
    m = b & 7
    val = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ex - 7))
    val = np.where((ex == 15) & (m == 7), np.nan, val)
    return sign * val


def fp16(bits_or_array) -> np.ndarray:
    a = np.asarray(bits_or_array)
    if a.dtype != np.float16:
        a = a.astype(np.uint16).view(np.float16)
    return a.astype(np.float64)


def bf16(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_round(a) -> np.ndarray:
    """float32 values -> bfloat16 bit patterns, round to nearest even
    (NaN kept quiet)."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


# ------------------------------------------------------------ dequantization

def _nibbles(codes: np.ndarray) -> np.ndarray:
    lo = codes & 0xF
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)


def _crumbs(b: np.ndarray) -> np.ndarray:
    parts = [(b >> (2 * i)) & 3 for i in range(4)]
    return np.stack(parts, axis=-1).reshape(*b.shape[:-1], b.shape[-1] * 4)


def dequant(p, e: int = 0, rows=None) -> np.ndarray:
    """Exact float64 weights of matrix ``e`` of packed weight ``p``
    (rows ``rows`` only, if given): shape [len(rows) or n][k]."""
    sel = slice(None) if rows is None else np.asarray(rows)
    k = p.k
    codes = p.codes[e][sel].astype(np.int64)
    if p.fmt == AFFINE4_G64:
        q = _nibbles(codes).astype(np.float64)
        sb = fp16(p.scales[e][sel])                          # [r][k/64][2]
        s = np.repeat(sb[..., 0], 64, axis=-1)
        b = np.repeat(sb[..., 1], 64, axis=-1)
        return s * q + b
    if p.fmt == MXFP4:
        v = e2m1(_nibbles(codes))
        sc = np.repeat(e8m0(p.scales[e][sel]), 32, axis=-1)
        return v * sc
    if p.fmt == NVFP4:
        v = e2m1(_nibbles(codes))
        sc = np.repeat(e4m3(p.scales[e][sel]), 16, axis=-1)
        g = float(np.float32(p.tensor_scale[e]))
        return v * sc * g
    if p.fmt == Q6_K:
        lo = _nibbles(codes)
        hi = _crumbs(p.codes_hi[e][sel].astype(np.int64))
        q = lo | (hi << 4)
        sc = np.repeat(p.scales[e][sel].astype(np.int8).astype(np.float64), 16, axis=-1)
        d = np.repeat(fp16(p.scales2[e][sel]), 256, axis=-1)
        assert q.shape[-1] == k
        return d * sc * (q - 32).astype(np.float64)
    raise ValueError(f"unknown format {p.fmt}")


def dequant_f32(p, e: int = 0, rows=None) -> np.ndarray:
    """Canonical float32 weights: the exact value rounded once to nearest."""
    return dequant(p, e, rows).astype(np.float32)


def dequant_bf16(p, e: int = 0, rows=None) -> np.ndarray:
    """Canonical bfloat16 weights (uint16 bits): the canonical float32 value
    rounded to nearest even."""
    return bf16_round(dequant_f32(p, e, rows))


# ------------------------------------------------------------ products

def gemv(p, x_bits, residual_bits=None, rows=None, e: int = 0):
    """y_ref [m][n_sel] and its magnitude sum for y = W x^T (+ residual).

    ``x_bits``: bfloat16 bits [m][k]; ``residual_bits``: bfloat16 bits [m][n]."""
    w = dequant(p, e, rows)                      # [r][k]
    x = bf16(x_bits)                             # [m][k]
    y = x @ w.T
    mag = np.abs(x) @ np.abs(w).T
    if residual_bits is not None:
        r = bf16(residual_bits)
        if rows is not None:
            r = r[:, np.asarray(rows)]
        y = y + r
        mag = mag + np.abs(r)
    return y, mag


gemm = gemv


def silu(g):
    return g / (1.0 + np.exp(-g))


def moe(gate_up, down, x_bits, topk_ids, topk_w, num_routed: int, num_shared: int,
        shared_w=None, tokens=None, h_given=None):
    """Grouped MoE layer, token by token.

    ``gate_up``: batch E+S packed weights, n = 2I (rows 0..I-1 gate, I..2I-1 up),
    k = H.  ``down``: batch E+S, n = H, k = I.  ``x_bits`` [T][H] bf16 bits.
    ``topk_ids`` int [T][k], ``topk_w`` float32 [T][k]; shared experts are
    stored after the routed ones and every token visits them with weight
    ``shared_w[t]`` (1 when None).

    ``h_given`` (optional): dict (t, slot) -> bf16 bits [I] of the SwiGLU
    output to use instead of the oracle's own (slot = 0..k-1 routed,
    k.. for shared), so that the down stage can be checked on exactly the
    activations another implementation produced.

    Returns (y [nt][H], mag [nt][H], h dict (t, slot) -> bf16 bits [I]).
    """
    T = x_bits.shape[0]
    tokens = range(T) if tokens is None else tokens
    inter = gate_up.n // 2
    cache_gu, cache_dn = {}, {}

    def w_gu(e):
        if e not in cache_gu:
            cache_gu[e] = dequant(gate_up, e)
        return cache_gu[e]

    def w_dn(e):
        if e not in cache_dn:
            cache_dn[e] = dequant(down, e)
        return cache_dn[e]

    ys, mags, hs = [], [], {}
    for t in tokens:
        xt = bf16(x_bits[t])
        experts = [(int(topk_ids[t][j]), float(np.float32(topk_w[t][j])), j)
                   for j in range(topk_ids.shape[1])]
        for s in range(num_shared):
            sw = 1.0 if shared_w is None else float(np.float32(shared_w[t]))
            experts.append((num_routed + s, sw, topk_ids.shape[1] + s))
        y = np.zeros(down.n)
        mag = np.zeros(down.n)
        for e, wt, slot in experts:
            gu = w_gu(e) @ xt
            if h_given is not None:
                hb = np.asarray(h_given[(t, slot)])
            else:
                h32 = (silu(gu[:inter]) * gu[inter:]).astype(np.float32)
                hb = bf16_round(h32)
            hs[(t, slot)] = hb
            h = bf16(hb)
            wd = w_dn(e)
            y += wt * (wd @ h)
            mag += abs(wt) * (np.abs(wd) @ np.abs(h))
        ys.append(y)
        mags.append(mag)
    return np.array(ys), np.array(mags), hs


def router(logits, k: int):
    """Router top-k and softmax ("TurboEXL3" section 4.2: the router's top-k
    and softmax).  ``logits`` float [T][E] (taken exactly); returns (ids int32
    [T][k], weights float64 [T][k]): per token the experts ordered by
    descending logit, equal logits by ascending id (-0 == +0), first k kept,
    weights exp(l_r - max) / sum over the k chosen of exp(l_j - max)."""
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    wts = np.empty((T, k))
    for t in range(T):
        # sort key: (-logit, id); -0.0 and +0.0 compare equal as floats
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        top = lg[t, order]
        z = np.exp(top - top.max())
        ids[t] = order
        wts[t] = z / z.sum()
    return ids, wts


def moe_grouping(topk_ids, num_routed: int, num_shared: int, tile_rows: int = 128):
    """The route step ("TurboEXL3" section 4.1, step 1: count each expert's
    tokens, group the tokens by expert, build the table of row tiles; 128-row
    tiles per step 6), written as the plain count / exclusive-scan / split.

    An id outside [0, num_routed) names no expert: its slot is dropped.
    Shared experts follow the routed ones and take every token.

    Returns a dict with the parts of the grouping that are unique:
      counts [E+S], offsets [E+S+1] (exclusive prefix sums, last = total rows),
      valid bool [T][k], active (experts with rows, ascending),
      tiles [(expert, first_row, rows)] in expert order, err (1 if any slot was
      dropped).  Which row of its expert's group a slot lands on is not unique.
    """
    ids = np.asarray(topk_ids).astype(np.int64)
    T = ids.shape[0]
    E, S = num_routed, num_shared
    valid = (ids >= 0) & (ids < E)
    counts = [0] * (E + S)
    for e in ids[valid].ravel():
        counts[int(e)] += 1
    for s in range(S):
        counts[E + s] = T
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    active = [e for e in range(E + S) if counts[e] > 0]
    tiles = []
    for e in active:
        for r in range(0, counts[e], tile_rows):
            tiles.append((e, offsets[e] + r, min(tile_rows, counts[e] - r)))
    return dict(counts=np.array(counts, np.int64), offsets=np.array(offsets, np.int64),
                valid=valid, active=np.array(active, np.int64),
                tiles=np.array(tiles, np.int64).reshape(-1, 3), err=int((~valid).any()))


# ------------------------------------------------------------ W4A4

def mxfp4_quantize(x_bits):
    """Activations (bfloat16 bits [m][k], k a multiple of 32) -> MXFP4: codes
    uint8 [m][k/2] (element 2j in the low nibble of byte j) and E8M0 scales
    uint8 [m][k/32], by the rule in the module docstring."""
    x = bf16(x_bits)
    m, k = x.shape
    blk = x.reshape(m, k // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    # floor(log2(amax)) from frexp: amax = f * 2^e with f in [0.5, 1)
    _, e = np.frexp(amax)
    shared = (e - 1) - 2
    e8m0 = np.where(amax > 0, np.maximum(shared + 127, 0), 0).astype(np.int64)
    scale = np.ldexp(1.0, e8m0 - 127)[..., None]
    v = np.where(amax[..., None] > 0, blk / scale, 0.0)
    a = np.abs(v)
    # nearest magnitude in the printed list, ties to the even index
    mags = np.asarray(E2M1_MAGNITUDES)
    dist = np.abs(a[..., None] - mags)                   # [m][k/32][32][8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                                  # one or two nearest
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    codes = np.where(idx > 0, idx | np.where(v < 0, 8, 0), 0).astype(np.uint8)
    codes = codes.reshape(m, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, e8m0.astype(np.uint8)


def mxfp4_dequantize_activations(codes, scales):
    """Exact float64 activations [m][k] of MXFP4 codes [m][k/2] and E8M0
    scales [m][k/32]."""
    c = _nibbles(np.asarray(codes).astype(np.int64))
    return e2m1(c) * np.repeat(e8m0(scales), 32, axis=-1)


def gemm_w4a4(p, x_bits, residual_bits=None, rows=None):
    """W4A4 product: y_ref [m][n_sel] = dequant(w) . dequant(mxfp4(x))^T
    (+ residual) in float64, and its magnitude sum.  ``p`` is an MXFP4
    weight."""
    if p.fmt != MXFP4:
        raise ValueError("W4A4 takes MXFP4 weights")
    codes, scales = mxfp4_quantize(x_bits)
    xq = mxfp4_dequantize_activations(codes, scales)
    w = dequant(p, 0, rows)
    y = xq @ w.T
    mag = np.abs(xq) @ np.abs(w).T
    if residual_bits is not None:
        r = bf16(residual_bits)
        if rows is not None:
            r = r[:, np.asarray(rows)]
        y = y + r
        mag = mag + np.abs(r)
    return y, mag


# ------------------------------------------------------------ Hadamard stages

HADAMARD_BLOCK = 128


def sylvester_hadamard(n: int) -> np.ndarray:
    """The n x n Sylvester Hadamard matrix (n a power of two), entries +-1."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def _blocks_transform(v):
    """[rows][len] -> each 128-block multiplied by H_128 / sqrt(128)."""
    rows, ln = v.shape
    h = sylvester_hadamard(HADAMARD_BLOCK) / np.sqrt(HADAMARD_BLOCK)
    b = v.reshape(rows, ln // HADAMARD_BLOCK, HADAMARD_BLOCK)
    return (b @ h.T).reshape(rows, ln)


def hadamard_prepare(x_bits, scale_f16=None):
    """Prepare stage: bf16 x [m][k] -> (float64 H(s * x) before its output
    rounding [m][k], bf16 bits of it, magnitude sum per output
    sum |H_ij| |s_j x_j| = sum |s_j x_j| / sqrt(128) over the block)."""
    x = bf16(x_bits)
    s = np.ones(x.shape[1]) if scale_f16 is None else fp16(scale_f16)
    v = x * s
    y = _blocks_transform(v)
    m, k = v.shape
    mag = np.repeat(np.abs(v).reshape(m, k // HADAMARD_BLOCK, HADAMARD_BLOCK).sum(-1)
                    / np.sqrt(HADAMARD_BLOCK), HADAMARD_BLOCK, axis=-1).reshape(m, k)
    return y, bf16_round(y.astype(np.float32)), mag


def hadamard_finish(y, scale_f16=None):
    """Finish stage: float32 y [m][n] -> (float64 s * H y [m][n], magnitude
    sum |s| sum |y| / sqrt(128) over the block)."""
    v = np.asarray(y, np.float64)
    s = np.ones(v.shape[1]) if scale_f16 is None else fp16(scale_f16)
    out = _blocks_transform(v) * s
    m, n = v.shape
    mag = np.repeat(np.abs(v).reshape(m, n // HADAMARD_BLOCK, HADAMARD_BLOCK).sum(-1)
                    / np.sqrt(HADAMARD_BLOCK), HADAMARD_BLOCK, axis=-1).reshape(m, n) * np.abs(s)
    return out, mag


def within_tolerance(y, y_ref, mag, rel: float = 2e-3):
    """Elementwise |y - y_ref| <= rel * mag (the parity rule for products)."""
    return np.abs(np.asarray(y, np.float64) - y_ref) <= rel * mag


def bf16_half_ulp(v) -> np.ndarray:
    """Half a unit in the last place of bfloat16 (8 significant bits) at |v|."""
    _, e = np.frexp(np.abs(np.asarray(v, np.float64)))
    return np.ldexp(1.0, e - 9)


def within_tolerance_bf16(y, y_ref, mag, rel: float = 2e-3):
    """The product rule for results stored as bfloat16: the accumulation bound
    plus the output's own rounding, which the reference applies at the same
    point (TurboEXL3 section 4.4: tolerance kernels keep the reference's
    rounding points and differ only in summation order)."""
    return np.abs(np.asarray(y, np.float64) - y_ref) <= rel * mag + bf16_half_ulp(y_ref)
