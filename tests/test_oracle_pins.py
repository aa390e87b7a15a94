"""Pins of the CPU oracle to facts that do not come from the oracle itself:
values printed on the pages (tests/golden), closed forms, library decoders,
exact integer arithmetic and brute force in exact rationals."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import formats as F
from synth import quant, rng, routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ------------------------------------------------------------ element types

def test_e2m1_matches_printed_magnitudes():
    rows = _golden("e2m1.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = float(oracle.e2m1(int(code)))
        assert got == float(val)
        assert np.signbit(got) == val.startswith("-")


def test_e2m1_is_a_two_bit_exponent_float():
    # OCP E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
    # subnormal with value m/2.  An independent route to the same 16 values.
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        v = -v if s else v
        assert float(oracle.e2m1(c)) == v


def test_e8m0_closed_form():
    e = np.arange(255)
    v = oracle.e8m0(e)
    assert v[127] == 1.0 and v[128] == 2.0 and v[126] == 0.5
    assert v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    assert np.all(v[1:] == 2 * v[:-1])
    assert np.isnan(oracle.e8m0(255))


def test_e4m3_matches_torch_float8_e4m3fn_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_anchor_values():
    assert oracle.e4m3(0x38) == 1.0
    assert oracle.e4m3(0x7E) == 448.0
    assert oracle.e4m3(0x01) == 2.0 ** -9
    assert oracle.e4m3(0x08) == 2.0 ** -6
    assert oracle.e4m3(0xB8) == -1.0
    assert np.isnan(oracle.e4m3(0x7F))
    v = oracle.e4m3(np.arange(0x7F))
    assert np.all(np.diff(v) > 0)


def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_round_matches_torch():
    r = np.random.default_rng(7)
    a = np.concatenate([
        r.standard_normal(100000).astype(np.float32),
        (r.standard_normal(10000) * 1e-39).astype(np.float32),     # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.0e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                 np.float32),
    ])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_round(a), ref)


def test_fp16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    got = oracle.fp16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------ layouts

def test_bits_per_weight():
    rows = _golden("bits_per_weight.txt")
    n, k = 96, 1024
    for row in rows:
        if row[0] == "q6_k_output":
            nn, kk, gb = int(row[1]), int(row[2]), float(row[3])
            total = nn * kk * 6.5625 / 8
            assert round(total / 1e9, 2) == gb
            continue
        fmt, bpw, extra = F.BY_NAME[row[0]], float(row[1]), int(row[2])
        p = F.empty(fmt, n, k)
        assert p.nbytes() == n * k * bpw / 8 + extra


def test_q6k_output_layer_bytes_exact():
    # 210 bytes per 256 weights at 248320 x 5120
    assert 248320 * 5120 // 256 * 210 == 1_042_944_000


# ------------------------------------------------------------ Q6_K identities

def _q6k_superblock(codes, d_bits, sc):
    """Pack one row of 256 six-bit codes by the layout definition, written
    here independently of the encoders: nibble k=2j+h in bits 4h of byte j,
    high bits of k=4j+i in bits 2i of byte j."""
    p = F.empty(F.Q6_K, 1, 256)
    for j in range(128):
        p.codes[0, 0, j] = (codes[2 * j] & 15) | ((codes[2 * j + 1] & 15) << 4)
    for j in range(64):
        b = 0
        for i in range(4):
            b |= (codes[4 * j + i] >> 4) << (2 * i)
        p.codes_hi[0, 0, j] = b
    p.scales[0, 0, :] = sc
    p.scales2[0, 0, 0] = np.uint16(d_bits).view(np.float16)
    return p


def test_q6k_operand_identity_exhaustive():
    g = {r[0]: r[1] for r in _golden("q6k_operand.txt")}
    base, sub = int(g["fp16_base"], 16), float(g["subtract"])
    codes = np.arange(64)
    half = (np.uint16(base) | (codes << 4).astype(np.uint16)).view(np.float16).astype(np.float64)
    assert np.array_equal(half, 1 + codes / 64)
    assert np.array_equal(half - sub, (codes - int(g["zero_point"])) / 64)
    assert np.array_equal((int(g["old_offset"]) + codes) + int(g["old_seed"]), codes - 32)
    # bfloat16 analogue used for bf16 operands: 0x3F80 | code << 1 = 1 + code/64
    hb = oracle.bf16((0x3F80 | (codes << 1)).astype(np.uint16))
    assert np.array_equal(hb - 1.5, (codes - 32) / 64)


def test_q6k_dequant_through_page_identity():
    codes = np.array([(7 * k + 3) % 64 for k in range(256)])
    # d = 1/64 (float16 0x2400), every sub-block scale 1 -> w = (code - 32)/64,
    # which the page writes as the float16 1 + code/64 less 1.5.
    p = _q6k_superblock(codes, 0x2400, 1)
    w = oracle.dequant(p)[0]
    ident = (np.uint16(0x3C00) | (codes << 4).astype(np.uint16)).view(np.float16).astype(np.float64) - 1.5
    assert np.array_equal(w, ident)
    # epilogue form: 64 s * sum((code-32)/64 x) = s * sum((code-32) x)
    sc = np.array([(-1) ** j * (j + 1) for j in range(16)], np.int8)
    p2 = _q6k_superblock(codes, 0x3C00, sc)              # d = 1
    w2 = oracle.dequant(p2)[0]
    assert np.array_equal(w2, np.repeat(sc.astype(np.float64), 16) * (codes - 32))


# ------------------------------------------------------------ exact rationals

def _frac_fp16(h):
    return Fraction(float(np.float16(h)))


def _frac_value(p, e, n, k):
    """Exact weight (n, k) from the stored bytes, decoded in rationals from
    the format definitions (E2M1 as a 2-bit-exponent float)."""
    byte = int(p.codes[e, n, k // 2])
    nib = (byte >> (4 * (k % 2))) & 15
    if p.fmt == F.AFFINE4_G64:
        s, b = p.scales[e, n, k // 64]
        return _frac_fp16(s) * nib + _frac_fp16(b)
    if p.fmt in (F.MXFP4, F.NVFP4):
        sg, ex, m = nib >> 3, (nib >> 1) & 3, nib & 1
        v = Fraction(m, 2) if ex == 0 else Fraction(2) ** (ex - 1) * (1 + Fraction(m, 2))
        v = -v if sg else v
        if p.fmt == F.MXFP4:
            return v * Fraction(2) ** (int(p.scales[e, n, k // 32]) - 127)
        sb = int(p.scales[e, n, k // 16])
        es, mm = (sb >> 3) & 15, sb & 7
        sv = Fraction(mm, 512) if es == 0 else (1 + Fraction(mm, 8)) * Fraction(2) ** (es - 7)
        sv = -sv if sb & 0x80 else sv
        return v * sv * Fraction(float(p.tensor_scale[e]))
    hi = (int(p.codes_hi[e, n, k // 4]) >> (2 * (k % 4))) & 3
    q = nib | (hi << 4)
    return _frac_fp16(p.scales2[e, n, k // 256]) * int(p.scales[e, n, k // 16]) * (q - 32)


@pytest.mark.parametrize("fmt,k", [(F.AFFINE4_G64, 128), (F.MXFP4, 64), (F.NVFP4, 32), (F.Q6_K, 256)])
def test_oracle_vs_exact_rationals(fmt, k):
    n, m = 3, 2
    p = quant.synthetic_weight(fmt, n, k, name=f"frac{fmt}", outlier_rate=0.05)
    # random bytes in the code planes too, so every code value is exercised
    p.codes[:] = rng.randint_bytes(11, f"c{fmt}", p.codes.size).reshape(p.codes.shape)
    if p.codes_hi is not None:
        p.codes_hi[:] = rng.randint_bytes(12, "h", p.codes_hi.size).reshape(p.codes_hi.shape)
    x = quant.synthetic_bf16(m, k, name=f"fx{fmt}")
    r = quant.synthetic_bf16(m, n, name=f"fr{fmt}")
    y, mag = oracle.gemv(p, x, r)
    xf = [[Fraction(float(v)) for v in oracle.bf16(x[i])] for i in range(m)]
    rf = [[Fraction(float(v)) for v in oracle.bf16(r[i])] for i in range(m)]
    for i in range(m):
        for j in range(n):
            exact = sum(_frac_value(p, 0, j, kk) * xf[i][kk] for kk in range(k)) + rf[i][j]
            absmag = sum(abs(_frac_value(p, 0, j, kk) * xf[i][kk]) for kk in range(k)) + abs(rf[i][j])
            assert abs(Fraction(y[i, j]) - exact) <= absmag * Fraction(1, 2 ** 40)
            assert abs(Fraction(mag[i, j]) - absmag) <= absmag * Fraction(1, 2 ** 40)


def test_dequant_exact_rationals_every_element():
    for fmt, k in [(F.AFFINE4_G64, 128), (F.MXFP4, 64), (F.NVFP4, 32), (F.Q6_K, 256)]:
        p = quant.synthetic_weight(fmt, 2, k, name=f"dq{fmt}")
        p.codes[:] = rng.randint_bytes(3, f"dq{fmt}", p.codes.size).reshape(p.codes.shape)
        w = oracle.dequant(p)
        for n in range(2):
            for kk in range(k):
                assert Fraction(w[n, kk]) == _frac_value(p, 0, n, kk)


# ------------------------------------------------------------ integer arithmetic

def _unit_scale(fmt, n, k, codes, codes_hi=None):
    p = F.empty(fmt, n, k)
    p.codes[0] = codes
    if fmt == F.AFFINE4_G64:
        p.scales[0, ..., 0] = 1.0
        p.scales[0, ..., 1] = -8.0
    elif fmt == F.MXFP4:
        p.scales[:] = 127
    elif fmt == F.NVFP4:
        p.scales[:] = 0x38
        p.tensor_scale[:] = 1.0
    else:
        p.codes_hi[0] = codes_hi
        p.scales[:] = 1
        p.scales2[:] = np.float16(2.0 ** -6)
    return p


@pytest.mark.parametrize("fmt", [F.AFFINE4_G64, F.MXFP4, F.NVFP4, F.Q6_K])
def test_exact_arithmetic_integer_route(fmt):
    n, k, m = 16, 512, 3
    codes = rng.randint_bytes(5, "ea", n * k // 2).reshape(n, k // 2)
    hi = rng.randint_bytes(6, "eah", n * k // 4).reshape(n, k // 4)
    p = _unit_scale(fmt, n, k, codes, hi)
    xi = rng.randint_bytes(7, "eax", m * k, 0, 9).astype(np.int64).reshape(m, k) - 4
    xb = quant.bf16_bits(xi.astype(np.float64))
    lo = np.stack([codes & 15, codes >> 4], -1).reshape(n, k).astype(np.int64)
    if fmt == F.AFFINE4_G64:
        wi, den = lo - 8, 1
    elif fmt in (F.MXFP4, F.NVFP4):
        twice = np.array([0, 1, 2, 3, 4, 6, 8, 12])           # 2 x the printed magnitudes
        wi, den = np.where(lo & 8, -1, 1) * twice[lo & 7], 2
    else:
        h = np.stack([(hi >> (2 * i)) & 3 for i in range(4)], -1).reshape(n, k).astype(np.int64)
        wi, den = (lo | (h << 4)) - 32, 64
    exact = xi @ wi.T
    y, _ = oracle.gemv(p, xb)
    assert np.array_equal(y * den, exact.astype(np.float64))


@pytest.mark.parametrize("fmt", [F.AFFINE4_G64, F.MXFP4, F.NVFP4, F.Q6_K])
def test_one_hot_block_addressing(fmt):
    n, k = 3, 512
    blk = F.BLOCK[fmt]
    x = quant.synthetic_bf16(2, k, name="oh")
    xf = oracle.bf16(x)
    for row in range(n):
        for b in range(k // blk):
            p = F.empty(fmt, n, k)
            if fmt == F.AFFINE4_G64:
                p.scales[0, row, b] = (2.0, 0.5)     # w = 2 q + 0.5 in the hot block only
            elif fmt == F.MXFP4:
                p.scales[0, row, b] = 128            # scale 2 in the hot block
            elif fmt == F.NVFP4:
                p.scales[0, row, b] = 0x40           # scale 2
            else:
                p.codes[:] = 0x00
                p.codes_hi[:] = 0xAA                 # q = 32 everywhere -> w = 0
                p.scales2[0, row, b] = np.float16(1.0)
                p.scales[0, row, b * 16:(b + 1) * 16] = 2
            lo, hi = b * blk, (b + 1) * blk
            kk = np.arange(lo, hi)
            qv = (kk * 5 + 1) % 8                     # codes 0..7 (E2M1: positive values)
            for t, q in zip(kk, qv):
                byte = p.codes[0, row, t // 2]
                p.codes[0, row, t // 2] = (byte & ~(15 << (4 * (t % 2)))) | (q << (4 * (t % 2)))
            w = oracle.dequant(p)
            y, _ = oracle.gemv(p, x)
            if fmt == F.AFFINE4_G64:
                val = 2.0 * qv + 0.5
            elif fmt in (F.MXFP4, F.NVFP4):
                val = 2.0 * np.array([0, .5, 1, 1.5, 2, 3, 4, 6])[qv]
            else:
                val = 2.0 * ((qv | (2 << 4)) - 32.0)      # high bits 2 -> q = 32 + qv
            expect_w = np.zeros((n, k))
            expect_w[row, lo:hi] = val
            assert np.array_equal(w, expect_w), (row, b)
            assert np.allclose(y[:, row], xf[:, lo:hi] @ val, rtol=1e-13, atol=0)
            others = [r for r in range(n) if r != row]
            assert np.all(y[:, others] == 0)


# ------------------------------------------------------------ routing

def test_routing_statistics_against_printed_values():
    """The oracle router on N(0, 1) logits reproduces the routing statistics
    the pages print: ten slots per token, 160 rows per expert at 8192 tokens,
    and about 39 distinct experts in a 4-token call (expectation
    512 (1 - (1 - 10/512)^4) = 38.84)."""
    g = {r[0]: int(r[1]) for r in _golden("routing.txt")}
    E, k = g["experts"], g["topk"]
    lg = routing.router_logits(g["tokens_prefill"], E)
    ids, w = oracle.router(lg, k)
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.sum() == g["tokens_prefill"] * k
    assert counts.mean() == g["mean_tokens_per_expert"]
    assert np.allclose(w.sum(1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.all([len(set(r)) == k for r in ids[:200]])
    dist = []
    for s in range(400):
        ids4, _ = oracle.router(routing.router_logits(g["tokens_decode"], E, seed=1000 + s,
                                                      name="r4"), k)
        dist.append(len(np.unique(ids4)))
    expect = E * (1 - (1 - k / E) ** g["tokens_decode"])
    assert abs(expect - 38.84) < 0.01
    assert abs(np.mean(dist) - expect) < 0.15
    assert round(np.mean(dist)) == g["mean_distinct_synthetic"]
    assert ids4.size == g["slots_decode"]


def test_random_routing_generator_is_valid():
    """The parity tests' routing generator: k distinct ids in range per
    token, every expert about equally often, weights positive summing to 1."""
    ids, w = routing.random_routing(8192, 512, 10, name="pin/rr")
    assert ids.dtype == np.int32 and w.dtype == np.float32
    assert ((ids >= 0) & (ids < 512)).all()
    assert all(len(set(r)) == 10 for r in ids)
    c = np.bincount(ids.ravel(), minlength=512)
    assert c.sum() == 81920 and c.min() > 100 and c.max() < 230
    assert (w > 0).all() and np.allclose(w.sum(1), 1.0, atol=1e-6)
    ids1, _ = routing.random_routing(3, 5, 5, name="pin/rr5")
    assert (np.sort(ids1, 1) == np.arange(5)).all()


def test_topk_softmax_equals_full_softmax_renormalised():
    lg = routing.router_logits(64, 512, name="sm")
    ids, w = oracle.router(lg, 10)
    full = np.exp(lg.astype(np.float64) - lg.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, ids, 1)
    assert np.allclose(sel / sel.sum(1, keepdims=True), w, rtol=1e-12)


# ------------------------------------------------------------ SwiGLU and MoE

def test_silu_closed_forms():
    g = np.linspace(-30, 30, 601)
    s = oracle.silu(g)
    assert s[300] == 0.0
    assert np.allclose(s - oracle.silu(-g), g, rtol=0, atol=1e-12)   # x s(x) + x s(-x) = x
    assert np.allclose(s[-1], 30.0, rtol=1e-12) and abs(s[0]) < 1e-11


# E2M1 code of each value used below (sign in bit 3)
_E2M1_CODE = {0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}


def _e2m1_code(v):
    return _E2M1_CODE[abs(v)] | (8 if v < 0 else 0)


def _bf16_bits_by_torch(v):
    """float64 -> float32 (struct, round to nearest) -> bfloat16 bits (torch)."""
    import struct
    f32 = struct.unpack("<f", struct.pack("<f", v))[0]
    return int(torch.tensor([f32], dtype=torch.float32).to(torch.bfloat16)
               .view(torch.int16).item()) & 0xFFFF


def test_moe_swiglu_wiring_hand_built_expert():
    """One hand-built MXFP4 expert with unit scales and a one-hot input, so
    that every gate and up sum is a known exact value: gate row i holds a_i
    and up row I + i holds b_i at column 0, x is 1 at column 0 and 0
    elsewhere.  Then h_i = bf16(f32(silu(a_i) * b_i)) with silu(g) =
    g / (1 + e^-g) ("TurboEXL3" section 4.1: SwiGLU in 32-bit between the
    gate/up and down multiplies), computed here with math.exp, struct and
    torch rounding.  The down matrix is a one-hot identity on the first I
    outputs, so y_j = w * h_j exactly.  A gate/up swap, a missing or extra
    rounding of h, or a wrong combine weight fails."""
    import math
    inter, H = 32, 128
    pairs = [(1.0, 3.0), (-2.0, 1.5), (0.5, -4.0), (6.0, 0.5), (-1.0, -3.0), (3.0, 2.0),
             (1.5, -6.0), (-0.5, 4.0)]
    gu = F.empty(F.MXFP4, 2 * inter, H, 1)
    gu.scales[:] = 127                                      # E8M0 1.0
    q = np.zeros((2 * inter, H), np.uint8)
    for i, (a, b) in enumerate(pairs):
        q[i, 0] = _e2m1_code(a)
        q[inter + i, 0] = _e2m1_code(b)
    gu.codes[0] = F.pack_nibbles(q)
    dn = F.empty(F.MXFP4, H, inter, 1)
    dn.scales[:] = 127
    qd = np.zeros((H, inter), np.uint8)
    for j in range(inter):
        qd[j, j] = _e2m1_code(1.0)
    dn.codes[0] = F.pack_nibbles(qd)
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = 0x3F80                                        # 1.0
    ids = np.zeros((1, 1), np.int32)
    wt = np.array([[0.5]], np.float32)
    y, _, hs = oracle.moe(gu, dn, x, ids, wt, num_routed=1, num_shared=0)
    h = np.asarray(hs[(0, 0)])
    for i in range(inter):
        a, b = pairs[i] if i < len(pairs) else (0.0, 0.0)
        expect = _bf16_bits_by_torch(a / (1.0 + math.exp(-a)) * b)
        assert int(h[i]) == expect, (i, hex(int(h[i])), hex(expect))
        hv = float(torch.tensor([expect], dtype=torch.int32).to(torch.int16)
                   .view(torch.bfloat16).float().item())
        assert y[0, i] == 0.5 * hv
    assert (y[0, inter:] == 0).all()
    # the swapped wiring would give different values for every pair above,
    # and h is not representable in bfloat16 before its rounding
    import struct
    for a, b in pairs:
        f32 = struct.unpack("<f", struct.pack("<f", a / (1 + math.exp(-a)) * b))[0]
        assert struct.unpack("<I", struct.pack("<f", f32))[0] & 0xFFFF != 0
        assert _bf16_bits_by_torch(a / (1 + math.exp(-a)) * b) != \
            _bf16_bits_by_torch(b / (1 + math.exp(-b)) * a)


def test_moe_single_expert_reduces_to_two_gemvs():
    H, inter, T = 256, 64, 5
    gu = quant.synthetic_weight(F.NVFP4, 2 * inter, H, name="mgu")
    dn = quant.synthetic_weight(F.NVFP4, H, inter, name="mdn")
    x = quant.synthetic_bf16(T, H, name="mx")
    ids = np.zeros((T, 1), np.int32)
    w = np.ones((T, 1), np.float32)
    y, mag, hs = oracle.moe(gu, dn, x, ids, w, num_routed=1, num_shared=0)
    g_u, _ = oracle.gemv(gu, x)                             # [T][2I]
    h32 = (oracle.silu(g_u[:, :inter]) * g_u[:, inter:]).astype(np.float32)
    hb = oracle.bf16_round(h32)
    y2, mag2 = oracle.gemv(dn, hb)
    assert np.array_equal(y, y2)
    assert np.array_equal(mag, mag2)


def test_moe_shared_expert_and_weights_linear():
    H, inter, T, E = 128, 32, 3, 4
    gu = quant.synthetic_weight(F.NVFP4, 2 * inter, H, batch=E + 1, name="lgu")
    dn = quant.synthetic_weight(F.NVFP4, H, inter, batch=E + 1, name="ldn")
    x = quant.synthetic_bf16(T, H, name="lx")
    ids, w = routing.random_routing(T, E, 2, name="lr")
    y, _, hs = oracle.moe(gu, dn, x, ids, w, E, 1)
    # recompose by hand from the per-slot outputs
    for t in range(T):
        acc = np.zeros(H)
        for j in range(2):
            d = oracle.dequant(dn, int(ids[t, j])) @ oracle.bf16(hs[(t, j)])
            acc += float(w[t, j]) * d
        acc += oracle.dequant(dn, E) @ oracle.bf16(hs[(t, 2)])
        assert np.allclose(y[t], acc, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ encoder sanity

@pytest.mark.parametrize("fmt", [F.AFFINE4_G64, F.MXFP4, F.NVFP4, F.Q6_K])
def test_encoder_round_trip_error(fmt):
    n, k = 8, 1024
    w = rng.normal_matrix(1, "rt", n, k, 0.02)
    p = quant.quantize(fmt, w)
    err = np.abs(oracle.dequant(p) - w)
    if fmt == F.AFFINE4_G64:
        s = np.repeat(oracle.fp16(p.scales[0, ..., 0]), 64, axis=-1)
        assert np.all(err <= 0.5 * s + 2e-6)
    elif fmt == F.Q6_K:
        step = np.repeat(oracle.fp16(p.scales2[0]), 256, -1) * np.repeat(p.scales[0].astype(float), 16, -1)
        assert np.all(err <= 0.5 * step + 1e-3 * np.abs(w) + 1e-7)
    else:
        rel = err / np.maximum(np.abs(w), 1e-30)
        # E2M1 spacing is at most a third of the value above 1.5 and at most
        # 0.5 below; with block scaling the error stays below half a step
        amax_blk = np.repeat(np.abs(w.reshape(n, -1, F.BLOCK[fmt])).max(-1), F.BLOCK[fmt], -1)
        assert np.all(err <= amax_blk * (0.25 if fmt == F.NVFP4 else 0.35))
        assert np.median(rel) < 0.2


def test_bf16_half_ulp_closed_form():
    v = np.array([1.0, 1.5, 2.0, 3.99, 0.75, -6.0, 2.0 ** -20])
    ulp = np.array([2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -8, 2.0 ** -5, 2.0 ** -27])
    assert np.array_equal(oracle.bf16_half_ulp(v), ulp / 2)
    # one ulp step of bf16 around 1.0 is 2^-7
    assert oracle.bf16(np.uint16(0x3F81)) - 1.0 == 2.0 ** -7


def test_moe_grouping_hand_worked_example():
    """Three tokens, top-2 of 3 routed experts plus one shared expert; the
    table is worked by hand: expert 0 gets tokens 0 and 2, expert 1 token 1,
    expert 2 tokens 0, 1, 2, the shared expert all three."""
    ids = np.array([[2, 0], [2, 1], [0, 2]])
    g = oracle.moe_grouping(ids, 3, 1)
    assert g["counts"].tolist() == [2, 1, 3, 3]
    assert g["offsets"].tolist() == [0, 2, 3, 6, 9]
    assert g["active"].tolist() == [0, 1, 2, 3]
    assert g["tiles"].tolist() == [[0, 0, 2], [1, 2, 1], [2, 3, 3], [3, 6, 3]]
    assert g["err"] == 0
    # tiles of 2 rows split expert 2's three rows into 2 + 1
    g2 = oracle.moe_grouping(ids, 3, 0, tile_rows=2)
    assert g2["tiles"].tolist() == [[0, 0, 2], [1, 2, 1], [2, 3, 2], [2, 5, 1]]
    # an id outside [0, E) is dropped and flagged; an unused expert has no tile
    g3 = oracle.moe_grouping(np.array([[1, 7], [-1, 1]]), 3, 0)
    assert g3["counts"].tolist() == [0, 2, 0]
    assert g3["valid"].tolist() == [[True, False], [False, True]]
    assert g3["active"].tolist() == [1]
    assert g3["tiles"].tolist() == [[1, 0, 2]]
    assert g3["err"] == 1


def test_moe_grouping_invariants_at_prefill_size():
    """8192 tokens, top-10 of 512: the counts add to the slot total, the mean
    is the 160 rows per expert the pages derive ("TurboEXL3" section 3.1),
    every tile lies inside its expert's rows and the tiles cover them once."""
    ids, _ = routing.random_routing(8192, 512, 10, name="pin/group")
    g = oracle.moe_grouping(ids, 512, 1)
    c = g["counts"]
    assert c[:512].sum() == 81920 and c[512] == 8192
    assert c[:512].mean() == 160
    assert np.array_equal(np.bincount(ids.ravel(), minlength=512), c[:512])
    covered = np.zeros(g["offsets"][-1], np.int64)
    for e, r0, rows in g["tiles"]:
        assert 1 <= rows <= 128
        assert g["offsets"][e] <= r0 and r0 + rows <= g["offsets"][e + 1]
        covered[r0:r0 + rows] += 1
    assert (covered == 1).all()
    assert len(g["tiles"]) == int(np.sum((c + 127) // 128))


# ------------------------------------------------------------ router

def test_router_equal_logits_closed_form():
    """All logits equal: the k lowest ids, each with weight exactly 1/k."""
    ids, w = oracle.router(np.full((3, 16), 0.75, np.float32), 4)
    assert (ids == np.arange(4)).all()
    assert (w == 0.25).all()


def test_router_single_expert_weight_one():
    lg = rng.normal_matrix(rng.BASE_SEED, "pin/router1", 5, 40, 1.0).astype(np.float32)
    ids, w = oracle.router(lg, 1)
    assert (ids[:, 0] == np.argmax(lg, axis=1)).all()
    assert (w == 1.0).all()


def test_router_ties_and_signed_zero():
    ids, w = oracle.router(np.array([[1.0, 3.0, 3.0, 2.0], [0.0, -0.0, 0.0, -1.0]], np.float32), 2)
    assert ids.tolist() == [[1, 2], [0, 1]]
    assert (w == 0.5).all()


def test_router_brute_force_and_library_softmax():
    """The chosen set is the k-subset with the largest logit sum (brute force
    over all subsets, distinct logits); the weights are scipy's softmax over
    all experts renormalised over the chosen ones; the order is descending."""
    from itertools import combinations

    from scipy.special import softmax
    lg = rng.normal_matrix(rng.BASE_SEED, "pin/router_bf", 6, 9, 1.0).astype(np.float32)
    ids, w = oracle.router(lg, 3)
    for t in range(lg.shape[0]):
        row = lg[t].astype(np.float64)
        best = max(combinations(range(9), 3), key=lambda c: sum(row[list(c)]))
        assert sorted(ids[t].tolist()) == sorted(best)
        assert (np.diff(row[ids[t]]) <= 0).all()
        p = softmax(row)
        np.testing.assert_allclose(w[t], p[ids[t]] / p[ids[t]].sum(), rtol=1e-14)


def test_router_shift_invariant():
    lg = rng.normal_matrix(rng.BASE_SEED, "pin/router_sh", 4, 64, 1.0)
    ids0, w0 = oracle.router(lg, 10)
    ids1, w1 = oracle.router(lg + 7.5, 10)
    assert (ids0 == ids1).all()
    np.testing.assert_allclose(w0, w1, rtol=1e-12)


# ------------------------------------------------------------ W4A4

def _bf16_bits_of(tok):
    if tok.startswith("0x"):
        return int(tok, 16)
    return int(torch.tensor([float(tok)], dtype=torch.float32).to(torch.bfloat16)
               .view(torch.int16).item()) & 0xFFFF


def test_mxfp4_activation_quantizer_hand_worked_blocks():
    """Blocks worked by hand from the MXFP4 conversion rule
    (tests/golden/w4a4_blocks.txt): shared exponent, ties to even,
    saturation, zero blocks, subnormal and huge inputs."""
    rows = []
    with open(os.path.join(GOLDEN, "w4a4_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    x = np.zeros((1, 32 * len(rows)), np.uint16)
    expect_s, expect_c = [], np.zeros(32 * len(rows), np.int64)
    for b, line in enumerate(rows):
        left, right = line.split("|")
        tok = left.split()
        expect_s.append(int(tok[1]))
        vals = [_bf16_bits_of(t) for t in tok[2:]]
        x[0, 32 * b:32 * b + len(vals)] = vals
        codes = [int(c) for c in right.split()]
        expect_c[32 * b:32 * b + len(codes)] = codes
    codes, scales = oracle.mxfp4_quantize(x)
    assert scales[0].tolist() == expect_s
    got = np.stack([codes[0] & 15, codes[0] >> 4], axis=-1).reshape(-1)
    assert got.tolist() == expect_c.tolist()


def test_w4a4_equals_w4a16_on_grid_activations():
    """Activations already on the MXFP4 grid (each block's largest magnitude
    6 * 2^E, every value an E2M1 magnitude times 2^E) are quantized without
    loss, so W4A4 equals the W4A16 product on them, bit for bit in float64."""
    n, k, m = 24, 256, 3
    p = quant.synthetic_weight(F.MXFP4, n, k, name="pin/w4a4w")
    codes = rng.randint_bytes(rng.BASE_SEED, "pin/w4a4c", m * k, 0, 16).astype(np.int64)
    mags = np.asarray(oracle.E2M1_MAGNITUDES)
    v = np.where(codes & 8, -1.0, 1.0) * mags[codes & 7]
    v = v.reshape(m, k // 32, 32)
    v[..., 0] = 6.0                                    # amax 6 in every block
    ex = rng.randint_bytes(rng.BASE_SEED, "pin/w4a4e", m * k // 32, 0, 9).astype(np.int64) - 4
    x = (v * np.ldexp(1.0, ex).reshape(m, k // 32, 1)).reshape(m, k)
    xb = quant.bf16_bits(x)
    assert np.array_equal(oracle.bf16(xb), x)          # exact in bf16
    y4, mag4 = oracle.gemm_w4a4(p, xb)
    y16, mag16 = oracle.gemv(p, xb)
    assert np.array_equal(y4, y16) and np.array_equal(mag4, mag16)
    c, sc = oracle.mxfp4_quantize(xb)
    assert (sc.astype(np.int64) == ex.reshape(m, k // 32) + 127 - 0).all()


def test_w4a4_is_w4a16_on_the_dequantized_activations():
    """For any activations, the W4A4 product is the W4A16 product on the
    dequantized MXFP4 activations (exactly representable in bf16: 3
    significant bits)."""
    n, k, m = 40, 512, 5
    p = quant.synthetic_weight(F.MXFP4, n, k, outlier_rate=0.01, name="pin/w4a4b")
    xb = quant.synthetic_bf16(m, k, name="pin/w4a4x")
    codes, scales = oracle.mxfp4_quantize(xb)
    xq = oracle.mxfp4_dequantize_activations(codes, scales)
    xqb = quant.bf16_bits(xq)
    assert np.array_equal(oracle.bf16(xqb), xq)
    y4, mag4 = oracle.gemm_w4a4(p, xb)
    y16, mag16 = oracle.gemv(p, xqb)
    assert np.array_equal(y4, y16) and np.array_equal(mag4, mag16)


def test_mxfp4_quantizer_error_bound_and_scale():
    """Every value lands within half a grid step of its scaled value (the
    grid step at |v| is .5 below 2, 1 from 2 to 4, 2 from 4 to 6), the block
    maximum within [4, 8) after scaling, and saturation only above 6."""
    xb = quant.synthetic_bf16(16, 1024, name="pin/w4a4err", std=3.0)
    codes, scales = oracle.mxfp4_quantize(xb)
    x = oracle.bf16(xb).reshape(16, 32, 32)
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    v = x / sc
    q = oracle.mxfp4_dequantize_activations(codes, scales).reshape(16, 32, 32) / sc
    a = np.abs(v)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    assert (np.abs(q - v) <= step / 2 + 1e-12)[a <= 6].all()
    assert (np.abs(q)[a > 6] == 6).all()
    amax = a.max(-1)
    assert ((amax >= 4) & (amax < 8)).all()


# ------------------------------------------------------------ Hadamard stages

def test_sylvester_hadamard_is_the_library_matrix():
    """The oracle's H_128 is scipy's Hadamard matrix (Sylvester's
    construction) and H H^T = 128 I."""
    from scipy.linalg import hadamard
    h = oracle.sylvester_hadamard(128)
    assert np.array_equal(h, hadamard(128))
    assert np.array_equal(h @ h.T, 128 * np.eye(128))


def test_hadamard_prepare_closed_forms():
    """A one-hot block gives column j of H / sqrt(128) (entries +-2^-3.5) times
    the channel scale; a constant block gives sqrt(128) c at index 0 and zero
    elsewhere; blocks are independent; the transform preserves the norm."""
    from scipy.linalg import hadamard
    k = 256
    x = np.zeros((3, k))
    x[0, 5] = 1.0                  # one-hot in block 0
    x[1, 128:] = 0.5               # constant block 1
    x[2, 130] = -2.0
    s = np.ones(k, np.float16)
    s[5] = -1.0                    # a negative scale flips the sign
    y, _, _ = oracle.hadamard_prepare(quant.bf16_bits(x), s.view(np.uint16))
    np.testing.assert_allclose(y[0, :128], -hadamard(128)[:, 5] / np.sqrt(128), rtol=1e-15)
    assert (y[0, 128:] == 0).all()
    np.testing.assert_allclose(y[1, 128], 0.5 * np.sqrt(128), rtol=1e-15)
    assert np.abs(y[1, 129:]).max() < 1e-15 and (y[1, :128] == 0).all()
    np.testing.assert_allclose(y[2, 128:], -2.0 * hadamard(128)[:, 2] / np.sqrt(128), rtol=1e-15)
    xr = quant.synthetic_bf16(4, 512, name="pin/had")
    yr, _, _ = oracle.hadamard_prepare(xr)
    xb = oracle.bf16(xr).reshape(4, 4, 128)
    np.testing.assert_allclose(np.linalg.norm(yr.reshape(4, 4, 128), axis=-1),
                               np.linalg.norm(xb, axis=-1), rtol=1e-12)


def test_hadamard_finish_inverts_prepare():
    """H / sqrt(128) is symmetric and orthogonal, so finish (unit scales)
    applied to prepare's exact output returns the scaled input; with scales
    the finish multiplies after the transform."""
    x = quant.synthetic_bf16(3, 384, name="pin/had2")
    s = (rng.uniform_matrix(rng.BASE_SEED, "pin/hads", 1, 384)[0] * 2 - 1).astype(np.float16)
    y, _, _ = oracle.hadamard_prepare(x, s.view(np.uint16))
    back, _ = oracle.hadamard_finish(y)
    np.testing.assert_allclose(back, oracle.bf16(x) * s.astype(np.float64), rtol=1e-12, atol=1e-12)
    out, mag = oracle.hadamard_finish(y, s.view(np.uint16))
    np.testing.assert_allclose(out, back * s.astype(np.float64), rtol=1e-15)
    assert (mag >= np.abs(out) - 1e-12).all()
