"""GPU parity of qdequant and qgemv against the CPU oracle, through the C ABI.

Bars: dequantized weights bit-exact; products |y - y_ref| <= 2e-3 * sum|w||x|
per output; products of exact-arithmetic inputs bit-exact; repeated calls
bitwise identical."""

import numpy as np
import pytest
import torch

import oracle
from synth import formats as F
from synth import quant, rng

pytestmark = pytest.mark.gpu

FMTS = [F.AFFINE4_G64, F.MXFP4, F.NVFP4, F.Q6_K]
TOL = 2e-3


def _q():
    import gemm_dequant_gemv_amd as q
    return q


def _bits_f32(t):
    return t.cpu().numpy().view(np.uint32)


def _randomize_planes(p, seed):
    """Random bytes in every code and scale plane, so every code and scale
    value (including -0, NaN scales, subnormal and huge scales) occurs."""
    p.codes[:] = rng.randint_bytes(seed, "c", p.codes.size).reshape(p.codes.shape)
    if p.fmt == F.AFFINE4_G64:
        # random finite float16 scales and biases
        b = rng.randint_bytes(seed, "s", p.scales.size * 2).view(np.uint16)
        b = np.where((b & 0x7C00) == 0x7C00, b & 0xBFFF, b).astype(np.uint16)
        p.scales[:] = b.view(np.float16).reshape(p.scales.shape)
    elif p.fmt in (F.MXFP4, F.NVFP4):
        p.scales[:] = rng.randint_bytes(seed, "s", p.scales.size).reshape(p.scales.shape)
        if p.fmt == F.NVFP4:
            p.tensor_scale[:] = np.float32(0.37)
    else:
        p.codes_hi[:] = rng.randint_bytes(seed, "h", p.codes_hi.size).reshape(p.codes_hi.shape)
        p.scales[:] = rng.randint_bytes(seed, "s", p.scales.size).view(np.int8).reshape(p.scales.shape)
        d = rng.randint_bytes(seed, "d", p.scales2.size * 2).view(np.uint16)
        d = np.where((d & 0x7C00) == 0x7C00, d & 0xBFFF, d).astype(np.uint16)
        p.scales2[:] = d.view(np.float16).reshape(p.scales2.shape)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_bit_exact_random_planes(fmt):
    q = _q()
    k = 1024 if fmt == F.Q6_K else 512
    p = F.empty(fmt, 96, k, batch=2)
    _randomize_planes(p, 100 + fmt)
    w = q.Weight.from_host(p)
    out32 = q.dequant(w, torch.float32)
    out16 = q.dequant(w, torch.bfloat16)
    torch.cuda.synchronize()
    for e in range(2):
        with np.errstate(over="ignore", invalid="ignore"):
            ref32 = oracle.dequant_f32(p, e)
            ref16 = oracle.dequant_bf16(p, e)
        got32 = out32[e].cpu().numpy()
        nan = np.isnan(ref32)
        assert np.array_equal(np.isnan(got32), nan)
        assert np.array_equal(got32[~nan].view(np.uint32), ref32[~nan].view(np.uint32))
        got16 = out16[e].view(torch.int16).cpu().numpy().view(np.uint16)
        nan16 = (ref16 & 0x7FFF) > 0x7F80
        assert np.array_equal((got16 & 0x7FFF) > 0x7F80, nan16)
        assert np.array_equal(got16[~nan16], ref16[~nan16])


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_bit_exact_quantized_weights(fmt):
    q = _q()
    p = quant.synthetic_weight(fmt, 130, 2048, outlier_rate=0.01, name="dqw")
    w = q.Weight.from_host(p)
    got = q.dequant(w, torch.float32)[0].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.dequant_f32(p).view(np.uint32))


def _case(fmt, n, k, m, tag, outliers=0.0, residual=False):
    p = quant.synthetic_weight(fmt, n, k, outlier_rate=outliers, name=f"{tag}/W")
    x = quant.synthetic_bf16(m, k, name=f"{tag}/x")
    r = quant.synthetic_bf16(m, n, name=f"{tag}/r") if residual else None
    return p, x, r


def _to_dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _check_tol(y, yref, mag):
    ok = oracle.within_tolerance(y, yref, mag, TOL)
    assert ok.all(), (f"{(~ok).sum()} outputs outside tolerance; worst "
                      f"{np.max(np.abs(y - yref) / mag):.3e} of mag")


# Shapes with ragged row counts and ragged last K steps.  Up to K = 17408 the
# activations fit in LDS and the row-streaming kernel runs (no workspace);
# K = 81920 exceeds that at every M and takes the split-K kernel, whose
# workgroups finish split rows through the workspace.  (Q6_K at 4 rows of
# 17408 values fits only with the records' bank padding left out.)
SHAPES = [(300, 896), (257, 2304), (128, 256), (1, 512), (515, 4096), (64, 6144), (40, 17408),
          (40, 81920)]
SPLIT_K = 81920


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", SHAPES)
def test_gemv_parity(fmt, m, shape):
    n, k = shape
    if fmt == F.Q6_K:
        k = (k + 255) // 256 * 256
    q = _q()
    p, x, r = _case(fmt, n, k, m, f"gv{fmt}{n}{k}", outliers=0.01, residual=(n % 2 == 1))
    w = q.Weight.from_host(p)
    # the kernel choice shows in the workspace it asks for: split-K whenever
    # the activations do not fit in LDS, row-streaming otherwise
    if k == SPLIT_K:
        assert q.gemv_workspace_size(w, m) > 0
    else:
        assert q.gemv_workspace_size(w, m) == 0
    y = q.gemv(w, _to_dev_bf16(x), None if r is None else _to_dev_bf16(r))
    yref, mag = oracle.gemv(p, x, r)
    _check_tol(y.cpu().numpy().astype(np.float64), yref, mag)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_bf16_output(fmt):
    q = _q()
    k = 1024
    p, x, r = _case(fmt, 200, k, 2, f"gvb{fmt}", residual=True)
    w = q.Weight.from_host(p)
    y = q.gemv(w, _to_dev_bf16(x), _to_dev_bf16(r), y_dtype=torch.bfloat16)
    y32 = q.gemv(w, _to_dev_bf16(x), _to_dev_bf16(r), y_dtype=torch.float32)
    # the bf16 output is the float32 result rounded to nearest even
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.bf16_round(y32.cpu().numpy()))


def _unit_scale_weight(fmt, n, k, seed):
    p = F.empty(fmt, n, k)
    p.codes[:] = rng.randint_bytes(seed, "ec", p.codes.size).reshape(p.codes.shape)
    if fmt == F.AFFINE4_G64:
        p.scales[..., 0] = 1.0
        p.scales[..., 1] = -8.0
    elif fmt == F.MXFP4:
        p.scales[:] = 127
    elif fmt == F.NVFP4:
        p.scales[:] = 0x38
        p.tensor_scale[:] = 1.0
    else:
        p.codes_hi[:] = rng.randint_bytes(seed, "eh", p.codes_hi.size).reshape(p.codes_hi.shape)
        p.scales[:] = 1
        p.scales2[:] = np.float16(2.0 ** -6)
    return p


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 4])
@pytest.mark.parametrize("shape", [(300, 2048), (200, 17408), (129, 512), (40, SPLIT_K)])
def test_gemv_exact_arithmetic_bit_exact(fmt, m, shape):
    """Unit scales and integer activations make every product and partial sum
    an exact float32, so any summation order must give the oracle's value."""
    n, k = shape
    q = _q()
    p = _unit_scale_weight(fmt, n, k, 40 + fmt)
    xi = rng.randint_bytes(41, "ex", m * k, 0, 9).astype(np.float64).reshape(m, k) - 4
    x = quant.bf16_bits(xi)
    w = q.Weight.from_host(p)
    y = q.gemv(w, _to_dev_bf16(x)).cpu().numpy()
    yref, _ = oracle.gemv(p, x)
    assert np.array_equal(y.astype(np.float64), yref)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_one_hot_blocks(fmt):
    """Every code zero-valued except one block per row, at a different block
    position in each row: catches any block/scale addressing slip."""
    q = _q()
    n, k = 64, 2048
    blk = F.BLOCK[fmt]
    p = F.empty(fmt, n, k)
    if fmt == F.Q6_K:
        p.codes_hi[:] = 0xAA            # q = 32 -> zero weight
        p.scales2[:] = np.float16(1.0)
    nb = k // blk
    for row in range(n):
        b = (row * 7) % nb
        lo = b * blk
        vals = (np.arange(blk) * 3 + row) % 8
        bytes_ = p.codes[0, row]
        for t in range(blk):
            kk = lo + t
            bytes_[kk // 2] |= np.uint8(vals[t] << (4 * (kk % 2)))
        if fmt == F.AFFINE4_G64:
            p.scales[0, row, b] = (0.5, 0.25)
        elif fmt == F.MXFP4:
            p.scales[0, row, b] = 126
        elif fmt == F.NVFP4:
            p.scales[0, row, b] = 0x30
        else:
            p.scales[0, row, b * 16:(b + 1) * 16] = 3
    x = quant.synthetic_bf16(3, k, name="oh")
    w = q.Weight.from_host(p)
    y = q.gemv(w, _to_dev_bf16(x)).cpu().numpy().astype(np.float64)
    yref, mag = oracle.gemv(p, x)
    _check_tol(y, yref, mag)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_deterministic(fmt):
    q = _q()
    p, x, _ = _case(fmt, 1000, 5120, 4, f"det{fmt}")
    w = q.Weight.from_host(p)
    xd = _to_dev_bf16(x)
    ws = q.new_workspace(q.gemv_workspace_size(w, 4))
    ys = [q.gemv(w, xd, workspace=ws) for _ in range(3)]
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("fmt", [F.AFFINE4_G64, F.Q6_K])
def test_split_workspace_needs_no_zero_fill(fmt):
    """The split-K path on a workspace of 0xFF bytes, then on one whose bytes
    a qmoe_grouped call left behind (routing tables, h, d), then again on its
    own leftovers: every result meets the oracle's bar and all are bitwise
    equal (the call clears its own arrival counters)."""
    q = _q()
    p, x, r = _case(fmt, 515, SPLIT_K, 3, f"wsff{fmt}", residual=True)
    w = q.Weight.from_host(p)
    need = q.gemv_workspace_size(w, 3)
    assert need > 0
    xd, rd = _to_dev_bf16(x), _to_dev_bf16(r)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    y1 = q.gemv(w, xd, rd, workspace=ws)
    y2 = q.gemv(w, xd, rd, workspace=ws)
    # a workspace last used by an MoE layer
    from synth import routing
    E, S, H, inter, T, topk = 8, 1, 512, 128, 40, 2
    gu = q.Weight.from_host(quant.synthetic_weight(F.NVFP4, 2 * inter, H, batch=E + S, name="wsff/gu"))
    dn = q.Weight.from_host(quant.synthetic_weight(F.NVFP4, H, inter, batch=E + S, name="wsff/dn"))
    ids, wt = routing.random_routing(T, E, topk, name="wsff/r")
    mneed = q.moe_workspace_size(gu, dn, E, S, T, topk)
    wsm = torch.empty(max(mneed, need), dtype=torch.uint8, device="cuda")
    q.moe(gu, dn, _to_dev_bf16(quant.synthetic_bf16(T, H, name="wsff/x")),
          torch.from_numpy(ids).cuda(), torch.from_numpy(wt).cuda(), E, S, workspace=wsm[:mneed])
    y3 = q.gemv(w, xd, rd, workspace=wsm[:need])
    torch.cuda.synchronize()
    for y in (y2, y3):
        assert torch.equal(y1.view(torch.int32), y.view(torch.int32))
    yref, mag = oracle.gemv(p, x, r)
    _check_tol(y1.cpu().numpy().astype(np.float64), yref, mag)


def test_error_codes_before_launch():
    q = _q()
    p, x, _ = _case(F.AFFINE4_G64, 256, 1024, 1, "err")
    w = q.Weight.from_host(p)
    xd = _to_dev_bf16(x)
    with pytest.raises(q.QmmError) as e:
        q.gemv(w, torch.cat([xd] * 5))           # m = 5
    assert e.value.status == -5
    y = torch.empty((1, 256), device="cuda")
    ws_need = q.gemv_workspace_size(w, 1)
    if ws_need:
        small = torch.zeros(ws_need - 4, dtype=torch.uint8, device="cuda")
        with pytest.raises(q.QmmError) as e:
            q.gemv(w, xd, out=y, workspace=small)
        assert e.value.status == -6


# The decode matvecs at full size, as the benchmark launches them: every
# output is computed on the GPU, a sample of rows (spread over the matrix,
# including both ends) is checked against the oracle.
DECODE = [(F.AFFINE4_G64, 17408, 5120, False), (F.AFFINE4_G64, 5120, 17408, True),
          (F.Q6_K, 17408, 5120, False), (F.Q6_K, 5120, 17408, True),
          (F.MXFP4, 5120, 6144, False), (F.NVFP4, 5120, 5120, False),
          (F.MXFP4, 5120, 5120, False), (F.NVFP4, 5120, 6144, False)]


@pytest.fixture(scope="module")
def decode_weights():
    cache = {}

    def get(fmt, n, k):
        if (fmt, n, k) not in cache:
            cache[(fmt, n, k)] = quant.synthetic_weight(fmt, n, k, outlier_rate=0.01,
                                                        name=f"full{fmt}/{n}x{k}")
        return cache[(fmt, n, k)]
    return get


@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("case", DECODE)
def test_gemv_decode_full_size_sampled(decode_weights, case, m):
    fmt, n, k, res = case
    q = _q()
    p = decode_weights(fmt, n, k)
    x = quant.synthetic_bf16(m, k, name=f"fullx{m}/{k}")
    r = quant.synthetic_bf16(m, n, name=f"fullr{m}/{n}") if res else None
    w = q.Weight.from_host(p)
    y = q.gemv(w, _to_dev_bf16(x), None if r is None else _to_dev_bf16(r)).cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1],
                                     rng.randint_bytes(7, f"rows{n}", 60, 0, 256).astype(np.int64)
                                     * (n // 256) + 3]))
    yref, mag = oracle.gemv(p, x, r, rows=rows)
    _check_tol(y[:, rows].astype(np.float64), yref, mag)


def test_gemv_single_matvec_affine_1024():
    """The single-matvec configuration: affine 4-bit g64, W 1024 x 1024
    N(0, 0.02), x 1 x 1024 N(0, 1), float32 y; every output checked, and a
    second call is bitwise the same."""
    q = _q()
    p = quant.synthetic_weight(F.AFFINE4_G64, 1024, 1024, name="single/W")
    x = quant.synthetic_bf16(1, 1024, name="single/x")
    w = q.Weight.from_host(p)
    xd = _to_dev_bf16(x)
    y = q.gemv(w, xd)
    y2 = q.gemv(w, xd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    yref, mag = oracle.gemv(p, x)
    _check_tol(y.cpu().numpy().astype(np.float64), yref, mag)


# The FP4 output projection, 248320 x 5120 with 1% outliers at 8x, in the
# configuration the benchmark times, at every lane count: the GPU computes
# every output, the oracle checks rows spread over the whole matrix (both
# ends, and the last rows of the final workgroups).
@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", [F.MXFP4, F.NVFP4])
def test_gemv_output_projection_full_size_sampled(fmt):
    q = _q()
    n, k = 248320, 5120
    print(f"generating {F.NAMES[fmt]} {n}x{k}", flush=True)
    p = quant.synthetic_weight(fmt, n, k, outlier_rate=0.01, name=f"outproj{fmt}")
    w = q.Weight.from_host(p)
    rows = np.unique(np.concatenate([[0, 1, 2, 3, n // 2, n - 4, n - 3, n - 2, n - 1],
                                     rng.randint_bytes(9, f"oprows{fmt}", 55, 0, 256)
                                     .astype(np.int64) * (n // 256) + 5]))
    for m in (1, 2, 3, 4):
        x = quant.synthetic_bf16(m, k, name=f"outprojx{m}")
        y = q.gemv(w, _to_dev_bf16(x)).cpu().numpy()
        yref, mag = oracle.gemv(p, x, rows=rows)
        _check_tol(y[:, rows].astype(np.float64), yref, mag)
        print(f"  m={m} ok", flush=True)
