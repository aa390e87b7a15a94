"""GPU parity of the W4A4 path (MXFP4 weights x activations quantized to MXFP4
on the fly, FP4 x FP4 on the block-scaled matrix cores) against the CPU
oracle, through the C ABI.

Bars: the activation quantizer bit-exact (codes and E8M0 scales); products
|y - y_ref| <= 2e-3 * sum|w||q(x)| + half a bf16 ulp of y_ref per output (y
is stored as bf16); exact-arithmetic inputs give exactly the bf16 rounding of
the exact sum; repeated calls bitwise identical."""

import numpy as np
import pytest
import torch

import oracle
from synth import formats as F
from synth import quant, rng

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _q():
    import gemm_dequant_gemv_amd as q
    return q


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).cuda()


def _host_f64(t):
    return oracle.bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))


def _check(y, yref, mag):
    ok = oracle.within_tolerance_bf16(y, yref, mag, TOL)
    assert ok.all(), (f"{(~ok).sum()} of {ok.size} outside tolerance; worst "
                      f"{np.max(np.abs(y - yref) / np.maximum(mag, 1e-30)):.3e} of mag")


def _edge_activations(m, k, seed):
    """bf16 activations with every kind of block: N(0, 1) and N(0, 1000)
    values, all-zero blocks, blocks of bf16 subnormals, huge values, signed
    zeros and values exactly on the E2M1 decision points."""
    x = quant.synthetic_bf16(m, k, name=f"w4e{seed}").copy()
    big = quant.synthetic_bf16(m, k, name=f"w4b{seed}", std=1000.0)
    blk = x.reshape(m, k // 32, 32)
    bigb = big.reshape(m, k // 32, 32)
    kind = rng.randint_bytes(seed, "w4kind", m * (k // 32), 0, 6).reshape(m, k // 32)
    sub = rng.randint_bytes(seed, "w4sub", m * k, 0, 128).astype(np.uint16).reshape(m, k // 32, 32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float64)
    for i in range(m):
        for b in range(k // 32):
            if kind[i, b] == 1:
                blk[i, b] = bigb[i, b]
            elif kind[i, b] == 2:
                blk[i, b] = 0
            elif kind[i, b] == 3:
                blk[i, b] = sub[i, b] | (sub[i, b] & 1) << 15   # subnormals, both signs
            elif kind[i, b] == 4:
                blk[i, b] = 0x7B80 ^ (sub[i, b] & 0x8000)       # 2^120
                blk[i, b, :8] = 0x8000                          # -0
            elif kind[i, b] == 5:
                # points on the E2M1 decision thresholds after scaling by 2^-E:
                # amax 6 gives E = 0
                vals = np.resize(ties, 32) * np.where(np.arange(32) % 3 == 0, -1, 1)
                blk[i, b] = quant.bf16_bits(vals)
    return x


@pytest.mark.parametrize("m,k", [(1, 128), (7, 512), (64, 2048), (3, 5120)])
def test_quant_mxfp4_bit_exact(m, k):
    q = _q()
    x = _edge_activations(m, k, 11 + m)
    codes, scales = q.quant_mxfp4(_dev_bf16(x))
    rc, rs = oracle.mxfp4_quantize(x)
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quant_mxfp4_argument_errors():
    q = _q()
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")   # k not a multiple of 32
    with pytest.raises(q.QmmError) as e:
        q.quant_mxfp4(x)
    assert e.value.status == -3


# several 256 x 256 tiles with ragged m and n, residual on even m
# K a multiple of 256 takes 256-wide K slices, the others (384, 1408) 128-wide ones
SHAPES = [(1, 64, 256), (130, 300, 768), (257, 515, 1024), (256, 256, 512), (77, 1000, 2304),
          (33, 200, 384), (300, 520, 1408)]


@pytest.mark.parametrize("shape", SHAPES)
def test_gemm_w4a4_parity(shape):
    m, n, k = shape
    q = _q()
    p = quant.synthetic_weight(F.MXFP4, n, k, outlier_rate=0.01, name=f"w4w{n}{k}")
    x = quant.synthetic_bf16(m, k, name=f"w4x{m}{k}")
    r = quant.synthetic_bf16(m, n, name=f"w4r{m}{n}") if m % 2 == 0 else None
    w = q.Weight.from_host(p)
    xd = _dev_bf16(x)
    rd = None if r is None else _dev_bf16(r)
    y = q.gemm_w4a4(w, xd, rd)
    y2 = q.gemm_w4a4(w, xd, rd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    yref, mag = oracle.gemm_w4a4(p, x, r)
    _check(_host_f64(y), yref, mag)


def test_gemm_w4a4_exact_arithmetic():
    """Unit E8M0 weight scales and activations already on the MXFP4 grid with
    small exponents: every product and partial sum is exact in float32, so the
    output is exactly the bf16 rounding of the exact sum."""
    q = _q()
    m, n, k = 96, 300, 5120
    p = F.empty(F.MXFP4, n, k)
    p.codes[:] = rng.randint_bytes(41, "w4xc", p.codes.size).reshape(p.codes.shape)
    p.scales[:] = 127
    codes = rng.randint_bytes(42, "w4xa", m * k, 0, 16).astype(np.int64)
    mags = np.asarray(oracle.E2M1_MAGNITUDES)
    v = (np.where(codes & 8, -1.0, 1.0) * mags[codes & 7]).reshape(m, k // 32, 32)
    v[..., 0] = 6.0
    ex = rng.randint_bytes(43, "w4xe", m * (k // 32), 0, 3).astype(np.int64) - 1
    x = quant.bf16_bits((v * np.ldexp(1.0, ex).reshape(m, k // 32, 1)).reshape(m, k))
    w = q.Weight.from_host(p)
    y = q.gemm_w4a4(w, _dev_bf16(x)).view(torch.int16).cpu().numpy().view(np.uint16)
    yref, _ = oracle.gemm_w4a4(p, x)
    assert np.array_equal(y, oracle.bf16_round(yref.astype(np.float32)))


def test_gemm_w4a4_rejects():
    q = _q()
    p = quant.synthetic_weight(F.NVFP4, 64, 256, name="w4rej")
    w = q.Weight.from_host(p)
    x = _dev_bf16(quant.synthetic_bf16(4, 256, name="w4rejx"))
    with pytest.raises(q.QmmError) as e:
        q.gemm_w4a4(w, x, workspace=torch.empty(4096, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -2          # W4A4 takes MXFP4 weights
    pm = quant.synthetic_weight(F.MXFP4, 64, 256, name="w4rej2")
    wm = q.Weight.from_host(pm)
    with pytest.raises(q.QmmError) as e:
        q.gemm_w4a4(wm, x, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -6          # workspace too small


# The prefill workload's weight, 17408 x 5120 MXFP4, at the sizes the
# benchmark times (and M = 1024 and 1000, whose last round of 256 x 256 tiles
# runs as 64-row tiles, as at 2048; 1000 leaves the last of them ragged): the
# GPU computes every output, the oracle checks sampled activation rows (every
# output column of each), tile edges included.
@pytest.mark.parametrize("m", [128, 1000, 1024, 2048, 8192])
def test_gemm_w4a4_full_size_sampled(m):
    q = _q()
    n, k = 17408, 5120
    p = quant.synthetic_weight(F.MXFP4, n, k, name="w4full")
    x = quant.synthetic_bf16(m, k, name=f"w4fullx{m}")
    w = q.Weight.from_host(p)
    y = _host_f64(q.gemm_w4a4(w, _dev_bf16(x)))
    edges = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 959, 960, m // 2, m - 2, m - 1]
    rows = np.unique(np.concatenate([edges, rng.randint_bytes(73, f"w4fr{m}", 13, 0, 256)
                                     .astype(np.int64) * (m // 256)]))
    rows = rows[rows < m]
    yref, mag = oracle.gemm_w4a4(p, x[rows])
    _check(y[rows], yref, mag)
