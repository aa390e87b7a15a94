"""GPU parity of qgemm (prefill: weights dequantized to bf16 inside the kernel,
bf16 MFMA) against the CPU oracle, through the C ABI.  The small shapes run
the 128- and 192-row tile configurations; the sampled full-size cases run
the prefill workload's own configurations.

Bars: |y - y_ref| <= 2e-3 * sum|w||x| + half a bf16 ulp of y_ref per output
(y is stored as bf16, which the reference rounds too); exact-arithmetic
inputs give exactly the bf16 rounding of the exact sum; repeated calls are
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


def _dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _host_f64(t):
    return oracle.bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))


def _check(y, yref, mag):
    ok = oracle.within_tolerance_bf16(y, yref, mag, TOL)
    assert ok.all(), (f"{(~ok).sum()} of {ok.size} outside tolerance; worst "
                      f"{np.max(np.abs(y - yref) / mag):.3e} of mag")


# several 128 x 128 tiles with ragged m and n, K granules of each format
SHAPES = [(130, 300, 768), (257, 129, 1024), (1, 64, 512), (128, 256, 256), (200, 1000, 2304)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", SHAPES)
def test_gemm_parity(fmt, shape):
    m, n, k = shape
    if fmt == F.Q6_K:
        k = (k + 255) // 256 * 256
    q = _q()
    p = quant.synthetic_weight(fmt, n, k, outlier_rate=0.01, name=f"gm{fmt}{n}{k}")
    x = quant.synthetic_bf16(m, k, name=f"gmx{m}{k}")
    r = quant.synthetic_bf16(m, n, name=f"gmr{m}{n}") if m % 2 == 0 else None
    w = q.Weight.from_host(p)
    y = q.gemm(w, _dev_bf16(x), None if r is None else _dev_bf16(r))
    yref, mag = oracle.gemm(p, x, r)
    _check(_host_f64(y), yref, mag)


def _unit_scale_weight(fmt, n, k, seed):
    p = F.empty(fmt, n, k)
    p.codes[:] = rng.randint_bytes(seed, "gec", p.codes.size).reshape(p.codes.shape)
    if fmt == F.AFFINE4_G64:
        p.scales[..., 0] = 1.0
        p.scales[..., 1] = -8.0
    elif fmt == F.MXFP4:
        p.scales[:] = 127
    elif fmt == F.NVFP4:
        p.scales[:] = 0x38
        p.tensor_scale[:] = 1.0
    else:
        p.codes_hi[:] = rng.randint_bytes(seed, "geh", p.codes_hi.size).reshape(p.codes_hi.shape)
        p.scales[:] = 1
        p.scales2[:] = np.float16(2.0 ** -6)
    return p


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [150, 8, 13])
def test_gemm_exact_arithmetic(fmt, m):
    """Unit scales and integer activations: every product and partial sum is an
    exact float32, so the bf16 output must be the bf16 rounding of the exact
    sum, whatever the summation order (150 and 13 rows: MFMA tiles; 8 rows:
    the row-streaming GEMV)."""
    q = _q()
    n, k = 260, 5120
    p = _unit_scale_weight(fmt, n, k, 60 + fmt)
    xi = rng.randint_bytes(61, "gex", m * k, 0, 9).astype(np.float64).reshape(m, k) - 4
    x = quant.bf16_bits(xi)
    w = q.Weight.from_host(p)
    y = q.gemm(w, _dev_bf16(x)).view(torch.int16).cpu().numpy().view(np.uint16)
    yref, _ = oracle.gemm(p, x)
    assert np.array_equal(y, oracle.bf16_round(yref.astype(np.float32)))


@pytest.mark.parametrize("fmt", [F.AFFINE4_G64, F.NVFP4])
def test_gemm_deterministic(fmt):
    q = _q()
    p = quant.synthetic_weight(fmt, 1024, 2048, name="gdet")
    x = _dev_bf16(quant.synthetic_bf16(384, 2048, name="gdetx"))
    w = q.Weight.from_host(p)
    ys = [q.gemm(w, x) for _ in range(3)]
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int16), y.view(torch.int16))


def test_gemm_rejects():
    q = _q()
    p = quant.synthetic_weight(F.AFFINE4_G64, 64, 512, name="grej")
    w = q.Weight.from_host(p)
    x = _dev_bf16(quant.synthetic_bf16(4, 512, name="grejx"))
    with pytest.raises(q.QmmError) as e:
        q.gemm(w, x[:0])                             # m = 0
    assert e.value.status == -5


# The prefill workload's own sizes, in the tile configurations the library
# picks for them (320-row activation tiles at M = 8192; at 1024, 2048, 3072
# and 4096 256-row tiles for whole rounds of workgroups and tiles of 128
# weight rows for the last 1024, by 32 activation rows at M = 1024, 64 at
# 2048 and 128 at 3072 and 4096; 192-row at 512, and
# the mid band's tiles: 32 rows with 4 K splits at M = 8, 64 rows at 48, 128
# rows at 96, 64 rows at 192): the GPU computes
# the whole product; the oracle checks sampled activation rows (every output
# column of each), including both edges of the tiles.
FULL_N, FULL_K = 17408, 5120


@pytest.fixture(scope="module")
def full_weights():
    cache = {}

    def get(fmt):
        if fmt not in cache:
            cache[fmt] = quant.synthetic_weight(fmt, FULL_N, FULL_K, name=f"gfull{fmt}")
        return cache[fmt]
    return get


@pytest.mark.parametrize("fmt,m", [(F.AFFINE4_G64, 128), (F.AFFINE4_G64, 512),
                                   (F.AFFINE4_G64, 2048), (F.AFFINE4_G64, 8192),
                                   (F.AFFINE4_G64, 4096), (F.AFFINE4_G64, 3072), (F.NVFP4, 1024),
                                   (F.NVFP4, 128), (F.NVFP4, 512), (F.NVFP4, 2048),
                                   (F.NVFP4, 4096), (F.NVFP4, 8192), (F.AFFINE4_G64, 8), (F.NVFP4, 16),
                                   (F.Q6_K, 5), (F.NVFP4, 48), (F.Q6_K, 96), (F.NVFP4, 192)])
def test_gemm_prefill_full_size_sampled(full_weights, fmt, m):
    q = _q()
    p = full_weights(fmt)
    x = quant.synthetic_bf16(m, FULL_K, name=f"gfullx{m}")
    w = q.Weight.from_host(p)
    y = _host_f64(q.gemm(w, _dev_bf16(x)))
    edges = [0, 1, 31, 32, 63, 64, 127, 128, 191, 192, 255, 256, 319, 320, 639, 640, m // 2, m - 2,
             m - 1]
    rows = np.unique(np.concatenate([edges, rng.randint_bytes(71, f"gfr{m}", 21, 0, 256).astype(np.int64) * (m // 256)]))
    rows = rows[rows < m]
    yref, mag = oracle.gemm(p, x[rows])
    _check(y[rows], yref, mag)


# The prefill workload's down-projection shape, 5120 x 17408 (40 blocks of
# 128 weight rows, 272 K slices), at 17 to 256 rows: K split 4 ways over
# 32-row tiles at 24 rows, over 64-row tiles at 48 and over 128-row tiles at
# 96 and 128, 2 ways over 64-row tiles at 192 and over 128-row tiles at 256
# (float32 partials in the workspace the binding allocates), and unsplit
# when the caller's workspace is too small.
@pytest.mark.parametrize("fmt,m", [(F.AFFINE4_G64, 24), (F.NVFP4, 48), (F.NVFP4, 96),
                                   (F.AFFINE4_G64, 128), (F.NVFP4, 192), (F.AFFINE4_G64, 256)])
def test_gemm_down_shape_split_sampled(fmt, m):
    q = _q()
    n, k = 5120, 17408
    p = quant.synthetic_weight(fmt, n, k, name=f"gdown{fmt}")
    x = quant.synthetic_bf16(m, k, name=f"gdownx{m}")
    w = q.Weight.from_host(p)
    xd = _dev_bf16(x)
    y = _host_f64(q.gemm(w, xd))
    rows = np.array([0, 1, 31, 32, 63, 64, 95, 127, 128, 191, m // 2, m - 1])
    rows = np.unique(rows[rows < m])
    yref, mag = oracle.gemm(p, x[rows])
    _check(y[rows], yref, mag)
    # a workspace too small for the partials: the same call unsplit
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    y2 = _host_f64(q.gemm(w, xd, workspace=small))
    _check(y2[rows], yref, mag)


# The mid band: 5 to 8 rows whose activations fit in LDS take the
# row-streaming GEMV (no workspace), 9 and more the MFMA tiles (split K up to
# 32 rows); ragged n and a residual on even m; bf16 y within the product bound.
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [5, 6, 7, 8, 9, 12, 16])
def test_gemm_mid_band_parity(fmt, m):
    q = _q()
    n, k = 515, 2048
    p = quant.synthetic_weight(fmt, n, k, outlier_rate=0.01, name=f"gmid{fmt}")
    x = quant.synthetic_bf16(m, k, name=f"gmidx{m}")
    r = quant.synthetic_bf16(m, n, name=f"gmidr{m}") if m % 2 == 0 else None
    w = q.Weight.from_host(p)
    if m <= 8:  # the GEMV path needs no split workspace
        assert int(q.lib_handle().qgemm_workspace_size(w.c, m)) == 0
    y = q.gemm(w, _dev_bf16(x), None if r is None else _dev_bf16(r))
    yref, mag = oracle.gemm(p, x, r)
    _check(_host_f64(y), yref, mag)
    y2 = q.gemm(w, _dev_bf16(x), None if r is None else _dev_bf16(r))
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("fmt", [F.AFFINE4_G64, F.NVFP4, F.Q6_K])
@pytest.mark.parametrize("m", [3, 20, 29])
def test_gemm_split_k(fmt, m):
    """Up to 32 rows a call with qgemm_workspace_size bytes of workspace
    splits K (4 splits up to 16 rows, 2 above); one without runs unsplit.
    Both meet the oracle's bar, and the split one is bitwise the same on every
    call, starting from a workspace of 0xFF bytes (no zero-fill needed)."""
    q = _q()
    n, k = 700, 4096
    p = quant.synthetic_weight(fmt, n, k, outlier_rate=0.01, name=f"gsk{fmt}")
    x = quant.synthetic_bf16(m, k, name=f"gskx{m}")
    r = quant.synthetic_bf16(m, n, name=f"gskr{m}")
    w = q.Weight.from_host(p)
    need = int(q.lib_handle().qgemm_workspace_size(w.c, m))
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    ys = [q.gemm(w, _dev_bf16(x), _dev_bf16(r), workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int16), y.view(torch.int16))
    y1 = q.gemm(w, _dev_bf16(x), _dev_bf16(r), workspace=q.new_workspace(256))  # too small: unsplit
    yref, mag = oracle.gemm(p, x, r)
    _check(_host_f64(ys[0]), yref, mag)
    _check(_host_f64(y1), yref, mag)
