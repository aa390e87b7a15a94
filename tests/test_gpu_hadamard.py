"""GPU parity of the Hadamard prepare and finish stages against the CPU
oracle, through the C ABI.

Bar: the transform sums 128 products in float32 (seven butterfly stages), so
each output must be within 1e-6 of its magnitude sum sum |h_ij| |s_j x_j| of
the exact float64 value, plus half a bf16 ulp where the output is stored as
bf16 (the oracle's value is rounded at the same point)."""

import numpy as np
import pytest
import torch

import oracle
from synth import quant, rng

pytestmark = pytest.mark.gpu
REL = 1e-6


def _q():
    import gemm_dequant_gemv_amd as q
    return q


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).cuda()


def _scales(n, tag):
    """float16 channel scales in [-2, 2) with random signs."""
    u = rng.uniform_matrix(rng.BASE_SEED, tag, 1, n)[0]
    return (4.0 * u - 2.0).astype(np.float16)


@pytest.mark.parametrize("m,k", [(1, 128), (5, 512), (64, 5120), (3, 17408)])
@pytest.mark.parametrize("scaled", [False, True])
def test_hadamard_prepare_parity(m, k, scaled):
    q = _q()
    x = quant.synthetic_bf16(m, k, name=f"hadx{m}{k}")
    s = _scales(k, f"hads{k}") if scaled else None
    out = q.hadamard_prepare(_dev_bf16(x), None if s is None else torch.from_numpy(s).cuda())
    got = oracle.bf16(out.view(torch.int16).cpu().numpy().view(np.uint16))
    yref, _, mag = oracle.hadamard_prepare(x, None if s is None else s.view(np.uint16))
    ok = np.abs(got - yref) <= REL * mag + oracle.bf16_half_ulp(yref)
    assert ok.all(), f"{(~ok).sum()} outputs off"


def test_hadamard_prepare_one_hot_columns():
    """Input e_j in every block position j gives column j of H / sqrt(128):
    checks the ordering of every butterfly stage."""
    q = _q()
    k = 128
    x = np.zeros((k, k))
    np.fill_diagonal(x, 1.0)
    xb = quant.bf16_bits(x)
    out = q.hadamard_prepare(_dev_bf16(xb))
    got = oracle.bf16(out.view(torch.int16).cpu().numpy().view(np.uint16))
    from scipy.linalg import hadamard
    expect = oracle.bf16(oracle.bf16_round(np.float32(hadamard(128).T / np.sqrt(128))))
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("scaled", [False, True])
def test_hadamard_finish_parity(out_dtype, scaled):
    q = _q()
    m, n = 9, 2048
    y = (rng.normal_matrix(rng.BASE_SEED, "hady", m, n, 30.0)).astype(np.float32)
    s = _scales(n, "hadfs") if scaled else None
    out = q.hadamard_finish(torch.from_numpy(y).cuda(),
                            None if s is None else torch.from_numpy(s).cuda(), out_dtype=out_dtype)
    if out_dtype == torch.float32:
        got = out.cpu().numpy().astype(np.float64)
        half = 0.0
    else:
        got = oracle.bf16(out.view(torch.int16).cpu().numpy().view(np.uint16))
    oref, mag = oracle.hadamard_finish(y, None if s is None else s.view(np.uint16))
    if out_dtype == torch.bfloat16:
        half = oracle.bf16_half_ulp(oref)
    ok = np.abs(got - oref) <= REL * mag + half
    assert ok.all(), f"{(~ok).sum()} outputs off"


def test_hadamard_finish_after_prepare_returns_the_scaled_input():
    q = _q()
    x = quant.synthetic_bf16(4, 1024, name="hadrt")
    xd = _dev_bf16(x)
    p = q.hadamard_prepare(xd).float()
    back = q.hadamard_finish(p).cpu().numpy().astype(np.float64)
    xr = oracle.bf16(x)
    # prepare's bf16 rounding is the only loss: relative 2^-9 per value, and
    # the orthogonal transform keeps the error's norm
    err = np.linalg.norm((back - xr).reshape(4, 8, 128), axis=-1)
    assert (err <= 2.0 ** -8 * np.linalg.norm(xr.reshape(4, 8, 128), axis=-1)).all()


def test_hadamard_argument_errors():
    q = _q()
    x = torch.zeros((2, 200), dtype=torch.bfloat16, device="cuda")   # not a multiple of 128
    with pytest.raises(q.QmmError) as e:
        q.hadamard_prepare(x)
    assert e.value.status == -3
    y = torch.zeros((2, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(q.QmmError) as e:
        q.hadamard_finish(y, out=y)                                   # in place: alias
    assert e.value.status == -7


# qgemv_hadamard: prepare, the GEMV and finish in one call.  Bar: bitwise
# equal to qhadamard_prepare, qgemv and qhadamard_finish run in sequence
# (workspace carving, the in-place finish of a float32 y, the split-K GEMV at
# K = 81920), for every format, 1-4 rows, with and without channel scales,
# float32 and bf16 y.
HAD_SHAPES = [(640, 1024), (384, 5120), (256, 17408), (128, 81920)]


def _had_weight(fmt, n, k, name):
    return quant.synthetic_weight(fmt, n, k, outlier_rate=0.01, name=name)


@pytest.mark.parametrize("fmt", [1, 2, 3, 4])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", HAD_SHAPES)
def test_gemv_hadamard_equals_the_staged_calls(fmt, m, shape):
    q = _q()
    n, k = shape
    p = _had_weight(fmt, n, k, f"hg{fmt}{n}{k}")
    w = q.Weight.from_host(p)
    x = _dev_bf16(quant.synthetic_bf16(m, k, name=f"hgx{m}{k}"))
    si = torch.from_numpy(_scales(k, f"hgsi{k}")).cuda()
    so = torch.from_numpy(_scales(n, f"hgso{n}")).cuda()
    for scaled in (False, True):
        a, b = (si, so) if scaled else (None, None)
        for dt in (torch.float32, torch.bfloat16):
            fused = q.gemv_hadamard(w, x, a, b, y_dtype=dt)
            staged = q.hadamard_finish(q.gemv(w, q.hadamard_prepare(x, a)), b, out_dtype=dt)
            torch.cuda.synchronize()
            assert torch.equal(fused.view(torch.int16), staged.view(torch.int16)), (scaled, dt)


def test_gemv_hadamard_against_the_oracle_chain():
    """The chain against the oracle's stages: the oracle's GEMV on the GPU's
    prepared activations, then the oracle's finish; each output within
    2e-3 |s_out| sum_i mag_i / sqrt(128) over its block (the GEMV's bound
    carried through the orthonormal transform) plus 1e-6 of the finish's own
    magnitude sum."""
    q = _q()
    n, k, m = 384, 5120, 3
    p = _had_weight(4, n, k, "hgo")
    w = q.Weight.from_host(p)
    xb = quant.synthetic_bf16(m, k, name="hgox")
    si, so = _scales(k, "hgosi"), _scales(n, "hgoso")
    x = _dev_bf16(xb)
    y = q.gemv_hadamard(w, x, torch.from_numpy(si).cuda(), torch.from_numpy(so).cuda())
    y = y.cpu().numpy().astype(np.float64)
    xp = q.hadamard_prepare(x, torch.from_numpy(si).cuda()).view(torch.int16).cpu().numpy().view(np.uint16)
    ylin, mag = oracle.gemv(p, xp)
    yref, fmag = oracle.hadamard_finish(ylin.astype(np.float32), so.view(np.uint16))
    s_abs = np.abs(oracle.fp16(so.view(np.uint16)))
    blk_mag = np.repeat(mag.reshape(m, n // 128, 128).sum(-1) / np.sqrt(128), 128, axis=-1).reshape(m, n)
    bound = 2e-3 * s_abs * blk_mag + 1e-6 * fmag
    ok = np.abs(y - yref) <= bound
    assert ok.all(), f"{(~ok).sum()} outputs off"


def test_gemv_hadamard_argument_errors():
    q = _q()
    p = _had_weight(1, 256, 192, "hge")           # k not a multiple of 128
    w = q.Weight.from_host(p)
    x = _dev_bf16(quant.synthetic_bf16(2, 192, name="hgex"))
    with pytest.raises(q.QmmError) as e:
        q.gemv_hadamard(w, x)
    assert e.value.status == -3
    p2 = _had_weight(1, 256, 256, "hge2")
    w2 = q.Weight.from_host(p2)
    x5 = _dev_bf16(quant.synthetic_bf16(5, 256, name="hgex5"))
    with pytest.raises(q.QmmError) as e:
        q.gemv_hadamard(w2, x5)
    assert e.value.status == -5
