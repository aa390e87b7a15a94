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
