"""qmoe_grouped_noalloc (the MoE layer on the library's static scratch, for
callers that cannot allocate) against qmoe_grouped with a caller workspace,
through the C ABI: the same kernels run, so the outputs must be bitwise
equal.  Each case makes two calls in a row on the shared buffer, the second
with fewer tokens, and a call too large for the buffer is refused before
any launch."""


import numpy as np
import pytest
import torch

from synth import formats as F
from synth import quant, routing

pytestmark = pytest.mark.gpu


def _q():
    import gemm_dequant_gemv_amd as q
    return q


def _dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()


def _layer(E, S, H, inter, fmt, tag):
    q = _q()
    gu = q.Weight.from_host(quant.synthetic_weight(fmt, 2 * inter, H, batch=E + S, name=f"{tag}/gu"))
    dn = q.Weight.from_host(quant.synthetic_weight(fmt, H, inter, batch=E + S, name=f"{tag}/dn"))
    return gu, dn


def _inputs(T, E, H, topk, tag):
    x = _dev_bf16(quant.synthetic_bf16(T, H, name=f"{tag}/x{T}"))
    ids, w = routing.random_routing(T, E, topk, name=f"{tag}/r{T}")
    return x, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()


@pytest.mark.parametrize("tokens,y_dtype", [((8, 3), torch.float32), ((60, 20), torch.bfloat16),
                                            ((11, 4), torch.bfloat16)])
def test_noalloc_matches_workspace_call(tokens, y_dtype):
    """Decode form (up to 11 tokens of 10 + 1 slots) and grouped form (more
    tokens) on the 512 + 1-expert layer shape, two calls in a row with the
    second smaller; bitwise equal to qmoe_grouped with its own workspace."""
    q = _q()
    E, S, H, inter, topk = 512, 1, 2048, 512, 10
    gu, dn = _layer(E, S, H, inter, F.NVFP4, "noalloc")
    outs = []
    for T in tokens:
        x, ids, w = _inputs(T, E, H, topk, "noalloc")
        y = torch.empty((T, H), dtype=y_dtype, device="cuda")
        q.moe_noalloc(gu, dn, x, ids, w, E, S, y)
        outs.append((T, x, ids, w, y))
    torch.cuda.synchronize()
    for T, x, ids, w, y in outs:
        ref = q.moe(gu, dn, x, ids, w, E, S, y_dtype=y_dtype)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"T={T}"


def test_noalloc_shared_weight_and_other_format():
    """A weighted shared expert and mixed formats, two calls with the second
    smaller, against the workspace call."""
    q = _q()
    E, S, H, inter, topk = 16, 1, 512, 128, 4
    gu = q.Weight.from_host(quant.synthetic_weight(F.AFFINE4_G64, 2 * inter, H, batch=E + S,
                                                   name="noalloc2/gu"))
    dn = q.Weight.from_host(quant.synthetic_weight(F.MXFP4, H, inter, batch=E + S,
                                                   name="noalloc2/dn"))
    for T in (40, 7):
        x, ids, w = _inputs(T, E, H, topk, "noalloc2")
        sw = torch.rand(T, generator=torch.Generator().manual_seed(T)).cuda()
        y = torch.empty((T, H), dtype=torch.float32, device="cuda")
        q.moe_noalloc(gu, dn, x, ids, w, E, S, y, shared_w=sw)
        ref = q.moe(gu, dn, x, ids, w, E, S, shared_w=sw)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), f"T={T}"


def test_noalloc_refuses_calls_beyond_its_scratch():
    """8192 tokens of the 512-expert layer need far more than 16 MiB: the
    call is refused with QMM_ERR_SCRATCH and writes nothing."""
    q = _q()
    E, S, H, inter, topk = 512, 1, 2048, 512, 10
    gu, dn = _layer(E, S, H, inter, F.NVFP4, "noalloc")
    T = 8192
    assert q.moe_workspace_size(gu, dn, E, S, T, topk) > 16 << 20
    x, ids, w = _inputs(T, E, H, topk, "noalloc3")
    y = torch.full((T, H), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(q.QmmError) as e:
        q.moe_noalloc(gu, dn, x, ids, w, E, S, y)
    assert e.value.status == -11
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    lib = q.lib_handle()
    assert isinstance(lib.qstatus_string(-11), bytes)
