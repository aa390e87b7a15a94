"""The Python binding's argument checks, on the CPU: every malformed tensor
argument (dtype, shape, contiguity, device, plane sizes) raises before the
library is asked to launch anything.  CPU tensors stand in for device
tensors; a call whose tensors are all well formed fails last, on the device
check, so reaching that error shows that every earlier check passed."""

import numpy as np
import pytest
import torch

import gemm_dequant_gemv_amd as q
from synth import formats as F


def _weight(fmt=F.AFFINE4_G64, n=64, k=256, batch=1):
    return q.Weight.from_host(F.empty(fmt, n, k, batch), device="cpu")


def _bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def test_weight_plane_checks():
    p = F.empty(F.AFFINE4_G64, 64, 256)
    t = lambda a: torch.from_numpy(a.copy())  # noqa: E731
    q.Weight(p.fmt, 64, 256, 1, t(p.codes), t(p.scales))            # well formed
    with pytest.raises(ValueError, match="codes holds"):
        q.Weight(p.fmt, 64, 512, 1, t(p.codes), t(p.scales))         # k does not match
    with pytest.raises(TypeError, match="scales has dtype"):
        q.Weight(p.fmt, 64, 256, 1, t(p.codes), t(p.scales).view(torch.int16))
    with pytest.raises(ValueError, match="Q6_K only"):
        q.Weight(p.fmt, 64, 256, 1, t(p.codes), t(p.scales), codes_hi=t(p.codes))
    with pytest.raises(ValueError, match="NVFP4 only"):
        q.Weight(p.fmt, 64, 256, 1, t(p.codes), t(p.scales),
                 tensor_scale=torch.ones(1))
    with pytest.raises(ValueError, match="contiguous"):
        q.Weight(p.fmt, 64, 256, 1, t(p.codes), t(p.scales).transpose(1, 2))
    p6 = F.empty(F.Q6_K, 64, 256)
    with pytest.raises(ValueError, match="scales2 is missing"):
        q.Weight(p6.fmt, 64, 256, 1, t(p6.codes), t(p6.scales), codes_hi=t(p6.codes_hi))
    with pytest.raises(ValueError, match="unknown format"):
        q.Weight(9, 64, 256, 1, t(p.codes), t(p.scales))
    for fmt in (F.AFFINE4_G64, F.MXFP4, F.NVFP4, F.Q6_K):
        _weight(fmt, 32, 256, batch=3)


def test_gemv_argument_checks():
    w = _weight()
    with pytest.raises(TypeError, match="x has dtype"):
        q.gemv(w, torch.zeros((1, 256), dtype=torch.float16))
    with pytest.raises(ValueError, match="x has shape"):
        q.gemv(w, _bf16(1, 128))
    with pytest.raises(ValueError, match="contiguous"):
        q.gemv(w, _bf16(256, 2).t())
    with pytest.raises(ValueError, match="residual has shape"):
        q.gemv(w, _bf16(2, 256), residual=_bf16(1, 64))
    with pytest.raises(TypeError, match="out has dtype"):
        q.gemv(w, _bf16(2, 256), out=torch.zeros((2, 64), dtype=torch.float16))
    with pytest.raises(ValueError, match="out has shape"):
        q.gemv(w, _bf16(2, 256), out=torch.zeros((2, 63)))
    with pytest.raises(TypeError, match="workspace has dtype"):
        q.gemv(w, _bf16(2, 256), workspace=torch.zeros(64, dtype=torch.int32))
    with pytest.raises(ValueError, match="must live on a GPU"):
        q.gemv(w, _bf16(2, 256), out=torch.zeros((2, 64)))
    with pytest.raises(ValueError, match="must live on a GPU"):
        q.PreparedGemv(w, _bf16(2, 256), torch.zeros((2, 64)))
    with pytest.raises(ValueError, match="out has shape"):
        q.PreparedGemv(w, _bf16(2, 256), torch.zeros((1, 64)))


def test_gemm_and_dequant_argument_checks():
    w = _weight()
    with pytest.raises(TypeError, match="out has dtype"):
        q.gemm(w, _bf16(8, 256), out=torch.zeros((8, 64)))           # float32 out
    with pytest.raises(ValueError, match="x has shape"):
        q.gemm(w, _bf16(8, 255))
    with pytest.raises(ValueError, match="must live on a GPU"):
        q.gemm(w, _bf16(8, 256), out=_bf16(8, 64))
    with pytest.raises(ValueError, match="out has shape"):
        q.prepare_gemm(w, _bf16(8, 256), _bf16(8, 65))
    with pytest.raises(ValueError, match="out has shape"):
        q.dequant(w, out=torch.zeros((1, 64, 255)))
    with pytest.raises(ValueError, match="must live on a GPU"):
        q.dequant(w, out=torch.zeros((1, 64, 256)))


def _moe_weights(E=4, S=1, H=256, inter=128):
    gu = _weight(F.NVFP4, 2 * inter, H, batch=E + S)
    dn = _weight(F.NVFP4, H, inter, batch=E + S)
    return gu, dn


def test_moe_argument_checks():
    gu, dn = _moe_weights()
    x = _bf16(3, 256)
    ids = torch.zeros((3, 2), dtype=torch.int32)
    wt = torch.zeros((3, 2))
    with pytest.raises(TypeError, match="topk_ids has dtype"):
        q.moe(gu, dn, x, ids.long(), wt, 4, 1)
    with pytest.raises(ValueError, match="topk_ids has shape"):
        q.moe(gu, dn, x, ids[:2], wt, 4, 1)
    with pytest.raises(ValueError, match="topk_w has shape"):
        q.moe(gu, dn, x, ids, wt[:, :1].contiguous(), 4, 1)
    with pytest.raises(ValueError, match="x has shape"):
        q.moe(gu, dn, _bf16(3, 128), ids, wt, 4, 1)
    with pytest.raises(ValueError, match="shared_w has shape"):
        q.moe(gu, dn, x, ids, wt, 4, 1, shared_w=torch.ones(4))
    with pytest.raises(ValueError, match="out has shape"):
        q.moe(gu, dn, x, ids, wt, 4, 1, out=torch.zeros((3, 255)))
    with pytest.raises(ValueError, match="must live on a GPU"):
        q.moe(gu, dn, x, ids, wt, 4, 1, out=torch.zeros((3, 256)))
    with pytest.raises(ValueError, match="must live on a GPU"):
        q.prepare_moe(gu, dn, x, ids, wt, 4, 1, torch.zeros((3, 256)))
    with pytest.raises(ValueError, match="logits has shape"):
        q.moe_from_logits(gu, dn, x, torch.zeros((3, 5)), 2, 4, 1)
    with pytest.raises(ValueError, match="must live on a GPU"):
        q.moe_from_logits(gu, dn, x, torch.zeros((3, 4)), 2, 4, 1, out=torch.zeros((3, 256)))


def test_router_argument_checks():
    with pytest.raises(TypeError, match="logits has dtype"):
        q.moe_router(torch.zeros((2, 8), dtype=torch.float64), 2)
    with pytest.raises(ValueError, match="ids has shape"):
        q.moe_router(torch.zeros((2, 8)), 2, ids=torch.zeros((2, 3), dtype=torch.int32))
    with pytest.raises(ValueError, match="must live on a GPU"):
        q.moe_router(torch.zeros((2, 8)), 2)


def test_host_planes_round_trip_dtypes():
    """Weight.from_host keeps each plane's numpy dtype, which is the dtype the
    checks expect."""
    for fmt, dt in ((F.AFFINE4_G64, torch.float16), (F.MXFP4, torch.uint8),
                    (F.NVFP4, torch.uint8), (F.Q6_K, torch.int8)):
        w = _weight(fmt, 16, 256)
        assert w.scales.dtype == dt and w.codes.dtype == torch.uint8


def test_gemv_hadamard_and_stage_argument_checks():
    w = _weight()
    x = _bf16(2, 256)
    with pytest.raises(TypeError, match="in_scale has dtype"):
        q.gemv_hadamard(w, x, in_scale=torch.zeros(256))
    with pytest.raises(ValueError, match="in_scale has shape"):
        q.gemv_hadamard(w, x, in_scale=torch.zeros(128, dtype=torch.float16))
    with pytest.raises(ValueError, match="out_scale has shape"):
        q.gemv_hadamard(w, x, out_scale=torch.zeros(256, dtype=torch.float16))
    with pytest.raises(ValueError, match="x has shape"):
        q.gemv_hadamard(w, _bf16(2, 128))
    with pytest.raises(ValueError, match="must live on a GPU"):
        q.gemv_hadamard(w, x, in_scale=torch.zeros(256, dtype=torch.float16),
                        out_scale=torch.zeros(64, dtype=torch.float16))
    with pytest.raises(TypeError, match="x has dtype"):
        q.hadamard_prepare(torch.zeros((2, 256)))
    with pytest.raises(TypeError, match="y has dtype"):
        q.hadamard_finish(_bf16(2, 256))
