"""The C-ABI library loads without a GPU, exports every entry point the header
declares, and rejects bad arguments before launching anything."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(q\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import gemm_dequant_gemv_amd as q
    return q.lib_handle()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("qdequant", "qgemv", "qgemv_workspace_size", "qworkspace_init",
              "qstatus_string", "qlast_hip_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_binding_lists_every_declared_entry_point():
    from gemm_dequant_gemv_amd import qmm
    assert set(_declared()) <= set(qmm.ENTRY_POINTS)


def _w(fmt=1, n=128, k=256, batch=1, codes=0x10000, hi=None, sc=0x20000, s2=None, ts=None):
    from gemm_dequant_gemv_amd import qmm
    return qmm.QmmWeightC(fmt, n, k, batch, codes, hi, sc, s2, ts)


X, Y = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)


def _gemv(lib, w, m=1, x=X, y=Y, ydt=0, ws=None, wsb=0, res=None):
    return lib.qgemv(ctypes.byref(w), x, m, res, y, ydt, ws, wsb, None)


@pytest.mark.parametrize("case,status", [
    (dict(fmt=0), -2), (dict(fmt=5), -2),
    (dict(k=100), -3), (dict(k=0), -3), (dict(n=0), -3), (dict(k=48), -3), (dict(k=96), -3),
    (dict(fmt=2, k=192), -3), (dict(fmt=3, k=96), -3), (dict(n=1 << 20, k=1 << 13), -3),
    (dict(fmt=4, k=288, hi=0x30000, s2=0x40000), -3),
    (dict(codes=None), -1), (dict(sc=None), -1),
    (dict(fmt=4), -1),                               # Q6_K needs codes_hi and scales2
    (dict(hi=0x30000), -2),                          # affine has no codes_hi
    (dict(ts=0x50000), -2),                          # only NVFP4 has a tensor scale
    (dict(codes=0x10008), -4), (dict(sc=0x20002), -4),
    (dict(batch=2), -3),                             # qgemv takes one matrix
])
def test_gemv_rejects_bad_weights(lib, case, status):
    assert _gemv(lib, _w(**case)) == status


def test_gemv_rejects_bad_calls(lib):
    w = _w()
    assert _gemv(lib, w, m=0) == -5
    assert _gemv(lib, w, m=5) == -5
    assert _gemv(lib, w, ydt=7) == -9
    assert _gemv(lib, w, x=None) == -1
    assert _gemv(lib, w, y=None) == -1
    assert _gemv(lib, w, x=ctypes.c_void_p(0x100004)) == -4
    # y overlapping the codes
    assert _gemv(lib, w, y=ctypes.c_void_p(0x10000)) == -7
    assert _gemv(lib, w, y=ctypes.c_void_p(0x100000)) == -7          # y over x


def test_gemv_workspace_checks(lib):
    w = _w(n=512, k=8192)
    need = lib.qgemv_workspace_size(ctypes.byref(w), 2)
    assert need > 0 and need % 256 == 0
    assert _gemv(lib, w, m=2) == -6
    assert _gemv(lib, w, m=2, ws=ctypes.c_void_p(0x1000000), wsb=need - 1) == -6
    assert _gemv(lib, w, m=2, ws=ctypes.c_void_p(0x1000010), wsb=need) == -4


def test_workspace_size_zero_for_invalid(lib):
    assert lib.qgemv_workspace_size(ctypes.byref(_w(k=100)), 1) == 0
    assert lib.qgemv_workspace_size(ctypes.byref(_w()), 9) == 0


def test_dequant_rejects(lib):
    w = _w()
    assert lib.qdequant(ctypes.byref(w), 3, Y, None) == -9
    assert lib.qdequant(ctypes.byref(w), 0, None, None) == -1
    assert lib.qdequant(ctypes.byref(w), 0, ctypes.c_void_p(0x200008), None) == -4
    assert lib.qdequant(ctypes.byref(w), 0, ctypes.c_void_p(0x20000), None) == -7


def test_status_strings(lib):
    for s in range(-10, 1):
        assert lib.qstatus_string(s)
    assert lib.qlast_hip_error() == 0


VP = ctypes.c_void_p


def _router(lib, logits=0x42000000, t=4, e=64, k=8, ids=0x40000000, w=0x41000000):
    return lib.qmoe_router(VP(logits) if logits else None, t, e, k, VP(ids) if ids else None,
                           VP(w) if w else None, None)


def test_router_rejects_bad_calls(lib):
    assert _router(lib, logits=0) == -1
    assert _router(lib, ids=0) == -1
    assert _router(lib, w=0) == -1
    assert _router(lib, k=0) == -10
    assert _router(lib, k=65, e=128) == -10
    assert _router(lib, k=9, e=8) == -10         # more picks than experts
    assert _router(lib, e=0) == -10
    assert _router(lib, e=4097) == -10
    assert _router(lib, t=0) == -5
    assert _router(lib, logits=0x42000002) == -4
    assert _router(lib, ids=0x42000000 + 64) == -7   # ids over the logits
    assert _router(lib, w=0x40000000 + 16) == -7     # weights over the ids


def _moe_weights(E=4, S=1, H=256, I=128):
    gu = _w(fmt=1, n=2 * I, k=H, batch=E + S, codes=0x10000000, sc=0x11000000)
    dn = _w(fmt=1, n=H, k=I, batch=E + S, codes=0x12000000, sc=0x13000000)
    return gu, dn


def _moe_logits(lib, topk=2, logits=0x42000000, ids=0x40000000, w=0x41000000, x=0x20000000,
                y=0x21000000, t=4, E=4, S=1):
    gu, dn = _moe_weights(E, S)
    need = lib.qmoe_workspace_size(ctypes.byref(gu), ctypes.byref(dn), E, S, t, max(topk, 1))
    return lib.qmoe_grouped_logits(ctypes.byref(gu), ctypes.byref(dn), E, S, VP(x), t,
                                   VP(logits) if logits else None, topk, VP(ids), VP(w), None,
                                   VP(y), 0, VP(0x30000000), need, None)


def test_moe_from_logits_rejects_bad_calls(lib):
    assert _moe_logits(lib, logits=0) == -1
    assert _moe_logits(lib, topk=5) == -10            # more picks than routed experts
    assert _moe_logits(lib, topk=0) == -10
    assert _moe_logits(lib, logits=0x42000002) == -4
    assert _moe_logits(lib, ids=0x20000000) == -7     # routing written over x
    assert _moe_logits(lib, w=0x10000000) == -7       # routing written over the weights
    assert _moe_logits(lib, logits=0x21000000) == -7  # logits under y
    assert _moe_logits(lib, ids=0x42000000) == -7     # ids over the logits
