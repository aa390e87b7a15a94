"""Thin Python binding of libqmm (ctypes): argument marshalling only.

Every step of every call runs in the library's HIP kernels; PyTorch provides
device memory and the current stream.  If libqmm.so has not been built the
first call raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QMM_LIB_PATH selects another build of the same library (experiments only)
LIB_PATH = os.environ.get("QMM_LIB_PATH") or os.path.join(_HERE, "libqmm.so")

AFFINE4_G64, MXFP4, NVFP4, Q6_K = 1, 2, 3, 4
F32, BF16 = 0, 1
FORMATS = {"affine4_g64": AFFINE4_G64, "mxfp4": MXFP4, "nvfp4": NVFP4, "q6_k": Q6_K}

ENTRY_POINTS = ("qdequant", "qgemv", "qgemv_workspace_size", "qgemm", "qgemm_workspace_size",
                "qmoe_grouped", "qmoe_workspace_size", "qmoe_workspace_layout", "qmoe_router",
                "qmoe_grouped_logits",
                "qworkspace_init", "qbench_stream_read", "qbench_mfma_peak", "qstatus_string",
                "qlast_hip_error")


class QmmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().qstatus_string(status).decode()
        if status == -8:
            msg += f" (hipError_t {_lib().qlast_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


class QmmWeightC(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("codes_hi", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("scales2", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p)]


class QmoeLayoutC(ctypes.Structure):
    _fields_ = [(name, ctypes.c_size_t) for name in (
        "counts", "offsets", "row_of_slot", "row_of_shared", "token_of_row", "active",
        "scalars", "tiles", "h", "d", "bytes", "max_rows", "max_tiles", "slot_rows", "tile_rows")]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python -m gemm_dequant_gemv_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, VP = ctypes.POINTER(QmmWeightC), ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
        lib.qdequant.argtypes = [P, I32, VP, VP]
        lib.qgemv_workspace_size.argtypes = [P, I32]
        lib.qgemv_workspace_size.restype = SZ
        lib.qgemv.argtypes = [P, VP, I32, VP, VP, I32, VP, SZ, VP]
        lib.qgemm_workspace_size.argtypes = [P, I32]
        lib.qgemm_workspace_size.restype = SZ
        lib.qgemm.argtypes = [P, VP, I32, VP, VP, VP, SZ, VP]
        lib.qmoe_workspace_size.argtypes = [P, P, I32, I32, I32, I32]
        lib.qmoe_workspace_size.restype = SZ
        lib.qmoe_workspace_layout.argtypes = [P, P, I32, I32, I32, I32, ctypes.POINTER(QmoeLayoutC)]
        lib.qmoe_grouped.argtypes = [P, P, I32, I32, VP, I32, VP, VP, I32, VP, VP, I32, VP, SZ, VP]
        lib.qmoe_router.argtypes = [VP, I32, I32, I32, VP, VP, VP]
        lib.qmoe_grouped_logits.argtypes = [P, P, I32, I32, VP, I32, VP, I32, VP, VP, VP, VP, I32,
                                            VP, SZ, VP]
        lib.qworkspace_init.argtypes = [VP, SZ, VP]
        lib.qbench_stream_read.argtypes = [VP, SZ, VP, I32, VP]
        lib.qbench_mfma_peak.argtypes = [I32, I32, VP, ctypes.POINTER(ctypes.c_double), VP]
        lib.qstatus_string.restype = ctypes.c_char_p
        lib.qstatus_string.argtypes = [ctypes.c_int]
        _LIB = lib
    return _LIB


def lib_handle():
    return _lib()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise QmmError(status, where)


class Weight:
    """A packed weight (or batch of experts) resident on the device.

    Planes follow include/qmm.h: ``codes`` u8 [batch][n][k/2], ``codes_hi``
    u8 [batch][n][k/4] (Q6_K), ``scales`` (format dependent), ``scales2``
    f16 [batch][n][k/256] (Q6_K), ``tensor_scale`` f32 [batch] (NVFP4)."""

    def __init__(self, fmt: int, n: int, k: int, batch: int, codes, scales,
                 codes_hi=None, scales2=None, tensor_scale=None):
        self.fmt, self.n, self.k, self.batch = int(fmt), int(n), int(k), int(batch)
        self.codes, self.scales = codes, scales
        self.codes_hi, self.scales2, self.tensor_scale = codes_hi, scales2, tensor_scale
        self._c = QmmWeightC(self.fmt, self.n, self.k, self.batch, self.codes.data_ptr(),
                             None if codes_hi is None else codes_hi.data_ptr(),
                             self.scales.data_ptr(),
                             None if scales2 is None else scales2.data_ptr(),
                             None if tensor_scale is None else tensor_scale.data_ptr())

    @classmethod
    def from_host(cls, p, device="cuda"):
        """Upload an object with numpy planes (``fmt, n, k, batch, codes,
        scales, codes_hi, scales2, tensor_scale``)."""
        def up(a):
            if a is None:
                return None
            return torch.from_numpy(a.copy()).to(device)
        return cls(p.fmt, p.n, p.k, p.batch, up(p.codes), up(p.scales), up(p.codes_hi),
                   up(p.scales2), up(p.tensor_scale))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.codes, self.scales, self.codes_hi, self.scales2, self.tensor_scale)
                   if t is not None)

    @property
    def c(self):
        return ctypes.byref(self._c)


def dequant(w: Weight, out_dtype=torch.float32, out=None, stream=None):
    if out is None:
        out = torch.empty((w.batch, w.n, w.k), dtype=out_dtype, device=w.codes.device)
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qdequant(w.c, dt, _ptr(out), _stream(stream)), "qdequant")
    return out


def gemv_workspace_size(w: Weight, m: int) -> int:
    return int(_lib().qgemv_workspace_size(w.c, m))


def new_workspace(nbytes: int, device="cuda"):
    """A zero-filled workspace (the library leaves it zero-filled after each call)."""
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def gemv(w: Weight, x, residual=None, y_dtype=torch.float32, out=None, workspace=None,
         stream=None):
    """y[m][n] = sum_k w[n][k] x[m][k] (+ residual), m = x.shape[0] in 1..4."""
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, w.n), dtype=y_dtype, device=x.device)
    need = gemv_workspace_size(w, m)
    if workspace is None and need:
        workspace = new_workspace(need, x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qgemv(w.c, _ptr(x), m, _ptr(residual), _ptr(out), dt, _ptr(workspace),
                        ws_bytes, _stream(stream)), "qgemv")
    return out


def gemm(w: Weight, x, residual=None, out=None, workspace=None, stream=None):
    """y[m][n] = bf16(sum_k w16[n][k] x[m][k] (+ residual)), x bf16 [m][k]."""
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, w.n), dtype=torch.bfloat16, device=x.device)
    need = int(_lib().qgemm_workspace_size(w.c, m))
    if workspace is None and need:
        workspace = new_workspace(need, x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().qgemm(w.c, _ptr(x), m, _ptr(residual), _ptr(out), _ptr(workspace), ws_bytes,
                        _stream(stream)), "qgemm")
    return out


def moe_workspace_size(gate_up: Weight, down: Weight, num_routed: int, num_shared: int,
                       t: int, topk: int) -> int:
    return int(_lib().qmoe_workspace_size(gate_up.c, down.c, num_routed, num_shared, t, topk))


def moe_workspace_layout(gate_up: Weight, down: Weight, num_routed: int, num_shared: int,
                         t: int, topk: int) -> dict:
    """Byte offsets of the intermediates inside a qmoe_grouped workspace, by name."""
    out = QmoeLayoutC()
    _check(_lib().qmoe_workspace_layout(gate_up.c, down.c, num_routed, num_shared, t, topk,
                                        ctypes.byref(out)), "qmoe_workspace_layout")
    return {name: int(getattr(out, name)) for name, _ in QmoeLayoutC._fields_}


def moe(gate_up: Weight, down: Weight, x, topk_ids, topk_w, num_routed: int, num_shared: int,
        shared_w=None, y_dtype=torch.float32, out=None, workspace=None, stream=None):
    """One MoE layer; x bf16 [t][H], topk_ids int32 [t][topk], topk_w f32 [t][topk]."""
    t, topk = topk_ids.shape
    if out is None:
        out = torch.empty((t, down.n), dtype=y_dtype, device=x.device)
    need = moe_workspace_size(gate_up, down, num_routed, num_shared, t, topk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qmoe_grouped(gate_up.c, down.c, num_routed, num_shared, _ptr(x), t,
                               _ptr(topk_ids), _ptr(topk_w), topk, _ptr(shared_w), _ptr(out), dt,
                               _ptr(workspace), ws_bytes, _stream(stream)), "qmoe_grouped")
    return out


def moe_router(logits, topk: int, ids=None, w=None, stream=None):
    """Router top-k and softmax: logits float32 [t][E] -> (ids int32 [t][topk],
    weights float32 [t][topk])."""
    t, e = logits.shape
    if ids is None:
        ids = torch.empty((t, topk), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((t, topk), dtype=torch.float32, device=logits.device)
    _check(_lib().qmoe_router(_ptr(logits), t, e, topk, _ptr(ids), _ptr(w), _stream(stream)),
           "qmoe_router")
    return ids, w


def moe_from_logits(gate_up: Weight, down: Weight, x, logits, topk: int, num_routed: int,
                    num_shared: int, shared_w=None, y_dtype=torch.float32, out=None,
                    workspace=None, stream=None):
    """One MoE layer from router logits float32 [t][num_routed]; returns (y,
    ids, weights)."""
    t = logits.shape[0]
    if out is None:
        out = torch.empty((t, down.n), dtype=y_dtype, device=x.device)
    ids = torch.empty((t, topk), dtype=torch.int32, device=x.device)
    w = torch.empty((t, topk), dtype=torch.float32, device=x.device)
    need = moe_workspace_size(gate_up, down, num_routed, num_shared, t, topk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qmoe_grouped_logits(gate_up.c, down.c, num_routed, num_shared, _ptr(x), t,
                                      _ptr(logits), topk, _ptr(ids), _ptr(w), _ptr(shared_w),
                                      _ptr(out), dt, _ptr(workspace), ws_bytes, _stream(stream)),
           "qmoe_grouped_logits")
    return out, ids, w


def workspace_init(ws, stream=None):
    _check(_lib().qworkspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "qworkspace_init")


def bench_stream_read(buf, sink, blocks: int, stream=None):
    """Stream-read ``buf`` (a device tensor) once; see qbench_stream_read."""
    _check(_lib().qbench_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                     int(blocks), _stream(stream)), "qbench_stream_read")


def bench_mfma_peak(iters: int, blocks: int, sink, stream=None) -> float:
    """Launch the MFMA loop once; returns its operation count.  See
    qbench_mfma_peak."""
    flops = ctypes.c_double(0.0)
    _check(_lib().qbench_mfma_peak(int(iters), int(blocks), _ptr(sink), ctypes.byref(flops),
                                   _stream(stream)), "qbench_mfma_peak")
    return flops.value


class PreparedGemv:
    """A qgemv call with every argument marshalled once, for loops that launch
    the same call many times (benchmarks, decode loops).  Calling it launches
    the kernel on the stream given here (the current stream by default)."""

    def __init__(self, w: Weight, x, out, residual=None, workspace=None, stream=None):
        self.w, self.x, self.out, self.residual, self.workspace = w, x, out, residual, workspace
        need = gemv_workspace_size(w, x.shape[0])
        if need and workspace is None:
            raise ValueError("qgemv needs a workspace of %d bytes" % need)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        dt = F32 if out.dtype == torch.float32 else BF16
        self._args = (w.c, _ptr(x), x.shape[0], _ptr(residual), _ptr(out), dt, _ptr(workspace),
                      ws_bytes, _stream(stream))
        self._fn = _lib().qgemv

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            raise QmmError(st, "qgemv")


class _Prepared:
    """A library call with every argument marshalled once (benchmarks, decode
    loops); calling it launches on the stream given at construction."""

    def __init__(self, name, args, keep):
        self._fn = getattr(_lib(), name)
        self._name = name
        self._args = args
        self._keep = keep  # tensors the raw pointers refer to

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            raise QmmError(st, self._name)


def prepare_gemm(w: Weight, x, out, residual=None, stream=None):
    m = x.shape[0]
    need = int(_lib().qgemm_workspace_size(w.c, m))
    ws = new_workspace(need, x.device) if need else None
    ws_bytes = 0 if ws is None else ws.numel()
    return _Prepared("qgemm", (w.c, _ptr(x), m, _ptr(residual), _ptr(out), _ptr(ws), ws_bytes,
                               _stream(stream)), (w, x, out, residual, ws))


def prepare_moe(gate_up: Weight, down: Weight, x, topk_ids, topk_w, num_routed: int,
                num_shared: int, out, shared_w=None, stream=None):
    t, topk = topk_ids.shape
    need = moe_workspace_size(gate_up, down, num_routed, num_shared, t, topk)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    dt = F32 if out.dtype == torch.float32 else BF16
    return _Prepared("qmoe_grouped",
                     (gate_up.c, down.c, num_routed, num_shared, _ptr(x), t, _ptr(topk_ids),
                      _ptr(topk_w), topk, _ptr(shared_w), _ptr(out), dt, _ptr(ws), ws.numel(),
                      _stream(stream)),
                     (gate_up, down, x, topk_ids, topk_w, out, shared_w, ws))
