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
                "qmoe_grouped_logits", "qmoe_grouped_noalloc", "qquant_mxfp4",
                "qhadamard_prepare", "qhadamard_finish", "qgemv_hadamard_workspace_size",
                "qgemv_hadamard",
                "qgemm_w4a4_workspace_size", "qgemm_w4a4",
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
        "scalars", "tiles", "h", "d", "bytes", "max_rows", "max_tiles", "slot_rows", "tile_rows",
        "slot_of_row")]


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
        lib.qquant_mxfp4.argtypes = [VP, I32, I32, VP, VP, VP]
        lib.qhadamard_prepare.argtypes = [VP, I32, I32, VP, VP, VP]
        lib.qhadamard_finish.argtypes = [VP, I32, I32, VP, VP, I32, VP]
        lib.qgemv_hadamard_workspace_size.argtypes = [P, I32, I32]
        lib.qgemv_hadamard_workspace_size.restype = SZ
        lib.qgemv_hadamard.argtypes = [P, VP, I32, VP, VP, VP, I32, VP, SZ, VP]
        lib.qgemm_w4a4_workspace_size.argtypes = [P, I32]
        lib.qgemm_w4a4_workspace_size.restype = SZ
        lib.qgemm_w4a4.argtypes = [P, VP, I32, VP, VP, VP, SZ, VP]
        lib.qmoe_workspace_size.argtypes = [P, P, I32, I32, I32, I32]
        lib.qmoe_workspace_size.restype = SZ
        lib.qmoe_workspace_layout.argtypes = [P, P, I32, I32, I32, I32, ctypes.POINTER(QmoeLayoutC)]
        lib.qmoe_grouped.argtypes = [P, P, I32, I32, VP, I32, VP, VP, I32, VP, VP, I32, VP, SZ, VP]
        lib.qmoe_grouped_noalloc.argtypes = [P, P, I32, I32, VP, I32, VP, VP, I32, VP, VP, I32,
                                             VP]
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


def _tensor(where: str, name: str, t, dtypes, shape=None, device=None):
    """Check one tensor argument before anything is launched: its dtype, its
    shape, that it is contiguous and (when ``device`` is given) that it lives
    on that GPU.  Raises TypeError or ValueError."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{where}: {name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        want = ", ".join(str(d) for d in dtypes)
        raise TypeError(f"{where}: {name} has dtype {t.dtype}, expected {want}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{where}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{where}: {name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{where}: {name} is on {t.device}, expected {device}")


def _require_gpu(where: str, dev):
    """Checked after the dtypes and shapes: the call's tensors, which share
    device ``dev``, must live on a GPU."""
    if dev.type != "cuda":
        raise ValueError(f"{where}: tensors must live on a GPU, not {dev}")
    return dev


def _check_gemv(where, w, x, residual, out, workspace, out_dtypes):
    """Checks of a qgemv / qgemm call's tensors; returns (device, m)."""
    dev = w.codes.device
    _tensor(where, "x", x, _BF16, None, dev)
    if x.dim() != 2 or x.shape[1] != w.k:
        raise ValueError(f"{where}: x has shape {tuple(x.shape)}, expected (m, {w.k})")
    m = x.shape[0]
    if residual is not None:
        _tensor(where, "residual", residual, _BF16, (m, w.n), dev)
    if out is not None:
        _tensor(where, "out", out, out_dtypes, (m, w.n), dev)
    if workspace is not None:
        _tensor(where, "workspace", workspace, _U8, None, dev)
    return _require_gpu(where, dev), m


_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_U8 = (torch.uint8,)
_OUT = (torch.float32, torch.bfloat16)


class Weight:
    """A packed weight (or batch of experts) resident on the device.

    Planes follow include/qmm.h: ``codes`` u8 [batch][n][k/2], ``codes_hi``
    u8 [batch][n][k/4] (Q6_K), ``scales`` (format dependent), ``scales2``
    f16 [batch][n][k/256] (Q6_K), ``tensor_scale`` f32 [batch] (NVFP4)."""

    # dtype of the ``scales`` plane and K values per scales element, per format
    _SCALES = {AFFINE4_G64: (torch.float16, 32), MXFP4: (torch.uint8, 32),
               NVFP4: (torch.uint8, 16), Q6_K: (torch.int8, 16)}

    def __init__(self, fmt: int, n: int, k: int, batch: int, codes, scales,
                 codes_hi=None, scales2=None, tensor_scale=None):
        self.fmt, self.n, self.k, self.batch = int(fmt), int(n), int(k), int(batch)
        if self.fmt not in self._SCALES:
            raise ValueError(f"Weight: unknown format {fmt}")
        if self.n < 1 or self.k < 1 or self.batch < 1:
            raise ValueError(f"Weight: n, k, batch must be >= 1, got {n}, {k}, {batch}")
        rows = self.batch * self.n
        sdt, per = self._SCALES[self.fmt]
        q6 = self.fmt == Q6_K
        planes = [("codes", codes, _U8, rows * self.k // 2),
                  ("scales", scales, (sdt,), rows * self.k // per)]
        if q6:
            planes += [("codes_hi", codes_hi, _U8, rows * self.k // 4),
                       ("scales2", scales2, (torch.float16,), rows * (self.k // 256))]
        elif codes_hi is not None or scales2 is not None:
            raise ValueError("Weight: codes_hi and scales2 belong to Q6_K only")
        if self.fmt == NVFP4:
            if tensor_scale is not None:
                planes.append(("tensor_scale", tensor_scale, _F32, self.batch))
        elif tensor_scale is not None:
            raise ValueError("Weight: tensor_scale belongs to NVFP4 only")
        for name, t, dts, numel in planes:
            if t is None:
                raise ValueError(f"Weight: plane {name} is missing")
            _tensor("Weight", name, t, dts, device=codes.device)
            if t.numel() != numel:
                raise ValueError(f"Weight: plane {name} holds {t.numel()} elements, expected "
                                 f"{numel} for format {fmt}, n={n}, k={k}, batch={batch}")
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
    dev = w.codes.device
    if out is None:
        out = torch.empty((w.batch, w.n, w.k), dtype=out_dtype, device=dev)
    _tensor("qdequant", "out", out, _OUT, (w.batch, w.n, w.k), dev)
    _require_gpu("qdequant", dev)
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qdequant(w.c, dt, _ptr(out), _stream(stream)), "qdequant")
    return out


def gemv_workspace_size(w: Weight, m: int) -> int:
    return int(_lib().qgemv_workspace_size(w.c, m))


def new_workspace(nbytes: int, device="cuda"):
    """A workspace of ``nbytes`` bytes (zero-filled here, though no call needs
    that: the library accepts any contents)."""
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def gemv(w: Weight, x, residual=None, y_dtype=torch.float32, out=None, workspace=None,
         stream=None):
    """y[m][n] = sum_k w[n][k] x[m][k] (+ residual), m = x.shape[0] in 1..4."""
    dev, m = _check_gemv("qgemv", w, x, residual, out, workspace, _OUT)
    if out is None:
        out = torch.empty((m, w.n), dtype=y_dtype, device=dev)
        _tensor("qgemv", "out", out, _OUT)  # y_dtype must be float32 or bfloat16
    need = gemv_workspace_size(w, m)
    if workspace is None and need:
        workspace = new_workspace(need, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qgemv(w.c, _ptr(x), m, _ptr(residual), _ptr(out), dt, _ptr(workspace),
                        ws_bytes, _stream(stream)), "qgemv")
    return out


def gemm(w: Weight, x, residual=None, out=None, workspace=None, stream=None):
    """y[m][n] = bf16(sum_k w16[n][k] x[m][k] (+ residual)), x bf16 [m][k]."""
    dev, m = _check_gemv("qgemm", w, x, residual, out, workspace, _BF16)
    if out is None:
        out = torch.empty((m, w.n), dtype=torch.bfloat16, device=dev)
    need = int(_lib().qgemm_workspace_size(w.c, m))
    if workspace is None and need:
        workspace = new_workspace(need, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().qgemm(w.c, _ptr(x), m, _ptr(residual), _ptr(out), _ptr(workspace), ws_bytes,
                        _stream(stream)), "qgemm")
    return out


def hadamard_prepare(x, in_scale=None, out=None, stream=None):
    """qhadamard_prepare: bf16 x [m][k] -> bf16 H (s_in * x) per 128-block."""
    _tensor("qhadamard_prepare", "x", x, _BF16)
    if x.dim() != 2:
        raise ValueError(f"qhadamard_prepare: x must be 2-D, got {tuple(x.shape)}")
    m, k = x.shape
    dev = x.device
    if in_scale is not None:
        _tensor("qhadamard_prepare", "in_scale", in_scale, (torch.float16,), (k,), dev)
    if out is not None:
        _tensor("qhadamard_prepare", "out", out, _BF16, (m, k), dev)
    _require_gpu("qhadamard_prepare", dev)
    if out is None:
        out = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
    _check(_lib().qhadamard_prepare(_ptr(x), m, k, _ptr(in_scale), _ptr(out), _stream(stream)),
           "qhadamard_prepare")
    return out


def hadamard_finish(y, out_scale=None, out=None, out_dtype=torch.float32, stream=None):
    """qhadamard_finish: float32 y [m][n] -> s_out * H y per 128-block."""
    _tensor("qhadamard_finish", "y", y, _F32)
    if y.dim() != 2:
        raise ValueError(f"qhadamard_finish: y must be 2-D, got {tuple(y.shape)}")
    m, n = y.shape
    dev = y.device
    if out_scale is not None:
        _tensor("qhadamard_finish", "out_scale", out_scale, (torch.float16,), (n,), dev)
    if out is not None:
        _tensor("qhadamard_finish", "out", out, _OUT, (m, n), dev)
    _require_gpu("qhadamard_finish", dev)
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=dev)
        _tensor("qhadamard_finish", "out", out, _OUT)
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qhadamard_finish(_ptr(y), m, n, _ptr(out_scale), _ptr(out), dt,
                                   _stream(stream)), "qhadamard_finish")
    return out


def gemv_hadamard(w: Weight, x, in_scale=None, out_scale=None, y_dtype=torch.float32, out=None,
                  workspace=None, stream=None):
    """qgemv_hadamard: y = finish(W . prepare(x)), prepare fused into the GEMV,
    x bf16 [m][k] raw activations, m in 1..4."""
    where = "qgemv_hadamard"
    dev = w.codes.device
    _tensor(where, "x", x, _BF16, None, dev)
    if x.dim() != 2 or x.shape[1] != w.k:
        raise ValueError(f"{where}: x has shape {tuple(x.shape)}, expected (m, {w.k})")
    m = x.shape[0]
    if in_scale is not None:
        _tensor(where, "in_scale", in_scale, (torch.float16,), (w.k,), dev)
    if out_scale is not None:
        _tensor(where, "out_scale", out_scale, (torch.float16,), (w.n,), dev)
    if out is not None:
        _tensor(where, "out", out, _OUT, (m, w.n), dev)
    if workspace is not None:
        _tensor(where, "workspace", workspace, _U8, None, dev)
    _require_gpu(where, dev)
    if out is None:
        out = torch.empty((m, w.n), dtype=y_dtype, device=dev)
        _tensor("qgemv_hadamard", "out", out, _OUT)
    dt = F32 if out.dtype == torch.float32 else BF16
    need = int(_lib().qgemv_hadamard_workspace_size(w.c, m, dt))
    if workspace is None and need:
        workspace = new_workspace(need, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().qgemv_hadamard(w.c, _ptr(x), m, _ptr(in_scale), _ptr(out_scale), _ptr(out), dt,
                                 _ptr(workspace), ws_bytes, _stream(stream)), "qgemv_hadamard")
    return out


def quant_mxfp4(x, codes=None, scales=None, stream=None):
    """qquant_mxfp4: bf16 x [m][k] -> (codes uint8 [m][k/2], E8M0 scales
    uint8 [m][k/32])."""
    _tensor("qquant_mxfp4", "x", x, _BF16)
    if x.dim() != 2:
        raise ValueError(f"qquant_mxfp4: x must be 2-D [m][k], got {tuple(x.shape)}")
    m, k = x.shape
    dev = x.device
    if codes is not None:
        _tensor("qquant_mxfp4", "codes", codes, _U8, (m, k // 2), dev)
    if scales is not None:
        _tensor("qquant_mxfp4", "scales", scales, _U8, (m, k // 32), dev)
    _require_gpu("qquant_mxfp4", dev)
    if codes is None:
        codes = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.uint8, device=dev)
    _check(_lib().qquant_mxfp4(_ptr(x), m, k, _ptr(codes), _ptr(scales), _stream(stream)),
           "qquant_mxfp4")
    return codes, scales


def gemm_w4a4_workspace_size(w: Weight, m: int) -> int:
    return int(_lib().qgemm_w4a4_workspace_size(w.c, m))


def gemm_w4a4(w: Weight, x, residual=None, out=None, workspace=None, stream=None):
    """W4A4: y[m][n] = bf16(sum_k w[n][k] q(x)[m][k] (+ residual)), MXFP4 w,
    x bf16 [m][k] quantized to MXFP4 on the GPU."""
    dev, m = _check_gemv("qgemm_w4a4", w, x, residual, out, workspace, _BF16)
    if out is None:
        out = torch.empty((m, w.n), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = torch.empty(max(gemm_w4a4_workspace_size(w, m), 1), dtype=torch.uint8,
                                device=dev)
    _check(_lib().qgemm_w4a4(w.c, _ptr(x), m, _ptr(residual), _ptr(out), _ptr(workspace),
                             workspace.numel(), _stream(stream)), "qgemm_w4a4")
    return out


def prepare_gemm_w4a4(w: Weight, x, out, residual=None, stream=None):
    _, m = _check_gemv("qgemm_w4a4", w, x, residual, out, None, _BF16)
    ws = torch.empty(max(gemm_w4a4_workspace_size(w, m), 1), dtype=torch.uint8, device=x.device)
    return _Prepared("qgemm_w4a4", (w.c, _ptr(x), m, _ptr(residual), _ptr(out), _ptr(ws),
                                    ws.numel(), _stream(stream)), (w, x, out, residual, ws))


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
    dev = _check_moe_routing("qmoe_grouped", gate_up, down, x, topk_ids, topk_w, shared_w, out)
    t, topk = topk_ids.shape
    if out is None:
        out = torch.empty((t, down.n), dtype=y_dtype, device=dev)
        _tensor("qmoe_grouped", "out", out, _OUT)
    if workspace is not None:
        _tensor("qmoe_grouped", "workspace", workspace, _U8, None, dev)
    need = moe_workspace_size(gate_up, down, num_routed, num_shared, t, topk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qmoe_grouped(gate_up.c, down.c, num_routed, num_shared, _ptr(x), t,
                               _ptr(topk_ids), _ptr(topk_w), topk, _ptr(shared_w), _ptr(out), dt,
                               _ptr(workspace), ws_bytes, _stream(stream)), "qmoe_grouped")
    return out


def _moe_check(where, gate_up, down, x, shared_w):
    dev = gate_up.codes.device
    if down.codes.device != dev:
        raise ValueError(f"{where}: gate_up and down weights are on different devices")
    _tensor(where, "x", x, _BF16, None, dev)
    if x.dim() != 2 or x.shape[1] != gate_up.k:
        raise ValueError(f"{where}: x has shape {tuple(x.shape)}, expected (t, {gate_up.k})")
    if shared_w is not None:
        _tensor(where, "shared_w", shared_w, _F32, (x.shape[0],), dev)
    return dev


def moe_noalloc(gate_up: Weight, down: Weight, x, topk_ids, topk_w, num_routed: int,
                num_shared: int, out, shared_w=None, stream=None):
    """qmoe_grouped_noalloc: one MoE layer into ``out`` (float32 or bf16
    [t][H], allocated by the caller) with the library's static scratch in
    place of a workspace; the call allocates nothing."""
    _check_moe_routing("qmoe_grouped_noalloc", gate_up, down, x, topk_ids, topk_w, shared_w, out)
    t, topk = topk_ids.shape
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qmoe_grouped_noalloc(gate_up.c, down.c, num_routed, num_shared, _ptr(x), t,
                                       _ptr(topk_ids), _ptr(topk_w), topk, _ptr(shared_w),
                                       _ptr(out), dt, _stream(stream)), "qmoe_grouped_noalloc")
    return out


def _check_moe_routing(where, gate_up, down, x, topk_ids, topk_w, shared_w, out):
    dev = _moe_check(where, gate_up, down, x, shared_w)
    _tensor(where, "topk_ids", topk_ids, _I32, None, dev)
    if topk_ids.dim() != 2 or topk_ids.shape[0] != x.shape[0]:
        raise ValueError(f"{where}: topk_ids has shape {tuple(topk_ids.shape)}, "
                         f"expected ({x.shape[0]}, topk)")
    _tensor(where, "topk_w", topk_w, _F32, tuple(topk_ids.shape), dev)
    if out is not None:
        _tensor(where, "out", out, _OUT, (x.shape[0], down.n), dev)
    return _require_gpu(where, dev)


def moe_router(logits, topk: int, ids=None, w=None, stream=None):
    """Router top-k and softmax: logits float32 [t][E] -> (ids int32 [t][topk],
    weights float32 [t][topk])."""
    _tensor("qmoe_router", "logits", logits, _F32)
    if logits.dim() != 2:
        raise ValueError(f"qmoe_router: logits must be 2-D [t][E], got {tuple(logits.shape)}")
    dev = logits.device
    t, e = logits.shape
    if ids is not None:
        _tensor("qmoe_router", "ids", ids, _I32, (t, topk), dev)
    if w is not None:
        _tensor("qmoe_router", "w", w, _F32, (t, topk), dev)
    _require_gpu("qmoe_router", dev)
    if ids is None:
        ids = torch.empty((t, topk), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((t, topk), dtype=torch.float32, device=dev)
    _check(_lib().qmoe_router(_ptr(logits), t, e, topk, _ptr(ids), _ptr(w), _stream(stream)),
           "qmoe_router")
    return ids, w


def moe_from_logits(gate_up: Weight, down: Weight, x, logits, topk: int, num_routed: int,
                    num_shared: int, shared_w=None, y_dtype=torch.float32, out=None,
                    workspace=None, stream=None):
    """One MoE layer from router logits float32 [t][num_routed]; returns (y,
    ids, weights)."""
    dev = _moe_check("qmoe_grouped_logits", gate_up, down, x, shared_w)
    t = x.shape[0]
    _tensor("qmoe_grouped_logits", "logits", logits, _F32, (t, num_routed), dev)
    if out is not None:
        _tensor("qmoe_grouped_logits", "out", out, _OUT, (t, down.n), dev)
    if workspace is not None:
        _tensor("qmoe_grouped_logits", "workspace", workspace, _U8, None, dev)
    _require_gpu("qmoe_grouped_logits", dev)
    if out is None:
        out = torch.empty((t, down.n), dtype=y_dtype, device=dev)
        _tensor("qmoe_grouped_logits", "out", out, _OUT)
    ids = torch.empty((t, topk), dtype=torch.int32, device=dev)
    w = torch.empty((t, topk), dtype=torch.float32, device=dev)
    need = moe_workspace_size(gate_up, down, num_routed, num_shared, t, topk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    dt = F32 if out.dtype == torch.float32 else BF16
    _check(_lib().qmoe_grouped_logits(gate_up.c, down.c, num_routed, num_shared, _ptr(x), t,
                                      _ptr(logits), topk, _ptr(ids), _ptr(w), _ptr(shared_w),
                                      _ptr(out), dt, _ptr(workspace), ws_bytes, _stream(stream)),
           "qmoe_grouped_logits")
    return out, ids, w


def workspace_init(ws, stream=None):
    _tensor("qworkspace_init", "ws", ws, _U8)
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
        _check_gemv("qgemv", w, x, residual, out, workspace, _OUT)
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
    _, m = _check_gemv("qgemm", w, x, residual, out, None, _BF16)
    need = int(_lib().qgemm_workspace_size(w.c, m))
    ws = new_workspace(need, x.device) if need else None
    ws_bytes = 0 if ws is None else ws.numel()
    return _Prepared("qgemm", (w.c, _ptr(x), m, _ptr(residual), _ptr(out), _ptr(ws), ws_bytes,
                               _stream(stream)), (w, x, out, residual, ws))


def prepare_moe(gate_up: Weight, down: Weight, x, topk_ids, topk_w, num_routed: int,
                num_shared: int, out, shared_w=None, stream=None):
    _check_moe_routing("qmoe_grouped", gate_up, down, x, topk_ids, topk_w, shared_w, out)
    t, topk = topk_ids.shape
    need = moe_workspace_size(gate_up, down, num_routed, num_shared, t, topk)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    dt = F32 if out.dtype == torch.float32 else BF16
    return _Prepared("qmoe_grouped",
                     (gate_up.c, down.c, num_routed, num_shared, _ptr(x), t, _ptr(topk_ids),
                      _ptr(topk_w), topk, _ptr(shared_w), _ptr(out), dt, _ptr(ws), ws.numel(),
                      _stream(stream)),
                     (gate_up, down, x, topk_ids, topk_w, out, shared_w, ws))
