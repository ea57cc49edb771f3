"""ctypes binding of libmoeq.so (argument marshalling only).

Every computation happens in the HIP kernels behind the C ABI declared in
``include/moeq.h``; this module only turns torch device tensors into the
ABI's plain pointers and sizes, allocates outputs and workspaces with torch,
and passes torch's current HIP stream.  If the library is missing the first
call raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOEQ_LIBRARY names another build of the same library (the AddressSanitizer
# build of the host front end, for the host tests of the boundary)
LIB_PATH = os.environ.get("MOEQ_LIBRARY") or os.path.join(_HERE, "lib", "libmoeq.so")

PATH_ROUTE, PATH_DECODE, PATH_GATHER, PATH_GQMM, PATH_FORWARD, PATH_FORWARD_NORM = 0, 1, 2, 3, 4, 5
MODE_AFFINE, MODE_MXFP4 = 0, 1

STATUS = {
    0: "MOEQ_OK", -1: "MOEQ_ERR_NULL_PTR", -2: "MOEQ_ERR_BAD_BITS", -3: "MOEQ_ERR_BAD_GROUP",
    -4: "MOEQ_ERR_K_TAIL", -5: "MOEQ_ERR_SHAPE", -6: "MOEQ_ERR_OVERFLOW", -7: "MOEQ_ERR_ALIGN",
    -8: "MOEQ_ERR_WORKSPACE", -9: "MOEQ_ERR_UNSUPPORTED", -10: "MOEQ_ERR_LAUNCH",
    -11: "MOEQ_ERR_HOST_MEMORY", -12: "MOEQ_ERR_TIMEOUT",
}
MOEQ_ERR_TIMEOUT = -12


class MoeqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_text(status)})")


class QTensorStruct(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group_size", ctypes.c_int32), ("mode", ctypes.c_int32)]


class MoEStruct(ctypes.Structure):
    _fields_ = [("router", QTensorStruct), ("gate", QTensorStruct), ("up", QTensorStruct),
                ("down", QTensorStruct), ("has_shared", ctypes.c_int32),
                ("sh_gate", QTensorStruct), ("sh_up", QTensorStruct), ("sh_down", QTensorStruct),
                ("sh_expert_gate", QTensorStruct)]


class SlotCacheStruct(ctypes.Structure):
    _fields_ = [("host", MoEStruct), ("slots", MoEStruct), ("slot_expert", ctypes.c_void_p),
                ("slot_stamp", ctypes.c_void_p), ("clock", ctypes.c_int64), ("n_slots", ctypes.c_int32)]


class SlotCacheDevStruct(ctypes.Structure):
    _fields_ = [("host", MoEStruct), ("slots", MoEStruct), ("slot_expert", ctypes.c_void_p),
                ("slot_stamp", ctypes.c_void_p), ("copy_list", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "moeq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moeq_version": (ctypes.c_char_p, []),
    "moe_workspace_size": (_SZ, [ctypes.POINTER(MoEStruct), _I, _I, _I]),
    "qdequant": (ctypes.c_int, [ctypes.POINTER(QTensorStruct), _P, _P, _P]),
    "qmatvec": (ctypes.c_int, [ctypes.POINTER(QTensorStruct), _P, _I, _P, _P]),
    "requant_2bit": (ctypes.c_int, [ctypes.POINTER(QTensorStruct), _P, _P, _P, _P]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(QTensorStruct), _P, _I, _I, _I, _I, _P, _P, _P,
                                 _P, _SZ, _P]),
    "moe_expert_forward": (ctypes.c_int, [ctypes.POINTER(MoEStruct), _P, _P, _P, _I, _I, _P, _P,
                                          _P, _SZ, _P]),
    "moe_forward": (ctypes.c_int, [ctypes.POINTER(MoEStruct), _P, _I, _I, _I, _P, _P, _P, _P, _P,
                                   _SZ, _P]),
    "moe_gather_qmm": (ctypes.c_int, [ctypes.POINTER(MoEStruct), _P, _P, _P, _I, _I, _P, _P, _SZ,
                                      _P]),
    "moe_rms_norm": (ctypes.c_int, [_P, _I, _I, _P, ctypes.c_float, _P, _P]),
    "moe_stream_experts": (ctypes.c_int, [ctypes.POINTER(SlotCacheStruct), _P, _I, _I, _P, _P, _P]),
    "moe_stream_experts_device": (ctypes.c_int, [ctypes.POINTER(SlotCacheDevStruct), _P, _I, _I, _P,
                                                 _P, _P]),
    "moe_forward_norm": (ctypes.c_int, [ctypes.POINTER(MoEStruct), _P, _I, _I, _I, _P, ctypes.c_float,
                                        _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "gather_qmm": (ctypes.c_int, [ctypes.POINTER(QTensorStruct), _P, _P, _I, _I, _P, _P, _SZ, _P]),
    "moe_workspace_status": (ctypes.c_int, [_P, _P, _P]),
    "moe_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(MoEStruct), _P, _I, _I, _I, _P, _P, _P, _P,
                                           _P, _P]),
}


def use_library(path: str) -> None:
    """Load the library from ``path`` instead of lib/libmoeq.so (e.g. the
    instrumented timeline build); only before the first call."""
    global LIB_PATH
    if _lib is not None:
        raise RuntimeError("libmoeq is already loaded")
    LIB_PATH = path


def lib() -> ctypes.CDLL:
    """Load libmoeq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m quantized_moe_expert_unpack_amd.build` (there is no fallback path)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _text(status: int) -> str:
    try:
        return lib().moeq_status_string(status).decode()
    except Exception:  # noqa: BLE001 - message only
        return "?"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MoeqError(status, what)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoeq takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoeq takes contiguous tensors")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

@dataclass
class QTensor:
    """A quantized matrix (or stack) resident on the device.  ``q`` holds the
    uint32 words as int32, ``scales``/``biases`` the bf16 bit patterns as int16
    (affine), or ``scales`` the E8M0 bytes as uint8 and no biases (mxfp4)."""
    q: torch.Tensor
    scales: torch.Tensor
    biases: Optional[torch.Tensor]
    batch: int
    rows: int
    cols: int
    bits: int
    group_size: int = 64
    mode: int = MODE_AFFINE

    def struct(self) -> QTensorStruct:
        return QTensorStruct(_ptr(self.q), _ptr(self.scales), _ptr(self.biases), self.batch,
                             self.rows, self.cols, self.bits, self.group_size, self.mode)

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.q, self.scales, self.biases)
                   if t is not None)

    @staticmethod
    def from_host(d: dict, device="cuda") -> "QTensor":
        q = np.ascontiguousarray(d["q"]).view(np.int32)
        if d.get("mode", "affine") == "mxfp4":
            s = np.ascontiguousarray(d["scales"]).astype(np.uint8, copy=False)
            return QTensor(torch.from_numpy(q).to(device), torch.from_numpy(s).to(device), None,
                           int(d.get("batch", 1)), int(d["rows"]), int(d["cols"]), 4, 32,
                           MODE_MXFP4)
        s = np.ascontiguousarray(d["scales"]).view(np.int16)
        b = np.ascontiguousarray(d["biases"]).view(np.int16)
        return QTensor(torch.from_numpy(q).to(device), torch.from_numpy(s).to(device),
                       torch.from_numpy(b).to(device), int(d.get("batch", 1)), int(d["rows"]),
                       int(d["cols"]), int(d["bits"]), int(d.get("group_size", 64)))


def _empty_qt() -> QTensorStruct:
    return QTensorStruct(None, None, None, 0, 0, 0, 0, 0)


@dataclass
class MoELayer:
    """One MoE layer on the device (router, expert stacks, optional shared expert)."""
    router: Optional[QTensor]
    gate: QTensor
    up: QTensor
    down: QTensor
    shared: Optional[dict] = None      # {"gate","up","down","expert_gate"} -> QTensor
    _struct: Optional[MoEStruct] = field(default=None, repr=False)

    def struct(self) -> MoEStruct:
        if self._struct is None:
            sh = self.shared
            self._struct = MoEStruct(
                self.router.struct() if self.router is not None else _empty_qt(),
                self.gate.struct(), self.up.struct(), self.down.struct(), 1 if sh else 0,
                sh["gate"].struct() if sh else _empty_qt(),
                sh["up"].struct() if sh else _empty_qt(),
                sh["down"].struct() if sh else _empty_qt(),
                sh["expert_gate"].struct() if sh else _empty_qt())
        return self._struct

    @property
    def experts(self) -> int:
        return self.gate.batch

    @property
    def hidden(self) -> int:
        return self.gate.cols

    def requantized_2bit(self, stream=None) -> "MoELayer":
        """The layer with its routed and shared experts requantized to 2 bits
        on the device (requant_2bit, one launch per stack); the router and
        the shared expert gate are kept as they are."""
        sh = None
        if self.shared is not None:
            sh = {k: requant_2bit(v, stream) for k, v in self.shared.items() if k != "expert_gate"}
            sh["expert_gate"] = self.shared["expert_gate"]
        return MoELayer(self.router, requant_2bit(self.gate, stream), requant_2bit(self.up, stream),
                        requant_2bit(self.down, stream), sh)

    @staticmethod
    def from_host(layer: dict, device="cuda") -> "MoELayer":
        sh = None
        if layer.get("shared") is not None:
            sh = {k: QTensor.from_host(v, device) for k, v in layer["shared"].items()}
        router = QTensor.from_host(layer["router"], device) if layer.get("router") is not None else None
        return MoELayer(router, QTensor.from_host(layer["gate"], device),
                        QTensor.from_host(layer["up"], device),
                        QTensor.from_host(layer["down"], device), sh)


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def version() -> str:
    return lib().moeq_version().decode()


def workspace_size(layer: MoELayer, m: int, k: int, path: int) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(layer.struct()), m, k, path))


_DECODE_PATHS = (PATH_DECODE, PATH_FORWARD, PATH_FORWARD_NORM)
_tracked: Optional[list] = None


def workspace(layer: MoELayer, m: int, k: int, path: int, device="cuda") -> torch.Tensor:
    """A zeroed workspace of the size the library asks for (256-byte aligned:
    torch's caching allocator returns 512-byte aligned blocks)."""
    n = workspace_size(layer, m, k, path)
    if n == 0:
        raise MoeqError(-5, "moe_workspace_size")
    ws = torch.zeros(n, dtype=torch.uint8, device=device)
    if _tracked is not None and path in _DECODE_PATHS:
        _tracked.append(ws)
    return ws


def workspace_status(ws: torch.Tensor, stream=None) -> tuple:
    """(status, bits) of a decode-family workspace's error word, which is
    cleared (moe_workspace_status; synchronizes the host with the stream)."""
    out = torch.zeros(4, dtype=torch.int32, device=ws.device)
    _check(lib().moe_workspace_status(_ptr(ws), _ptr(out), _stream(stream)), "moe_workspace_status")
    st, bits = out[:2].tolist()
    return int(st), int(bits)


def track_workspaces(on: bool) -> None:
    """Start (and empty) or stop the record of the decode-family workspaces
    that workspace() makes, explicit ones and those the calls below make for
    themselves; check_workspaces() reads their error words."""
    global _tracked
    _tracked = [] if on else None


def check_workspaces() -> None:
    """Raise MoeqError(MOEQ_ERR_TIMEOUT) if a bounded wait gave up in any call
    on a recorded workspace (each error word is read and cleared)."""
    for ws in list(_tracked or []):
        st, bits = workspace_status(ws)
        if st != 0:
            raise MoeqError(st, f"decode workspace error word 0x{bits:x}")


def qdequant(W: QTensor, codes: bool = True, deq: bool = True, stream=None):
    dev = W.q.device
    shape = (W.batch, W.rows, W.cols)
    c = torch.empty(shape, dtype=torch.uint8, device=dev) if codes else None
    d = torch.empty(shape, dtype=torch.float32, device=dev) if deq else None
    _check(lib().qdequant(ctypes.byref(W.struct()), _ptr(c), _ptr(d), _stream(stream)), "qdequant")
    return c, d


def requant_2bit(W: QTensor, stream=None) -> QTensor:
    """2-bit requantization of a 4- or 8-bit tensor (same shape and group size)."""
    dev = W.q.device
    ng = W.cols // W.group_size
    q = torch.empty((W.batch, W.rows, W.cols // 16), dtype=torch.int32, device=dev)
    s = torch.empty((W.batch, W.rows, ng), dtype=torch.int16, device=dev)
    b = torch.empty((W.batch, W.rows, ng), dtype=torch.int16, device=dev)
    _check(lib().requant_2bit(ctypes.byref(W.struct()), _ptr(q), _ptr(s), _ptr(b), _stream(stream)),
           "requant_2bit")
    return QTensor(q, s, b, W.batch, W.rows, W.cols, 2, W.group_size)


def qmatvec(W: QTensor, x: torch.Tensor, y: Optional[torch.Tensor] = None, stream=None):
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, W.rows), dtype=torch.float32, device=x.device)
    _check(lib().qmatvec(ctypes.byref(W.struct()), _ptr(x), m, _ptr(y), _stream(stream)), "qmatvec")
    return y


def moe_route(gate: Optional[QTensor], x_or_logits: torch.Tensor, experts: int, k: int,
              renorm: bool = True, ws: Optional[torch.Tensor] = None,
              idx: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
              logits_out: Optional[torch.Tensor] = None, stream=None):
    m = x_or_logits.shape[0]
    dev = x_or_logits.device
    if idx is None:
        idx = torch.empty((m, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((m, k), dtype=torch.float32, device=dev)
    if gate is not None and ws is None:
        # the size the library asks for (a layer struct holding only the router)
        only = MoEStruct(gate.struct(), _empty_qt(), _empty_qt(), _empty_qt(), 0,
                         _empty_qt(), _empty_qt(), _empty_qt(), _empty_qt())
        n = int(lib().moe_workspace_size(ctypes.byref(only), m, k, PATH_ROUTE))
        if n == 0:
            raise MoeqError(-5, "moe_workspace_size")
        ws = torch.zeros(n, dtype=torch.uint8, device=dev)
    gs = ctypes.byref(gate.struct()) if gate is not None else None
    _check(lib().moe_route(gs, _ptr(x_or_logits), m, experts, k, 1 if renorm else 0, _ptr(idx),
                           _ptr(w), _ptr(logits_out), _ptr(ws),
                           ws.numel() if ws is not None else 0, _stream(stream)), "moe_route")
    return idx, w


def moe_expert_forward(layer: MoELayer, x: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                       residual: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                       y: Optional[torch.Tensor] = None, stream=None):
    m, k = idx.shape
    if ws is None:
        ws = workspace(layer, m, k, PATH_DECODE, x.device)
    if y is None:
        y = torch.empty((m, layer.hidden), dtype=torch.float32, device=x.device)
    _check(lib().moe_expert_forward(ctypes.byref(layer.struct()), _ptr(x), _ptr(idx), _ptr(w), m,
                                    k, _ptr(residual), _ptr(y), _ptr(ws), ws.numel(),
                                    _stream(stream)), "moe_expert_forward")
    return y


def moe_forward(layer: MoELayer, x: torch.Tensor, k: int, renorm: bool = True,
                residual: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                y: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                w: Optional[torch.Tensor] = None, stream=None):
    """Router + top-K + experts (one launch for an 8-bit router and M <= 4).
    Returns (y, idx, w)."""
    m = x.shape[0]
    dev = x.device
    if ws is None:
        ws = workspace(layer, m, k, PATH_FORWARD, dev)
    if y is None:
        y = torch.empty((m, layer.hidden), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((m, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((m, k), dtype=torch.float32, device=dev)
    _check(lib().moe_forward(ctypes.byref(layer.struct()), _ptr(x), m, k, int(bool(renorm)),
                             _ptr(residual), _ptr(y), _ptr(idx), _ptr(w), _ptr(ws), ws.numel(),
                             _stream(stream)), "moe_forward")
    return y, idx, w


def moe_forward_noalloc(layer: MoELayer, x: torch.Tensor, k: int, renorm: bool = True,
                        residual: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                        idx: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
                        status: Optional[torch.Tensor] = None, stream=None):
    """moe_forward on the library's static per-device workspace (no
    workspace argument).  ``status``: optional device int32 [>= 2] that
    receives the call's timeout status.  Returns (y, idx, w)."""
    m = x.shape[0]
    dev = x.device
    if y is None:
        y = torch.empty((m, layer.hidden), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((m, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((m, k), dtype=torch.float32, device=dev)
    _check(lib().moe_forward_noalloc(ctypes.byref(layer.struct()), _ptr(x), m, k, int(bool(renorm)),
                                     _ptr(residual), _ptr(y), _ptr(idx), _ptr(w), _ptr(status),
                                     _stream(stream)), "moe_forward_noalloc")
    return y, idx, w


def moe_rms_norm(x: torch.Tensor, norm_w: torch.Tensor, eps: float,
                 h: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """h = x / sqrt(mean(x^2) + eps) * norm_w per row (fp32)."""
    m, hdim = x.shape
    if h is None:
        h = torch.empty_like(x)
    _check(lib().moe_rms_norm(_ptr(x), m, hdim, _ptr(norm_w), float(eps), _ptr(h), _stream(stream)),
           "moe_rms_norm")
    return h


def moe_forward_norm(layer: MoELayer, x: torch.Tensor, k: int, norm_w: torch.Tensor, eps: float,
                     renorm: bool = True, ws: Optional[torch.Tensor] = None,
                     y: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                     w: Optional[torch.Tensor] = None, stream=None,
                     post_norm_w: Optional[torch.Tensor] = None,
                     y_norm: Optional[torch.Tensor] = None):
    """y = x + MoE(rms_norm(x)) (one launch for an 8-bit router and M <= 4).
    Returns (y, idx, w); with ``post_norm_w`` also the norm after the combine,
    rms_norm(y) * post_norm_w: (y, idx, w, y_norm)."""
    m = x.shape[0]
    dev = x.device
    if post_norm_w is not None and y_norm is None:
        y_norm = torch.empty((m, layer.hidden), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(layer, m, k, PATH_FORWARD_NORM, dev)
    if y is None:
        y = torch.empty((m, layer.hidden), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((m, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((m, k), dtype=torch.float32, device=dev)
    _check(lib().moe_forward_norm(ctypes.byref(layer.struct()), _ptr(x), m, k, int(bool(renorm)),
                                  _ptr(norm_w), float(eps), _ptr(y), _ptr(idx), _ptr(w),
                                  _ptr(post_norm_w), _ptr(y_norm), _ptr(ws), ws.numel(),
                                  _stream(stream)), "moe_forward_norm")
    return (y, idx, w) if post_norm_w is None else (y, idx, w, y_norm)


class ExpertCache:
    """Experts of one layer held in pinned host memory and S device slots
    (the buffers moe_stream_experts manages; allocated here with torch).
    ``layer`` is the device layer to run moe_expert_forward on: the slot
    stacks as its experts, the resident router and shared expert of
    ``resident``.  With ``device_lru`` the slot choice and the copies run on
    the device (``stream_device``, moe_stream_experts_device), else on the
    host (``stream``); one cache uses one of the two."""

    def __init__(self, host_layer: dict, n_slots: int, resident: "MoELayer", device="cuda",
                 device_lru: bool = False):
        def pinned(a):
            a = np.ascontiguousarray(a)
            t = torch.empty(a.shape, dtype=_TORCH_OF[a.dtype.str[1:]], pin_memory=True)
            t.copy_(torch.from_numpy(a.view(_VIEW_OF[a.dtype.str[1:]])))
            return t

        self.host = {}
        self.slots = {}
        for name in ("gate", "up", "down"):
            d = host_layer[name]
            q, sc = np.asarray(d["q"]), np.asarray(d["scales"])
            b = None if d.get("biases") is None else np.asarray(d["biases"])
            mode = MODE_MXFP4 if d.get("mode", "affine") == "mxfp4" else MODE_AFFINE
            E, rows, cols = int(d["batch"]), int(d["rows"]), int(d["cols"])
            self.host[name] = QTensor(pinned(q), pinned(sc), None if b is None else pinned(b), E, rows,
                                      cols, int(d["bits"]), int(d["group_size"]), mode)
            h = self.host[name]
            self.slots[name] = QTensor(
                torch.empty((n_slots,) + tuple(h.q.shape[1:]), dtype=h.q.dtype, device=device),
                torch.empty((n_slots,) + tuple(h.scales.shape[1:]), dtype=h.scales.dtype, device=device),
                None if h.biases is None else
                torch.empty((n_slots,) + tuple(h.biases.shape[1:]), dtype=h.biases.dtype, device=device),
                n_slots, rows, cols, h.bits, h.group_size, mode)
        self.n_slots = n_slots
        self.slot_expert = np.full(n_slots, -1, np.int32)
        self.slot_stamp = np.zeros(n_slots, np.int64)
        self.layer = MoELayer(resident.router, self.slots["gate"], self.slots["up"], self.slots["down"],
                              resident.shared)
        self._host_layer = MoELayer(None, self.host["gate"], self.host["up"], self.host["down"])
        self._cs = SlotCacheStruct(_host_struct(self._host_layer), _host_struct(
            MoELayer(None, self.slots["gate"], self.slots["up"], self.slots["down"])),
            self.slot_expert.ctypes.data, self.slot_stamp.ctypes.data, 0, n_slots)
        self.device_lru = bool(device_lru)
        if self.device_lru:
            self.slot_expert_dev = torch.full((n_slots,), -1, dtype=torch.int32, device=device)
            self.slot_stamp_dev = torch.zeros(n_slots + 1, dtype=torch.int64, device=device)
            self.copy_list = torch.zeros(2 * n_slots + 4, dtype=torch.int32, device=device)
            self._csd = SlotCacheDevStruct(
                self._cs.host, self._cs.slots, self.slot_expert_dev.data_ptr(),
                self.slot_stamp_dev.data_ptr(), self.copy_list.data_ptr(), n_slots)

    def stream(self, topk_idx_host: np.ndarray, stream=None):
        """Copy the experts ``topk_idx_host`` selects into slots (async on the
        stream); returns (slot indices [M][K] int32 host array, experts copied)."""
        if self.device_lru:
            raise ValueError("this cache keeps its LRU on the device: use stream_device")
        idx = np.ascontiguousarray(topk_idx_host, dtype=np.int32)
        m, k = idx.shape
        out = np.empty_like(idx)
        n = ctypes.c_int32(0)
        _check(lib().moe_stream_experts(ctypes.byref(self._cs), idx.ctypes.data, m, k,
                                        out.ctypes.data, ctypes.byref(n), _stream(stream)),
               "moe_stream_experts")
        return out, n.value

    def stream_device(self, topk_idx: torch.Tensor, slot_idx: Optional[torch.Tensor] = None,
                      n_copied: Optional[torch.Tensor] = None, stream=None):
        """Device-side form: ``topk_idx`` is moe_route's device output; the
        slot choice and the copies are queued on the stream with no host
        synchronization.  Returns (slot indices [M][K] int32, experts copied
        as a device int32 [1]), both device tensors."""
        if not self.device_lru:
            raise ValueError("this cache keeps its LRU on the host: use stream")
        m, k = topk_idx.shape
        if slot_idx is None:
            slot_idx = torch.empty((m, k), dtype=torch.int32, device=topk_idx.device)
        if n_copied is None:
            n_copied = torch.zeros(4, dtype=torch.int32, device=topk_idx.device)
        _check(lib().moe_stream_experts_device(ctypes.byref(self._csd), _ptr(topk_idx), m, k,
                                               _ptr(slot_idx), _ptr(n_copied), _stream(stream)),
               "moe_stream_experts_device")
        return slot_idx, n_copied[:1]


_TORCH_OF = {"u4": torch.int32, "u2": torch.int16, "u1": torch.uint8, "i4": torch.int32,
             "i2": torch.int16}
_VIEW_OF = {"u4": np.int32, "u2": np.int16, "u1": np.uint8, "i4": np.int32, "i2": np.int16}


def _host_struct(layer: "MoELayer") -> MoEStruct:
    """MoEStruct of expert stacks whose tensors may live in pinned host memory."""
    def qs(t: QTensor) -> QTensorStruct:
        ptr = lambda a: None if a is None else a.data_ptr()
        return QTensorStruct(ptr(t.q), ptr(t.scales), ptr(t.biases), t.batch, t.rows, t.cols,
                             t.bits, t.group_size, t.mode)
    return MoEStruct(_empty_qt(), qs(layer.gate), qs(layer.up), qs(layer.down), 0,
                     _empty_qt(), _empty_qt(), _empty_qt(), _empty_qt())


def moe_gather_qmm(layer: MoELayer, x_bf16: torch.Tensor, idx: torch.Tensor, w: torch.Tensor,
                   ws: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                   stream=None):
    m, k = idx.shape
    if ws is None:
        ws = workspace(layer, m, k, PATH_GATHER, x_bf16.device)
    if y is None:
        y = torch.empty((m, layer.hidden), dtype=torch.float32, device=x_bf16.device)
    _check(lib().moe_gather_qmm(ctypes.byref(layer.struct()), _ptr(x_bf16), _ptr(idx), _ptr(w), m,
                                k, _ptr(y), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_gather_qmm")
    return y


def gather_qmm(W: QTensor, x_bf16: torch.Tensor, rhs_idx: torch.Tensor, sorted_indices=False,
               ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, stream=None):
    n = rhs_idx.shape[0]
    if ws is None:
        probe = MoELayer(None, W, W, W)
        ws = workspace(probe, n, 1, PATH_GQMM, x_bf16.device)
    if out is None:
        out = torch.empty((n, W.rows), dtype=torch.float32, device=x_bf16.device)
    _check(lib().gather_qmm(ctypes.byref(W.struct()), _ptr(x_bf16), _ptr(rhs_idx), n,
                            1 if sorted_indices else 0, _ptr(out), _ptr(ws), ws.numel(),
                            _stream(stream)), "gather_qmm")
    return out
