"""ctypes binding of libmoe.so.

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  PyTorch supplies device memory and the current stream.  If the
library is not built, importing this module raises ImportError; there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_ENOTPINNED, MOE_ECAPACITY = range(7)
MOE_F32, MOE_BF16 = 0, 1
PATHS = {"auto": 0, "gemv": 1, "mfma": 2}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class QLayer(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int), ("bits", ctypes.c_int),
                ("base", ctypes.c_void_p), ("stride", ctypes.c_int64), ("slot_map", ctypes.c_void_p)]


class SlotStats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64), ("bytes_h2d", ctypes.c_uint64),
                ("resolves", ctypes.c_uint64), ("evictions", ctypes.c_uint64)]


COPY_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m expert_routed_ffn_amd.build` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    st = ctypes.c_int
    L.moe_abi_version.restype = i32
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [st]
    L.moe_expert_bytes.restype = sz
    L.moe_expert_bytes.argtypes = [i32, i32, i32]
    L.moe_route_topk.restype = st
    L.moe_route_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    L.moe_router_logits.restype = st
    L.moe_router_logits.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp]
    L.moe_router_topk.restype = st
    L.moe_router_topk.argtypes = [vp, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp]
    L.moe_dispatch_workspace_bytes.restype = sz
    L.moe_dispatch_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_dispatch.restype = st
    L.moe_dispatch.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn_workspace_bytes.restype = sz
    L.moe_expert_ffn_workspace_bytes.argtypes = [ctypes.POINTER(QLayer), i32, i32, i32]
    L.moe_expert_ffn_q.restype = st
    L.moe_expert_ffn_q.argtypes = [ctypes.POINTER(QLayer), vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, i32, vp, sz,
                                   vp]
    L.moe_combine.restype = st
    L.moe_combine.argtypes = [vp, i32, vp, i32, i32, i32, vp, i32, vp, vp, vp]
    L.moe_slot_table_create.restype = st
    L.moe_slot_table_create.argtypes = [i32, i32, i32, sz, vp, vp, vp, vp, ctypes.POINTER(vp)]
    L.moe_slot_table_preload.restype = st
    L.moe_slot_table_preload.argtypes = [vp, vp, i32, vp]
    L.moe_slot_table_resolve.restype = st
    L.moe_slot_table_resolve.argtypes = [vp, i32, vp, vp, vp]
    L.moe_slot_table_stats.restype = st
    L.moe_slot_table_stats.argtypes = [vp, ctypes.POINTER(SlotStats)]
    L.moe_slot_table_map_host.restype = st
    L.moe_slot_table_map_host.argtypes = [vp, vp]
    L.moe_slot_table_device_bytes.restype = sz
    L.moe_slot_table_device_bytes.argtypes = [i32, i32, i32]
    L.moe_slot_table_enable_device.restype = st
    L.moe_slot_table_enable_device.argtypes = [vp, vp, sz, vp]
    L.moe_slot_table_resolve_device.restype = st
    L.moe_slot_table_resolve_device.argtypes = [vp, i32, vp, vp, i32, vp]
    L.moe_slot_table_destroy.restype = None
    L.moe_slot_table_destroy.argtypes = [vp]
    L.moe_slot_table_create_host.restype = st
    L.moe_slot_table_create_host.argtypes = [i32, i32, i32, COPY_FN, vp, ctypes.POINTER(vp)]
    L.moe_slot_table_resolve_host.restype = st
    L.moe_slot_table_resolve_host.argtypes = [vp, i32, vp, i32]
    L.moe_layer_decode_workspace_bytes.restype = sz
    L.moe_layer_decode_workspace_bytes.argtypes = [ctypes.POINTER(QLayer), i32, i32]
    L.moe_layer_decode.restype = st
    L.moe_layer_decode.argtypes = [ctypes.POINTER(QLayer), vp, vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                   vp, i32, vp, vp, vp, sz, vp]
    L.moe_layer_decode_noalloc_max_bytes.restype = sz
    L.moe_layer_decode_noalloc_max_bytes.argtypes = []
    L.moe_layer_decode_noalloc.restype = st
    L.moe_layer_decode_noalloc.argtypes = [ctypes.POINTER(QLayer), vp, vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp,
                                           vp, vp, vp, i32, vp, vp, vp]
    L.moe_layer_decode_slots.restype = st
    L.moe_layer_decode_slots.argtypes = [ctypes.POINTER(QLayer), vp, i32, vp, vp, i32, i32, i32, vp, i32, vp, vp, vp,
                                         vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    L.moe_profile_next_launch.restype = st
    L.moe_profile_next_launch.argtypes = [i32, vp, vp]
    return L


lib = _load()


def header_functions() -> list[str]:
    """Names of the functions include/moe.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)) - {"moe_copy_fn"})


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib.moe_last_error().decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device=None):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _on(stream, device):
    """Context in which the binding allocates outputs and workspaces: the stream the kernels run on, so the
    caching allocator does not hand their memory to other work while the kernels are still queued."""
    import contextlib
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=device)
    return torch.cuda.stream(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


KERNELS = {"route": 0, "dispatch": 1, "gemv_gateup": 2, "gemv_down": 3, "mfma_gateup": 4, "mfma_down": 5,
           "combine": 6, "decode_prep": 7, "router": 8}


def profile_next_launch(kernel: str, start, stop):
    """Attach HIP events (raw hipEvent_t handles) to the next launch of `kernel` on this thread."""
    _check(lib.moe_profile_next_launch(KERNELS[kernel], ctypes.c_void_p(int(getattr(start, "value", start))),
                                       ctypes.c_void_p(int(getattr(stop, "value", stop)))))


def abi_version() -> int:
    return int(lib.moe_abi_version())


def expert_bytes(H: int, I: int, bits: int) -> int:
    return int(lib.moe_expert_bytes(H, I, bits))


# ---- moe_route_topk --------------------------------------------------------------

def route_topk(logits: torch.Tensor, k: int, ids: torch.Tensor | None = None, w: torch.Tensor | None = None,
               stream=None):
    _need(logits, "logits")
    T, E = logits.shape
    with _on(stream, logits.device):
        if ids is None:
            ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
        if w is None:
            w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib.moe_route_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream, logits.device)))
    return ids, w


# ---- router projection ----------------------------------------------------------------

def router_logits(x: torch.Tensor, w_r: torch.Tensor, logits: torch.Tensor | None = None, stream=None):
    """logits [T, E] fp32 = x [T, H] (fp32 or bf16) . w_r [E, H] (bf16)^T."""
    _need(x, "x")
    _need(w_r, "w_r")
    if w_r.dtype != torch.bfloat16:
        raise TypeError("w_r must be bfloat16")
    T, H = x.shape
    E = w_r.shape[0]
    with _on(stream, x.device):
        if logits is None:
            logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check(lib.moe_router_logits(_ptr(x), _dtype_code(x), _ptr(w_r), T, H, E, _ptr(logits),
                                 _stream(stream, x.device)))
    return logits


def router_topk(x: torch.Tensor, w_r: torch.Tensor, k: int, logits: torch.Tensor | None = None,
                ids: torch.Tensor | None = None, w: torch.Tensor | None = None, stream=None):
    """Router projection then top-k: (logits, ids, w)."""
    _need(x, "x")
    _need(w_r, "w_r")
    T, H = x.shape
    E = w_r.shape[0]
    dev = x.device
    with _on(stream, dev):
        if logits is None:
            logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        if ids is None:
            ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        if w is None:
            w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib.moe_router_topk(_ptr(x), _dtype_code(x), _ptr(w_r), T, H, E, k, _ptr(logits), _ptr(ids), _ptr(w),
                               _stream(stream, dev)))
    return logits, ids, w


# ---- moe_dispatch ------------------------------------------------------------------

class Dispatch:
    """Device outputs of moe_dispatch."""

    def __init__(self, T: int, k: int, E: int, device):
        n = T * k
        self.T, self.k, self.E = T, k, E
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.sorted_assign = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        self.assign_pos = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        self.active = torch.empty(max(min(E, n), 1), dtype=torch.int32, device=device)
        self.n_active = torch.empty(1, dtype=torch.int32, device=device)
        nb = int(lib.moe_dispatch_workspace_bytes(T, k, E))
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=device)


def dispatch(ids: torch.Tensor, E: int, out: Dispatch | None = None, stream=None) -> Dispatch:
    _need(ids, "ids")
    T, k = ids.shape
    with _on(stream, ids.device):
        d = out if out is not None else Dispatch(T, k, E, ids.device)
    _check(lib.moe_dispatch(_ptr(ids), T, k, E, _ptr(d.offsets), _ptr(d.sorted_assign), _ptr(d.assign_pos),
                            _ptr(d.active), _ptr(d.n_active), _ptr(d.ws), d.ws.numel(), _stream(stream, ids.device)))
    return d


# ---- moe_expert_ffn_q ------------------------------------------------------------

class ExpertLayer:
    """One layer's quantized experts in device memory: expert e's blob at base + idx(e) * stride."""

    def __init__(self, E: int, H: int, I: int, bits: int, base: torch.Tensor, stride: int | None = None,
                 slot_map: torch.Tensor | None = None, base_offset: int = 0):
        _need(base, "base")
        self.E, self.H, self.I, self.bits = E, H, I, bits
        self.base = base  # keeps the storage alive
        self.stride = stride if stride is not None else expert_bytes(H, I, bits)
        self.slot_map = slot_map
        self.q = QLayer(E, H, I, bits, base.data_ptr() + base_offset, self.stride,
                        None if slot_map is None else slot_map.data_ptr())

    def workspace_bytes(self, T: int, k: int, path: str = "auto") -> int:
        return int(lib.moe_expert_ffn_workspace_bytes(ctypes.byref(self.q), T, k, PATHS[path]))


def expert_ffn_q(layer: ExpertLayer, x: torch.Tensor, k: int, d: Dispatch, y: torch.Tensor | None = None,
                 y_dtype=torch.float32, path: str = "auto", ws: torch.Tensor | None = None, stream=None):
    _need(x, "x")
    T, H = x.shape
    with _on(stream, x.device):
        if y is None:
            y = torch.empty((T, k, H), dtype=y_dtype, device=x.device)
        if ws is None:
            ws = torch.empty(max(layer.workspace_bytes(T, k, path), 1), dtype=torch.uint8, device=x.device)
    _need(y, "y")
    _check(lib.moe_expert_ffn_q(ctypes.byref(layer.q), _ptr(x), _dtype_code(x), T, k, _ptr(d.offsets),
                                _ptr(d.sorted_assign), _ptr(d.active), _ptr(d.n_active), _ptr(y), _dtype_code(y),
                                PATHS[path], _ptr(ws), ws.numel(), _stream(stream, x.device)))
    return y


# ---- moe_combine -------------------------------------------------------------------

def combine(y: torch.Tensor, w: torch.Tensor, residual: torch.Tensor | None = None, out: torch.Tensor | None = None,
            out_bf16: torch.Tensor | None = None, stream=None):
    _need(y, "y")
    _need(w, "w")
    T, k, H = y.shape
    with _on(stream, y.device):
        if out is None:
            out = torch.empty((T, H), dtype=torch.float32, device=y.device)
    r_t = MOE_F32 if residual is None else _dtype_code(residual)
    _check(lib.moe_combine(_ptr(y), _dtype_code(y), _ptr(w), T, k, H, _ptr(residual), r_t, _ptr(out),
                           _ptr(out_bf16), _stream(stream, y.device)))
    return out


# ---- whole layer (four calls in order) ---------------------------------------------

def layer_forward(layer: ExpertLayer, x: torch.Tensor, logits: torch.Tensor, k: int, residual=None,
                  y_dtype=torch.float32, path: str = "auto", out_bf16: torch.Tensor | None = None, bufs=None,
                  stream=None):
    """route -> dispatch -> expert FFN -> combine.  Returns (ids, w, dispatch, y, out)."""
    T = x.shape[0]
    if bufs is None:
        bufs = {}
    ids, w = route_topk(logits, k, bufs.get("ids"), bufs.get("w"), stream)
    d = dispatch(ids, layer.E, bufs.get("dispatch"), stream)
    y = expert_ffn_q(layer, x, k, d, bufs.get("y"), y_dtype, path, bufs.get("ws"), stream)
    out = combine(y, w, residual, bufs.get("out"), out_bf16, stream)
    return ids, w, d, y, out


# ---- fused decode step ------------------------------------------------------------

def _decode_buffers(layer, T, k, H, y_dtype, b, stream, dev):
    """Outputs and workspace of a decode step: the caller's from `b`, the rest allocated on `stream`."""
    with _on(stream, dev):
        ids = b.get("ids")
        if ids is None:
            ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = b.get("w")
        if w is None:
            w = torch.empty((T, k), dtype=torch.float32, device=dev)
        d = b.get("dispatch") or Dispatch(T, k, layer.E, dev)
        y = b.get("y")
        if y is None:
            y = torch.empty((T, k, H), dtype=y_dtype, device=dev)
        out = b.get("out")
        if out is None:
            out = torch.empty((T, H), dtype=torch.float32, device=dev)
        ws = b.get("dws")
        if ws is None:
            ws = torch.empty(max(int(lib.moe_layer_decode_workspace_bytes(ctypes.byref(layer.q), T, k)), 1),
                             dtype=torch.uint8, device=dev)
    return ids, w, d, y, out, ws


def layer_decode(layer: ExpertLayer, x: torch.Tensor, logits: torch.Tensor, k: int, residual=None,
                 y_dtype=torch.float32, out_bf16: torch.Tensor | None = None, bufs=None, stream=None):
    """moe_layer_decode: the whole layer step (two launches for the decode shapes, else four).  Returns (ids, w, dispatch, y, out)."""
    _need(x, "x")
    _need(logits, "logits")
    T, H = x.shape
    dev = x.device
    ids, w, d, y, out, ws = _decode_buffers(layer, T, k, H, y_dtype, bufs or {}, stream, dev)
    r_t = MOE_F32 if residual is None else _dtype_code(residual)
    _check(lib.moe_layer_decode(ctypes.byref(layer.q), _ptr(logits), _ptr(x), _dtype_code(x), T, k, _ptr(residual),
                                r_t, _ptr(ids), _ptr(w), _ptr(d.offsets), _ptr(d.sorted_assign), _ptr(d.assign_pos),
                                _ptr(d.active), _ptr(d.n_active), _ptr(y), _dtype_code(y), _ptr(out), _ptr(out_bf16),
                                _ptr(ws), ws.numel(), _stream(stream, dev)))
    return ids, w, d, y, out


def layer_decode_noalloc(layer: ExpertLayer, x: torch.Tensor, logits: torch.Tensor, k: int, residual=None,
                         y_dtype=torch.float32, out_bf16: torch.Tensor | None = None, bufs=None, stream=None):
    """moe_layer_decode_noalloc: moe_layer_decode with the library's fixed device scratch as its workspace (no
    workspace argument; outputs from `bufs` or allocated here).  Returns (ids, w, dispatch, y, out)."""
    _need(x, "x")
    _need(logits, "logits")
    T, H = x.shape
    dev = x.device
    b = dict(bufs or {})
    b["dws"] = torch.empty(0, dtype=torch.uint8, device=dev)  # unused: the call takes no workspace
    ids, w, d, y, out, _ = _decode_buffers(layer, T, k, H, y_dtype, b, stream, dev)
    r_t = MOE_F32 if residual is None else _dtype_code(residual)
    _check(lib.moe_layer_decode_noalloc(ctypes.byref(layer.q), _ptr(logits), _ptr(x), _dtype_code(x), T, k,
                                        _ptr(residual), r_t, _ptr(ids), _ptr(w), _ptr(d.offsets),
                                        _ptr(d.sorted_assign), _ptr(d.assign_pos), _ptr(d.active), _ptr(d.n_active),
                                        _ptr(y), _dtype_code(y), _ptr(out), _ptr(out_bf16), _stream(stream, dev)))
    return ids, w, d, y, out


def noalloc_max_bytes() -> int:
    return int(lib.moe_layer_decode_noalloc_max_bytes())


def layer_decode_slots(table, l: int, layer: ExpertLayer, x: torch.Tensor, logits: torch.Tensor, k: int,
                       residual=None, y_dtype=torch.float32, out_bf16: torch.Tensor | None = None, bufs=None,
                       stream=None):
    """moe_layer_decode_slots: the layer step through `table` (device mode); `layer` is table.layer(l, ...)."""
    _need(x, "x")
    _need(logits, "logits")
    T, H = x.shape
    dev = x.device
    ids, w, d, y, out, ws = _decode_buffers(layer, T, k, H, y_dtype, bufs or {}, stream, dev)
    r_t = MOE_F32 if residual is None else _dtype_code(residual)
    _check(lib.moe_layer_decode_slots(ctypes.byref(layer.q), table.h, l, _ptr(logits), _ptr(x), _dtype_code(x), T, k,
                                      _ptr(residual), r_t, _ptr(ids), _ptr(w), _ptr(d.offsets), _ptr(d.sorted_assign),
                                      _ptr(d.assign_pos), _ptr(d.active), _ptr(d.n_active), _ptr(y), _dtype_code(y),
                                      _ptr(out), _ptr(out_bf16), _ptr(ws), ws.numel(), _stream(stream, dev)))
    return ids, w, d, y, out


def decode_workspace_bytes(layer: ExpertLayer, T: int, k: int) -> int:
    return int(lib.moe_layer_decode_workspace_bytes(ctypes.byref(layer.q), T, k))


# ---- slot table -------------------------------------------------------------------------

class SlotTable:
    """Resident-expert slot table over L*E page-locked host blobs (see moe.h)."""

    def __init__(self, L: int, E: int, n_slots: int, expert_bytes_: int, host_experts: torch.Tensor,
                 slots: torch.Tensor, slot_map: torch.Tensor, stream=None):
        self.L, self.E, self.n_slots, self.expert_bytes = L, E, n_slots, expert_bytes_
        self.host_experts, self.slots, self.slot_map = host_experts, slots, slot_map
        h = ctypes.c_void_p()
        _check(lib.moe_slot_table_create(L, E, n_slots, expert_bytes_, ctypes.c_void_p(host_experts.data_ptr()),
                                         _ptr(slots), _ptr(slot_map), _stream(stream, slots.device),
                                         ctypes.byref(h)))
        self.h = h

    def preload(self, pairs, stream=None):
        import numpy as np
        arr = np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1))
        _check(lib.moe_slot_table_preload(self.h, ctypes.c_void_p(arr.ctypes.data), arr.size // 2,
                                          _stream(stream, self.slots.device)))

    def resolve(self, layer: int, d: Dispatch, stream=None):
        _check(lib.moe_slot_table_resolve(self.h, layer, _ptr(d.active), _ptr(d.n_active),
                                          _stream(stream, self.slots.device)))

    def enable_device(self, stream=None):
        """Switch to device mode: the policy runs on the GPU (state in a device buffer this object keeps)."""
        nb = int(lib.moe_slot_table_device_bytes(self.L, self.E, self.n_slots))
        self.state = torch.empty(nb, dtype=torch.uint8, device=self.slots.device)
        _check(lib.moe_slot_table_enable_device(self.h, _ptr(self.state), nb, _stream(stream, self.slots.device)))

    def resolve_device(self, layer: int, d: Dispatch, max_active: int | None = None, stream=None):
        m = max_active if max_active is not None else min(self.E, d.T * d.k)
        _check(lib.moe_slot_table_resolve_device(self.h, layer, _ptr(d.active), _ptr(d.n_active), m,
                                                 _stream(stream, self.slots.device)))

    def layer(self, l: int, H: int, I: int, bits: int) -> ExpertLayer:
        return ExpertLayer(self.E, H, I, bits, self.slots, self.expert_bytes, self.slot_map[l * self.E:(l + 1) * self.E])

    def stats(self) -> dict:
        s = SlotStats()
        _check(lib.moe_slot_table_stats(self.h, ctypes.byref(s)))
        return {f: int(getattr(s, f)) for f, _ in SlotStats._fields_}

    def map_host(self):
        import numpy as np
        out = np.empty(self.L * self.E, np.int32)
        _check(lib.moe_slot_table_map_host(self.h, ctypes.c_void_p(out.ctypes.data)))
        return out

    def close(self):
        if self.h:
            lib.moe_slot_table_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class HostSlotTable:
    """Host-only slot table (no GPU): copies are reported to a Python callback."""

    def __init__(self, L: int, E: int, n_slots: int):
        self.copies = []

        def cb(user, slot, layer, expert):
            self.copies.append((slot, layer, expert))

        self._cb = COPY_FN(cb)
        h = ctypes.c_void_p()
        _check(lib.moe_slot_table_create_host(L, E, n_slots, self._cb, None, ctypes.byref(h)))
        self.h = h
        self.L, self.E = L, E

    def preload(self, pairs):
        import numpy as np
        arr = np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1))
        _check(lib.moe_slot_table_preload(self.h, ctypes.c_void_p(arr.ctypes.data), arr.size // 2, None))

    def resolve(self, layer: int, active):
        import numpy as np
        arr = np.ascontiguousarray(np.asarray(active, np.int32))
        _check(lib.moe_slot_table_resolve_host(self.h, layer, ctypes.c_void_p(arr.ctypes.data), arr.size))

    def stats(self) -> dict:
        s = SlotStats()
        _check(lib.moe_slot_table_stats(self.h, ctypes.byref(s)))
        return {f: int(getattr(s, f)) for f, _ in SlotStats._fields_}

    def map_host(self):
        import numpy as np
        out = np.empty(self.L * self.E, np.int32)
        _check(lib.moe_slot_table_map_host(self.h, ctypes.c_void_p(out.ctypes.data)))
        return out

    def close(self):
        if self.h:
            lib.moe_slot_table_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
