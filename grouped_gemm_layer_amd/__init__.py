"""Python binding of the MoE expert-layer HIP library (libmoe_gfx950.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  The
binding raises if the built library is missing; there is no fallback.

Names follow the C ABI in include/moe.h:
    workspace_size(dims) -> (route_ws, saved, fwd_ws, bwd_ws)
    route(dims, logits, routing, ws)
    route_noalloc(dims, logits, routing)
    weight_codes_size(dims); quantize_weights(dims, w13, w2, codes)
    forward_cached(dims, x, w13, w2, codes, routing, y, saved, ws)
    backward_cached(dims, dy, x, codes, routing, saved, dx, dw13, dw2, dgate, dlogits, ws)
    forward(dims, x, w13, w2, routing, y, saved, ws)
    backward(dims, dy, x, w13, w2, routing, saved, dx, dw13, dw2, dgate, dlogits, ws)
    mxfp8_quantize(src, along, codes, scales)
    mxfp8_quantize_grouped(src, offsets, capacity, pad_off, codes, scales)
plus allocation helpers (alloc_routing, alloc_workspace) and MoeLayer, a
small holder that owns the buffers of one shape.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MODE_FP32", "MODE_BF16", "MODE_MXFP8", "MODE_FP8_BWD", "Dims", "RoutingBuffers",
    "MoeError", "lib_path", "load_library", "workspace_size", "route", "forward", "backward",
    "alloc_routing", "alloc_workspace", "status_str", "MoeLayer", "num_kernels", "mxfp8_quantize",
    "mxfp8_quantize_grouped", "mxfp8_grouped_capacity", "route_noalloc", "weight_codes_size", "quantize_weights",
    "forward_cached", "backward_cached",
]

MODE_FP32, MODE_BF16, MODE_MXFP8, MODE_FP8_BWD = 0, 1, 2, 3
MODE_BY_NAME = {"fp32": MODE_FP32, "bf16": MODE_BF16, "mxfp8": MODE_MXFP8, "fp8_bwd": MODE_FP8_BWD}

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmoe_gfx950.so"

SYMBOLS = ("moe_workspace_size", "moe_route", "moe_forward", "moe_backward", "moe_status_str")


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("mode", ctypes.c_int32)]

    @classmethod
    def of(cls, T, H, I, E, k, mode):
        if isinstance(mode, str):
            mode = MODE_BY_NAME[mode]
        return cls(T, H, I, E, k, mode)


class _CRouting(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("sorted_to_flat", ctypes.c_void_p),
                ("flat_to_sorted", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


_lib = None


def lib_path() -> str:
    return os.path.join(_PKG, LIB_NAME)


def load_library():
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch's HIP runtime (same soname) must be the one in the process, so that
    # torch streams and device pointers are valid in the library's calls
    import torch  # noqa: F401
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with python -m grouped_gemm_layer_amd.build_lib")
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.moe_workspace_size.argtypes = [ctypes.POINTER(Dims)] + [ctypes.POINTER(sz)] * 4
    lib.moe_route.argtypes = [ctypes.POINTER(Dims), vp, ctypes.POINTER(_CRouting), vp, sz, vp]
    lib.moe_forward.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, ctypes.POINTER(_CRouting), vp, vp, vp, sz, vp]
    lib.moe_backward.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, ctypes.POINTER(_CRouting), vp, vp,
                                 vp, vp, vp, vp, vp, sz, vp]
    for f in ("moe_workspace_size", "moe_route", "moe_forward", "moe_backward"):
        getattr(lib, f).restype = ctypes.c_int
    lib.moe_weight_codes_size.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(sz)]
    lib.moe_weight_codes_size.restype = ctypes.c_int
    lib.moe_quantize_weights.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, sz, vp]
    lib.moe_quantize_weights.restype = ctypes.c_int
    lib.moe_forward_cached.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, ctypes.POINTER(_CRouting), vp, vp, vp,
                                       sz, vp]
    lib.moe_forward_cached.restype = ctypes.c_int
    lib.moe_backward_cached.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, ctypes.POINTER(_CRouting), vp, vp, vp, vp,
                                        vp, vp, vp, sz, vp]
    lib.moe_backward_cached.restype = ctypes.c_int
    lib.moe_route_noalloc.argtypes = [ctypes.POINTER(Dims), vp, ctypes.POINTER(_CRouting), vp]
    lib.moe_route_noalloc.restype = ctypes.c_int
    lib.moe_route_project.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, ctypes.POINTER(_CRouting), vp, sz, vp]
    lib.moe_route_project.restype = ctypes.c_int
    lib.moe_router_backward.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(_CRouting), vp, vp, vp, vp, vp, vp]
    lib.moe_router_backward.restype = ctypes.c_int
    lib.moe_backward_accumulate.argtypes = lib.moe_backward.argtypes
    lib.moe_backward_accumulate.restype = ctypes.c_int
    lib.moe_forward_recompute.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, ctypes.POINTER(_CRouting), vp, vp, sz,
                                          vp]
    lib.moe_forward_recompute.restype = ctypes.c_int
    lib.moe_forward_timed.argtypes = lib.moe_forward.argtypes + [vp, ctypes.c_int]
    lib.moe_backward_timed.argtypes = lib.moe_backward.argtypes + [vp, ctypes.c_int]
    lib.moe_forward_timed.restype = ctypes.c_int
    lib.moe_backward_timed.restype = ctypes.c_int
    lib.moe_num_kernels.argtypes = [ctypes.POINTER(Dims), ctypes.c_int]
    lib.moe_num_kernels.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.moe_mxfp8_quantize.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.moe_mxfp8_quantize.restype = ctypes.c_int
    lib.moe_mxfp8_quantize_grouped.argtypes = [vp, i32, i32, vp, i32, i32, vp, vp, vp, vp]
    lib.moe_mxfp8_quantize_grouped.restype = ctypes.c_int
    lib.moe_mxfp8_grouped_capacity.argtypes = [i32, i32]
    lib.moe_mxfp8_grouped_capacity.restype = sz
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_wgrad_chunk_rows.argtypes = []
    lib.moe_wgrad_chunk_rows.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


def wgrad_chunk_rows() -> int:
    """Rows per weight-gradient chunk (experts with more rows are split)."""
    return int(load_library().moe_wgrad_chunk_rows())


def _check(st: int, what: str):
    if st != 0:
        raise MoeError(st, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_size(dims: Dims):
    lib = load_library()
    out = [ctypes.c_size_t(0) for _ in range(4)]
    _check(lib.moe_workspace_size(ctypes.byref(dims), *[ctypes.byref(o) for o in out]), "moe_workspace_size")
    return tuple(o.value for o in out)


class RoutingBuffers:
    """Device tensors of the routing state (torch int32/float32)."""

    def __init__(self, topk_idx, gate, counts, offsets, sorted_to_flat, flat_to_sorted):
        self.topk_idx, self.gate, self.counts = topk_idx, gate, counts
        self.offsets, self.sorted_to_flat, self.flat_to_sorted = offsets, sorted_to_flat, flat_to_sorted

    def c(self) -> _CRouting:
        return _CRouting(self.topk_idx.data_ptr(), self.gate.data_ptr(), self.counts.data_ptr(),
                         self.offsets.data_ptr(), self.sorted_to_flat.data_ptr(), self.flat_to_sorted.data_ptr())


def alloc_routing(dims: Dims, device="cuda") -> RoutingBuffers:
    import torch
    T, k, E = dims.T, dims.k, dims.E
    i32 = dict(dtype=torch.int32, device=device)
    return RoutingBuffers(torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=device),
                          torch.empty((E,), **i32), torch.empty((E + 1,), **i32),
                          torch.empty((T * k,), **i32), torch.empty((T * k,), **i32))


def alloc_workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty((max(int(nbytes), 1),), dtype=torch.uint8, device=device)


def route(dims: Dims, logits, routing: RoutingBuffers, ws, stream=None):
    lib = load_library()
    r = routing.c()
    _check(lib.moe_route(ctypes.byref(dims), _ptr(logits), ctypes.byref(r), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_route")


def route_noalloc(dims: Dims, logits, routing: RoutingBuffers, stream=None):
    """moe_route_noalloc: routing without a workspace (the library's static
    per-device scratch; calls that overlap on one GPU race)."""
    lib = load_library()
    r = routing.c()
    _check(lib.moe_route_noalloc(ctypes.byref(dims), _ptr(logits), ctypes.byref(r), _stream(stream)),
           "moe_route_noalloc")


def route_project(dims: Dims, x, w_router, logits, routing: RoutingBuffers, ws, stream=None):
    """logits = x w_router^T (written to `logits`), then route (moe_route_project)."""
    lib = load_library()
    r = routing.c()
    _check(lib.moe_route_project(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(logits), ctypes.byref(r),
                                 _ptr(ws), ws.numel(), _stream(stream)), "moe_route_project")


def router_backward(dims: Dims, routing: RoutingBuffers, dlogits, x, w_router, dx, dw_router, stream=None):
    """dx += dlogits w_router; dw_router = dlogits^T x (moe_router_backward)."""
    lib = load_library()
    r = routing.c()
    _check(lib.moe_router_backward(ctypes.byref(dims), ctypes.byref(r), _ptr(dlogits), _ptr(x), _ptr(w_router),
                                   _ptr(dx), _ptr(dw_router), _stream(stream)), "moe_router_backward")


def forward(dims: Dims, x, w13, w2, routing: RoutingBuffers, y, saved, ws, stream=None, events=None):
    """events: optional ctypes array of hipEvent_t (moe_forward_timed)."""
    lib = load_library()
    r = routing.c()
    args = [ctypes.byref(dims), _ptr(x), _ptr(w13), _ptr(w2), ctypes.byref(r), _ptr(y), _ptr(saved), _ptr(ws),
            ws.numel(), _stream(stream)]
    if events is None:
        _check(lib.moe_forward(*args), "moe_forward")
    else:
        _check(lib.moe_forward_timed(*args, events, len(events)), "moe_forward_timed")


def forward_recompute(dims: Dims, x, w13, w2, routing: RoutingBuffers, saved, ws, stream=None):
    """moe_forward_recompute: restore `saved` for the backward without computing y."""
    lib = load_library()
    r = routing.c()
    _check(lib.moe_forward_recompute(ctypes.byref(dims), _ptr(x), _ptr(w13), _ptr(w2), ctypes.byref(r),
                                     _ptr(saved), _ptr(ws), ws.numel(), _stream(stream)), "moe_forward_recompute")


def backward(dims: Dims, dy, x, w13, w2, routing: RoutingBuffers, saved, dx, dw13, dw2, dgate, dlogits, ws,
             stream=None, events=None, accumulate=False):
    """events: optional ctypes array of hipEvent_t (moe_backward_timed).
    accumulate: add the weight gradients to dw13 / dw2 (moe_backward_accumulate)."""
    lib = load_library()
    r = routing.c()
    args = [ctypes.byref(dims), _ptr(dy), _ptr(x), _ptr(w13), _ptr(w2), ctypes.byref(r), _ptr(saved), _ptr(dx),
            _ptr(dw13), _ptr(dw2), _ptr(dgate), _ptr(dlogits), _ptr(ws), ws.numel(), _stream(stream)]
    if accumulate:
        if events is not None:
            raise ValueError("timed accumulate-into is not provided")
        _check(lib.moe_backward_accumulate(*args), "moe_backward_accumulate")
    elif events is None:
        _check(lib.moe_backward(*args), "moe_backward")
    else:
        _check(lib.moe_backward_timed(*args, events, len(events)), "moe_backward_timed")


def weight_codes_size(dims: Dims) -> int:
    """Bytes of the MXFP8 weight copies of an fp8 mode (moe_weight_codes_size)."""
    out = ctypes.c_size_t(0)
    _check(load_library().moe_weight_codes_size(ctypes.byref(dims), ctypes.byref(out)), "moe_weight_codes_size")
    return out.value


def quantize_weights(dims: Dims, w13, w2, codes, stream=None):
    """MXFP8 copies of the weights into `codes` (uint8 tensor, moe_quantize_weights)."""
    _check(load_library().moe_quantize_weights(ctypes.byref(dims), _ptr(w13), _ptr(w2), _ptr(codes), codes.numel(),
                                               _stream(stream)), "moe_quantize_weights")


def forward_cached(dims: Dims, x, w13, w2, codes, routing: RoutingBuffers, y, saved, ws, stream=None):
    """moe_forward_cached: the MXFP8 GEMMs take their weights from `codes`."""
    r = routing.c()
    _check(load_library().moe_forward_cached(ctypes.byref(dims), _ptr(x), _ptr(w13), _ptr(w2), _ptr(codes),
                                             ctypes.byref(r), _ptr(y), _ptr(saved), _ptr(ws), ws.numel(),
                                             _stream(stream)), "moe_forward_cached")


def backward_cached(dims: Dims, dy, x, codes, routing: RoutingBuffers, saved, dx, dw13, dw2, dgate, dlogits, ws,
                    stream=None):
    """moe_backward_cached: the MXFP8 GEMMs take their weights from `codes`."""
    r = routing.c()
    _check(load_library().moe_backward_cached(ctypes.byref(dims), _ptr(dy), _ptr(x), _ptr(codes), ctypes.byref(r),
                                              _ptr(saved), _ptr(dx), _ptr(dw13), _ptr(dw2), _ptr(dgate),
                                              _ptr(dlogits), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_backward_cached")


def num_kernels(dims: Dims, which: str) -> int:
    n = load_library().moe_num_kernels(ctypes.byref(dims), {"route": 0, "forward": 1, "backward": 2}[which])
    if n < 0:
        raise MoeError(2, "moe_num_kernels")
    return n


def mxfp8_quantize(src, along: int, codes, scales, stream=None):
    """src: bf16 [rows, cols]; along=1 -> codes [rows, cols], scales [rows, cols/32];
    along=0 -> codes [cols, rows], scales [cols, rows/32] (uint8 tensors)."""
    rows, cols = src.shape
    _check(load_library().moe_mxfp8_quantize(_ptr(src), rows, cols, along, _ptr(codes), _ptr(scales),
                                             _stream(stream)), "moe_mxfp8_quantize")


def mxfp8_grouped_capacity(rows: int, E: int) -> int:
    return int(load_library().moe_mxfp8_grouped_capacity(rows, E))


def mxfp8_quantize_grouped(src, offsets, capacity: int, pad_off, codes, scales, stream=None):
    """src: bf16 [rows, cols] in expert order (offsets int32 [E+1]); codes
    [cols, capacity], scales [cols, capacity/32] (uint8), pad_off int32 [E+1]."""
    rows, cols = src.shape
    E = offsets.numel() - 1
    _check(load_library().moe_mxfp8_quantize_grouped(_ptr(src), rows, cols, _ptr(offsets), E, capacity,
                                                     _ptr(pad_off), _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_mxfp8_quantize_grouped")


class MoeLayer:
    """Owns the routing state, saved buffer, outputs and workspaces of one shape.

    Weights and activations are passed per call; all buffers are torch device
    tensors allocated once here (never inside route/forward/backward)."""

    def __init__(self, T, H, I, E, k, mode="bf16", device="cuda"):
        import torch
        self.dims = Dims.of(T, H, I, E, k, mode)
        self.device = device
        self.act_dtype = torch.float32 if self.dims.mode == MODE_FP32 else torch.bfloat16
        rws, saved, fws, bws = workspace_size(self.dims)
        self.routing = alloc_routing(self.dims, device)
        self.route_ws = alloc_workspace(rws, device)
        self.saved = alloc_workspace(saved, device)
        self.fwd_ws = alloc_workspace(fws, device)
        self.bwd_ws = alloc_workspace(bws, device)
        self.y = torch.empty((T, H), dtype=self.act_dtype, device=device)
        self.dx = torch.empty((T, H), dtype=self.act_dtype, device=device)
        self.dw13 = torch.empty((E, 2 * I, H), dtype=torch.float32, device=device)
        self.dw2 = torch.empty((E, H, I), dtype=torch.float32, device=device)
        self.dgate = torch.empty((T, k), dtype=torch.float32, device=device)
        self.dlogits = torch.empty((T, E), dtype=torch.float32, device=device)

    def route(self, logits, stream=None):
        route(self.dims, logits, self.routing, self.route_ws, stream)

    def route_project(self, x, w_router, stream=None):
        """Router projection logits = x w_router^T (kept in self.logits), then route."""
        import torch
        if getattr(self, "logits", None) is None:
            self.logits = torch.empty((self.dims.T, self.dims.E), dtype=torch.float32, device=self.device)
        route_project(self.dims, x, w_router, self.logits, self.routing, self.route_ws, stream)
        return self.logits

    def router_backward(self, x, w_router, dw_router, stream=None):
        """After backward(want_dlogits=True): dx += dlogits w_router, dw_router = dlogits^T x."""
        router_backward(self.dims, self.routing, self.dlogits, x, w_router, self.dx, dw_router, stream)

    def forward(self, x, w13, w2, stream=None, events=None, keep_saved=True):
        """keep_saved=False: keep no state for a backward (checkpointing's first forward)."""
        forward(self.dims, x, w13, w2, self.routing, self.y, self.saved if keep_saved else None, self.fwd_ws,
                stream, events)
        return self.y

    def forward_recompute(self, x, w13, w2, stream=None):
        """Second forward of activation checkpointing: `saved` as forward() writes it, y untouched."""
        forward_recompute(self.dims, x, w13, w2, self.routing, self.saved, self.fwd_ws, stream)

    def quantize_weights(self, w13, w2, stream=None):
        """MXFP8 copies of the weights (fp8 modes), kept in self.wcodes for the cached calls."""
        if getattr(self, "wcodes", None) is None:
            self.wcodes = alloc_workspace(weight_codes_size(self.dims), self.device)
        quantize_weights(self.dims, w13, w2, self.wcodes, stream)
        return self.wcodes

    def forward_cached(self, x, w13, w2, stream=None):
        forward_cached(self.dims, x, w13, w2, self.wcodes, self.routing, self.y, self.saved, self.fwd_ws, stream)
        return self.y

    def backward_cached(self, dy, x, want_dlogits=True, stream=None):
        backward_cached(self.dims, dy, x, self.wcodes, self.routing, self.saved, self.dx, self.dw13, self.dw2,
                        self.dgate, self.dlogits if want_dlogits else None, self.bwd_ws, stream)
        return self.dx, self.dw13, self.dw2, self.dgate, (self.dlogits if want_dlogits else None)

    def backward(self, dy, x, w13, w2, want_dlogits=True, stream=None, events=None, accumulate=False):
        backward(self.dims, dy, x, w13, w2, self.routing, self.saved, self.dx, self.dw13, self.dw2, self.dgate,
                 self.dlogits if want_dlogits else None, self.bwd_ws, stream, events, accumulate)
        return self.dx, self.dw13, self.dw2, self.dgate, (self.dlogits if want_dlogits else None)
