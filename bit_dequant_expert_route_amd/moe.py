"""ctypes binding of libmoe (include/moe.h).

Argument marshalling only: every step of the path runs in the HIP library.
Tensors are torch CUDA tensors (torch provides device memory and streams);
each call passes `tensor.data_ptr()` and the current stream's handle.  The
library must have been built (`python -m bit_dequant_expert_route_amd.build`);
importing this module without it raises, there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_LIB", os.path.join(HERE, "libmoe.so"))
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EALIGN, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16 = 0, 1
MOE_SHARED = -1
GROUP = 64


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: {detail} (status {status})")
        self.status = status


class LayerStruct(C.Structure):
    _fields_ = [
        ("hidden", C.c_int), ("inter", C.c_int), ("n_experts", C.c_int), ("top_k", C.c_int),
        ("group", C.c_int), ("bits_routed", C.c_int), ("bits_shared", C.c_int),
        ("renorm_topk", C.c_int),
        ("router_dtype", C.c_int), ("router", C.c_void_p),
        ("gate_dtype", C.c_int), ("shared_gate", C.c_void_p),
        ("experts", C.c_void_p), ("expert_stride", C.c_size_t),
        ("shared_expert", C.c_void_p), ("router_tiles", C.c_void_p),
    ]


class GdnLayerStruct(C.Structure):
    _fields_ = [("n_heads", C.c_int), ("d_head", C.c_int), ("bits", C.c_int),
                ("rec_qko", C.c_void_p), ("rec_vab", C.c_void_p), ("state", C.c_void_p)]


class WsView(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("sigma", C.c_void_p),
                ("h_routed", C.c_void_p), ("h_shared", C.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmoe is not built ({LIB_PATH} missing): run "
                          "python -m bit_dequant_expert_route_amd.build")
    lib = C.CDLL(LIB_PATH)
    P, I, Z, V = C.c_void_p, C.c_int, C.c_size_t, None
    sig = {
        "moe_strerror": (C.c_char_p, [I]),
        "moe_last_error": (C.c_char_p, []),
        "moe_abi_version": (I, []),
        "moe_qmatrix_bytes": (Z, [I, I, I, I]),
        "moe_expert_bytes": (Z, [I, I, I, I]),
        "moe_expert_offsets": (I, [I, I, I, I, C.POINTER(C.c_size_t)]),
        "moe_layer_workspace_bytes": (Z, [C.POINTER(LayerStruct), I]),
        "moe_stack_workspace_bytes": (Z, [C.POINTER(LayerStruct), I]),
        "moe_route": (I, [C.POINTER(LayerStruct), I, I, P, P, P, P, P, P, Z, P]),
        "moe_expert_forward_q4": (I, [C.POINTER(LayerStruct), I, P, P, I, P, P, P, Z, P]),
        "moe_expert_forward_q2": (I, [C.POINTER(LayerStruct), I, P, P, I, P, P, P, Z, P]),
        "moe_combine": (I, [I, I, P, P, P, P, P, P, P]),
        "moe_layer_decode": (I, [C.POINTER(LayerStruct), I, I, P, P, P, P, P, P, Z, P]),
        "moe_layer_decode_noalloc": (I, [C.POINTER(LayerStruct), I, I, P, P, P, P, P, P]),
        "moe_layer_ws_view": (I, [C.POINTER(LayerStruct), I, P, Z, C.POINTER(WsView)]),
        "moe_stack_decode": (I, [C.POINTER(LayerStruct), I, P, P, P, P, P, Z, P]),
        "moe_router_tile": (I, [P, I, I, I, P, P]),
        "moe_stack_gdn_workspace_bytes": (Z, [C.POINTER(LayerStruct), C.POINTER(GdnLayerStruct), I]),
        "moe_stack_decode_gdn": (I, [C.POINTER(LayerStruct), C.POINTER(GdnLayerStruct), I, P, P, P,
                                     P, P, Z, P]),
        "moe_graph_capture_begin": (I, [P]),
        "moe_graph_capture_end": (I, [P, C.POINTER(P)]),
        "moe_graph_create_stack": (I, [C.POINTER(LayerStruct), I, P, P, P, P, P, Z, P, C.POINTER(P)]),
        "moe_graph_launch": (I, [P, P]),
        "moe_graph_destroy": (I, [P]),
        "moe_fill_experts": (I, [P, Z, I, C.c_uint64, I, I, I, I, I, C.c_double, C.c_double,
                                 C.c_double, C.c_double, P]),
        "moe_zero": (I, [P, Z, P]),
        "moe_gdn_step": (I, [I, I, I, I, P, P, P, P, P, P, P, P]),
        "moe_tier_state_bytes": (Z, [I, I]),
        "moe_tier_create": (I, [P, I, Z, P, I, P, C.POINTER(P)]),
        "moe_tier_destroy": (I, [P]),
        "moe_tier_reset": (I, [P, P]),
        "moe_tier_layer_decode": (I, [C.POINTER(LayerStruct), P, I, P, P, P, P, P, P, Z, P]),
        "moe_tier_stats": (I, [P, P, C.POINTER(C.c_ulonglong), C.POINTER(C.c_ulonglong),
                               C.POINTER(C.c_ulonglong), P]),
        "moe_profile_begin": (I, [I]),
        "moe_profile_end": (I, [C.POINTER(C.c_float), C.POINTER(C.c_int), I, C.POINTER(C.c_int)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
lib = _lib


def header_functions() -> list[str]:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def _check(status: int, fn: str):
    if status != MOE_OK:
        raise MoeError(status, fn, _lib.moe_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------------------
# sizes
# ---------------------------------------------------------------------------
def expert_bytes(hidden: int, inter: int, bits: int) -> int:
    return int(_lib.moe_expert_bytes(hidden, inter, bits, GROUP))


def qmatrix_bytes(rows: int, cols: int, bits: int) -> int:
    return int(_lib.moe_qmatrix_bytes(rows, cols, bits, GROUP))


def expert_offsets(hidden: int, inter: int, bits: int) -> list[int]:
    out = (C.c_size_t * 6)()
    _check(_lib.moe_expert_offsets(hidden, inter, bits, GROUP, out), "moe_expert_offsets")
    return list(out)


# ---------------------------------------------------------------------------
# layer description
# ---------------------------------------------------------------------------
class Layer:
    """A MoE layer's shapes and weights (torch CUDA tensors it keeps alive)."""

    def __init__(self, *, hidden, inter, n_experts, top_k, bits_routed, bits_shared,
                 renorm, router, gate_vec, experts, expert_stride, shared_expert,
                 router_tiles=None):
        self.router, self.gate_vec = router, gate_vec
        self.experts, self.shared_expert = experts, shared_expert
        self.router_tiles = router_tiles
        self.s = LayerStruct(hidden, inter, n_experts, top_k, GROUP, bits_routed, bits_shared,
                             int(renorm), _dtype_code(router), _ptr(router),
                             _dtype_code(gate_vec), _ptr(gate_vec),
                             _ptr(experts), expert_stride, _ptr(shared_expert),
                             _ptr(router_tiles))

    def with_router_tiles(self, stream=None) -> "Layer":
        """This layer with its router's column tiles (moe_router_tile), which
        stacks read to form the routing sums."""
        if self.router_tiles is None:
            self.router_tiles = router_tile(self.router, self.s.n_experts, self.s.hidden, stream=stream)
            self.s.router_tiles = _ptr(self.router_tiles)
        return self

    def __getattr__(self, name):
        s = self.__dict__.get("s")
        if s is not None and name in dict(LayerStruct._fields_):
            return getattr(s, name)
        raise AttributeError(name)

    def workspace_bytes(self, n_tokens: int = 1) -> int:
        return int(_lib.moe_layer_workspace_bytes(C.byref(self.s), n_tokens))

    def workspace(self, n_tokens: int = 1) -> torch.Tensor:
        return torch.empty(self.workspace_bytes(n_tokens), dtype=torch.uint8, device="cuda")


def router_tile(router, n_experts=None, hidden=None, stream=None):
    """moe_router_tile: the [E][H] router as [H/8][E][8] column tiles."""
    E, H = (n_experts, hidden) if n_experts is not None else router.shape
    out = torch.empty(H // 8, E, 8, dtype=router.dtype, device=router.device)
    _check(_lib.moe_router_tile(_ptr(router), E, H, _dtype_code(router), _ptr(out), _stream(stream)),
           "moe_router_tile")
    return out


def _ws(layer: Layer, ws, n_tokens: int):
    if ws is None:
        ws = layer.workspace(n_tokens)
    return ws, _ptr(ws), ws.numel()


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def route(layer: Layer, x, topk_idx, topk_w, sigma, logits=None, ws=None, stream=None):
    T = x.shape[0] if x.dim() == 2 else 1
    ws, wp, wb = _ws(layer, ws, T)
    _check(_lib.moe_route(C.byref(layer.s), T, _dtype_code(x), _ptr(x), _ptr(topk_idx),
                          _ptr(topk_w), _ptr(sigma), _ptr(logits), wp, wb, _stream(stream)),
           "moe_route")


def expert_forward(layer: Layer, bits: int, x, ids, y, h=None, ws=None, stream=None):
    ws, wp, wb = _ws(layer, ws, 1)
    fn = _lib.moe_expert_forward_q4 if bits == 4 else _lib.moe_expert_forward_q2
    _check(fn(C.byref(layer.s), _dtype_code(x), _ptr(x), _ptr(ids), ids.numel(), _ptr(y),
              _ptr(h), wp, wb, _stream(stream)), f"moe_expert_forward_q{bits}")


def combine(h_res, y, w, y_shared, sigma, out, stream=None):
    _check(_lib.moe_combine(h_res.numel(), w.numel(), _ptr(h_res), _ptr(y), _ptr(w),
                            _ptr(y_shared), _ptr(sigma), _ptr(out), _stream(stream)),
           "moe_combine")


def layer_decode(layer: Layer, x, h_res, h_out, topk_idx, topk_w, ws=None, stream=None):
    T = x.shape[0] if x.dim() == 2 else 1
    ws, wp, wb = _ws(layer, ws, T)
    _check(_lib.moe_layer_decode(C.byref(layer.s), T, _dtype_code(x), _ptr(x), _ptr(h_res),
                                 _ptr(h_out), _ptr(topk_idx), _ptr(topk_w), wp, wb,
                                 _stream(stream)), "moe_layer_decode")


def layer_decode_noalloc(layer: Layer, x, h_res, h_out, topk_idx, topk_w, stream=None):
    """moe_layer_decode with the library's own scratch array as the workspace."""
    T = x.shape[0] if x.dim() == 2 else 1
    _check(_lib.moe_layer_decode_noalloc(C.byref(layer.s), T, _dtype_code(x), _ptr(x),
                                         _ptr(h_res), _ptr(h_out), _ptr(topk_idx),
                                         _ptr(topk_w), _stream(stream)),
           "moe_layer_decode_noalloc")


def ws_view(layer: Layer, n_tokens: int, ws) -> dict:
    """Views (fp32 tensors) of the intermediates moe_layer_decode leaves in ws."""
    v = WsView()
    _check(_lib.moe_layer_ws_view(C.byref(layer.s), n_tokens, _ptr(ws), ws.numel(), C.byref(v)),
           "moe_layer_ws_view")
    base = ws.data_ptr()
    E, K, I = layer.n_experts, layer.top_k, layer.inter
    f = ws.view(torch.uint8)

    def sl(ptr, n):
        o = ptr - base
        return f[o:o + 4 * n].view(torch.float32)
    return dict(logits=sl(v.logits, n_tokens * E).view(n_tokens, E),
                sigma=sl(v.sigma, n_tokens),
                h_routed=sl(v.h_routed, n_tokens * K * I).view(n_tokens, K, I),
                h_shared=sl(v.h_shared, n_tokens * I).view(n_tokens, I))


class Stack:
    """Layers of one resident expert stack (all shaped like layers[0]); with
    router_tiles (the default) each layer gets its router's column tiles."""

    def __init__(self, layers: list[Layer], router_tiles: bool = True):
        structs = []
        for l in layers:
            if router_tiles:
                l.with_router_tiles()
            st = LayerStruct.from_buffer_copy(l.s)
            if not router_tiles:
                st.router_tiles = None
            structs.append(st)
        self.layers = layers
        self.arr = (LayerStruct * len(layers))(*structs)

    def workspace(self) -> torch.Tensor:
        n = int(_lib.moe_stack_workspace_bytes(C.byref(self.arr[0]), len(self.layers)))
        return torch.empty(n, dtype=torch.uint8, device="cuda")


def stack_decode(stack: Stack, updates, h, idx_log, w_log, ws, stream=None):
    _check(_lib.moe_stack_decode(stack.arr, len(stack.layers), _ptr(updates), _ptr(h),
                                 _ptr(idx_log), _ptr(w_log), _ptr(ws), ws.numel(),
                                 _stream(stream)), "moe_stack_decode")


class GdnStack:
    """A stack whose layers may open with a linear-attention block: `gdn[l]`
    is None for a full-attention layer (its update is used) or a dict with
    n_heads, d_head, bits and the CUDA tensors rec_qko, rec_vab (projection
    records) and state ([n_heads][d_head][d_head] fp32, updated in place)."""

    def __init__(self, layers: list[Layer], gdn: list):
        self.layers, self.gdn = layers, gdn
        self.arr = (LayerStruct * len(layers))(*[l.s for l in layers])
        structs = []
        for g in gdn:
            if g is None:
                structs.append(GdnLayerStruct(0, 0, 0, None, None, None))
            else:
                structs.append(GdnLayerStruct(g["n_heads"], g["d_head"], g["bits"], _ptr(g["rec_qko"]),
                                              _ptr(g["rec_vab"]), _ptr(g["state"])))
        self.garr = (GdnLayerStruct * len(layers))(*structs)

    def workspace(self) -> torch.Tensor:
        n = int(_lib.moe_stack_gdn_workspace_bytes(C.byref(self.arr[0]), self.garr, len(self.layers)))
        return torch.empty(n, dtype=torch.uint8, device="cuda")


def stack_decode_gdn(stack: GdnStack, updates, h, idx_log, w_log, ws, stream=None):
    _check(_lib.moe_stack_decode_gdn(stack.arr, stack.garr, len(stack.layers), _ptr(updates), _ptr(h),
                                     _ptr(idx_log), _ptr(w_log), _ptr(ws), ws.numel(),
                                     _stream(stream)), "moe_stack_decode_gdn")


class Graph:
    """An instantiated HIP graph (moe_graph_t)."""

    def __init__(self, handle, keep=()):
        self.h = handle
        self.keep = keep  # tensors the graph's pointers refer to

    def launch(self, stream=None):
        _check(_lib.moe_graph_launch(self.h, _stream(stream)), "moe_graph_launch")

    def destroy(self):
        if self.h:
            _check(_lib.moe_graph_destroy(self.h), "moe_graph_destroy")
            self.h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


def capture_begin(stream):
    _check(_lib.moe_graph_capture_begin(stream.cuda_stream), "moe_graph_capture_begin")


def capture_end(stream, keep=()) -> Graph:
    h = C.c_void_p()
    _check(_lib.moe_graph_capture_end(stream.cuda_stream, C.byref(h)), "moe_graph_capture_end")
    return Graph(h, keep)


def graph_stack(stack: Stack, updates, h, idx_log, w_log, ws, stream) -> Graph:
    g = C.c_void_p()
    _check(_lib.moe_graph_create_stack(stack.arr, len(stack.layers), _ptr(updates), _ptr(h),
                                       _ptr(idx_log), _ptr(w_log), _ptr(ws), ws.numel(),
                                       stream.cuda_stream, C.byref(g)), "moe_graph_create_stack")
    return Graph(g, (stack, updates, h, idx_log, w_log, ws))


def fill_experts(dst, stride: int, n: int, seed: int, layer: int, first_expert: int,
                 hidden: int, inter: int, bits: int, dist, stream=None, offset: int = 0):
    _check(_lib.moe_fill_experts(_ptr(dst) + offset, stride, n, seed, layer, first_expert,
                                 hidden, inter, bits, dist.scale_lo, dist.scale_hi,
                                 dist.bias_lo, dist.bias_hi, _stream(stream)),
           "moe_fill_experts")


KERNEL_NAMES = {1: "head", 2: "gateup", 3: "down_combine", 4: "down_y", 5: "topk",
                6: "combine", 7: "other", 8: "gdn_in", 9: "gdn_step", 10: "gdn_out"}


def profile_begin(max_launches: int):
    _check(_lib.moe_profile_begin(max_launches), "moe_profile_begin")


def profile_end(capacity: int):
    """[(kernel name, ms), ...] of the launches recorded since profile_begin."""
    ms = (C.c_float * capacity)()
    ids = (C.c_int * capacity)()
    n = C.c_int(0)
    _check(_lib.moe_profile_end(ms, ids, capacity, C.byref(n)), "moe_profile_end")
    return [(KERNEL_NAMES.get(ids[i], str(ids[i])), float(ms[i])) for i in range(n.value)]


def gdn_step(q, k, v, alpha, beta, state, out, stream=None):
    """One gated delta-rule decode step (moe_gdn_step): state
    [n_seq][n_heads][d_v][d_k] is updated in place, out [n_seq][n_heads][d_v]
    receives S q.  fp32 device tensors."""
    n_seq, n_heads, d_v, d_k = state.shape
    _check(_lib.moe_gdn_step(n_seq, n_heads, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                             _ptr(beta), _ptr(state), _ptr(out), _stream(stream)), "moe_gdn_step")


def zero(t, stream=None):
    _check(_lib.moe_zero(_ptr(t), t.numel() * t.element_size(), _stream(stream)), "moe_zero")


class Tier:
    """Host-memory expert tier (moe_tier_*): `host` holds the layer's E routed
    records (a page-locked CPU uint8 tensor), `cache` is a CUDA uint8 tensor of
    n_slots * stride bytes, and the tier's device state is allocated here (a
    CUDA tensor) and reset.  host and cache must outlive the tier."""

    def __init__(self, host, n_experts: int, stride: int, cache, n_slots: int,
                 host_ptr: int | None = None, cache_ptr: int | None = None,
                 state_ptr: int | None = None, reset: bool = True):
        self.host, self.cache, self.n_slots = host, cache, n_slots
        nb = int(_lib.moe_tier_state_bytes(n_experts, n_slots))
        self.state = None
        if state_ptr is None:
            self.state = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
            state_ptr = self.state.data_ptr()
        hp = host_ptr if host_ptr is not None else host.data_ptr()
        cp = cache_ptr if cache_ptr is not None else _ptr(cache)
        h = C.c_void_p()
        _check(_lib.moe_tier_create(hp, n_experts, stride, cp, n_slots, state_ptr, C.byref(h)),
               "moe_tier_create")
        self.h = h
        if reset:
            self.reset()

    def reset(self, stream=None):
        _check(_lib.moe_tier_reset(self.h, _stream(stream)), "moe_tier_reset")

    def stats(self, stream=None):
        """(hits, misses, record bytes read from host memory) since the reset."""
        h, m, b = C.c_ulonglong(), C.c_ulonglong(), C.c_ulonglong()
        _check(_lib.moe_tier_stats(self.h, _stream(stream), C.byref(h), C.byref(m), C.byref(b), None),
               "moe_tier_stats")
        return int(h.value), int(m.value), int(b.value)

    def slots(self, stream=None):
        """The expert in each slot (-1: empty)."""
        own = (C.c_int32 * self.n_slots)()
        _check(_lib.moe_tier_stats(self.h, _stream(stream), None, None, None, own), "moe_tier_stats")
        return list(own)

    def layer_decode(self, layer: "Layer", x, h_res, h_out, topk_idx, topk_w, ws=None, stream=None):
        ws, wp, wb = _ws(layer, ws, 1)
        _check(_lib.moe_tier_layer_decode(C.byref(layer.s), self.h, _dtype_code(x), _ptr(x), _ptr(h_res),
                                          _ptr(h_out), _ptr(topk_idx), _ptr(topk_w), wp, wb,
                                          _stream(stream)), "moe_tier_layer_decode")

    def close(self):
        if self.h:
            _check(_lib.moe_tier_destroy(self.h), "moe_tier_destroy")
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
