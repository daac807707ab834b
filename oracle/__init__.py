"""fp64 CPU oracle of the MoE expert forward -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
binding) never does.

`Oracle` wraps the plain C implementation in `moe_oracle.c` (fp64, fixed
sequential summation order); `oracle.dense` is an independent NumPy brute force
for tiny shapes that materialises every weight matrix.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_dp = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_ip = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")

DTYPE_CODE = {"f32": 0, "bf16": 1}


def _raw(a: np.ndarray, dtype: str) -> np.ndarray:
    want = np.float32 if dtype == "f32" else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"expected {want} array for dtype {dtype}, got {a.dtype}")
    return a


class Oracle:
    def __init__(self, path: str | None = None):
        if path is None:
            path = _build.ensure_built()
        self.path = path
        L = C.CDLL(path)
        self._L = L
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [C.c_int]
        L.oracle_max_threads.restype = C.c_int
        L.oracle_max_threads.argtypes = []
        L.oracle_record_bytes.restype = C.c_size_t
        L.oracle_record_bytes.argtypes = [C.c_int, C.c_int, C.c_int]
        L.oracle_qmatvec.restype = None
        L.oracle_qmatvec.argtypes = [_u32p, _u32p, C.c_int, C.c_int, C.c_int, _dp, _dp]
        L.oracle_dequant_matrix.restype = None
        L.oracle_dequant_matrix.argtypes = [_u32p, _u32p, C.c_int, C.c_int, C.c_int, _dp]
        L.oracle_router.restype = None
        L.oracle_router.argtypes = [C.c_int, C.c_void_p, C.c_int, C.c_int, _dp, _dp]
        L.oracle_softmax.restype = None
        L.oracle_softmax.argtypes = [_dp, C.c_int, _dp]
        L.oracle_topk.restype = None
        L.oracle_topk.argtypes = [_dp, C.c_int, C.c_int, _ip]
        L.oracle_topk_weights.restype = None
        L.oracle_topk_weights.argtypes = [_dp, _ip, C.c_int, C.c_int, _dp]
        L.oracle_shared_gate.restype = C.c_double
        L.oracle_shared_gate.argtypes = [C.c_int, C.c_void_p, C.c_int, _dp]
        L.oracle_expert.restype = None
        L.oracle_expert.argtypes = [_u8p, C.c_int, C.c_int, C.c_int, _dp, _dp, _dp]
        L.oracle_combine.restype = None
        L.oracle_combine.argtypes = [C.c_int, C.c_int, _dp, _dp, _dp, _dp, C.c_double, _dp]
        L.oracle_rmsnorm.restype = None
        L.oracle_rmsnorm.argtypes = [_dp, C.c_int, C.c_double, _dp]
        L.oracle_bf16_to_f64.restype = C.c_double
        L.oracle_bf16_to_f64.argtypes = [C.c_uint16]
        L.oracle_gdn_step.restype = None
        L.oracle_gdn_step.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, _dp, _dp, _dp, _dp,
                                      _dp, _dp, _dp]
        L.oracle_gdn_block.restype = None
        L.oracle_gdn_block.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, _u8p, _u8p, _dp, _dp,
                                       _dp, _dp, _dp]
        L.oracle_layer.restype = None
        L.oracle_layer.argtypes = [
            C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
            C.c_int, C.c_void_p, C.c_int, C.c_void_p,
            _u8p, C.c_size_t, _u8p, _dp, _dp,
            _dp, _dp, _ip, _dp, C.POINTER(C.c_double), _dp, _dp, _dp]

    # -- format ---------------------------------------------------------
    def record_bytes(self, hidden: int, inter: int, bits: int) -> int:
        return int(self._L.oracle_record_bytes(hidden, inter, bits))

    # -- building blocks ------------------------------------------------
    def qmatvec(self, codes, sb, rows, cols, bits, x):
        codes = np.ascontiguousarray(codes, dtype=np.uint32)
        sb = np.ascontiguousarray(sb, dtype=np.uint32)
        x = np.ascontiguousarray(x, dtype=np.float64)
        assert codes.size == rows * cols * bits // 32 and sb.size == rows * cols // 64
        assert x.size == cols
        y = np.empty(rows, dtype=np.float64)
        self._L.oracle_qmatvec(codes, sb, rows, cols, bits, x, y)
        return y

    def dequant_matrix(self, codes, sb, rows, cols, bits):
        w = np.empty((rows, cols), dtype=np.float64)
        self._L.oracle_dequant_matrix(np.ascontiguousarray(codes, dtype=np.uint32),
                                      np.ascontiguousarray(sb, dtype=np.uint32),
                                      rows, cols, bits, w)
        return w

    def router(self, w, dtype: str, x):
        w = _raw(w, dtype)
        E, H = w.shape
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(E, dtype=np.float64)
        self._L.oracle_router(DTYPE_CODE[dtype], w.ctypes.data, E, H, x, out)
        return out

    def softmax(self, logits):
        logits = np.ascontiguousarray(logits, dtype=np.float64)
        p = np.empty_like(logits)
        self._L.oracle_softmax(logits, logits.size, p)
        return p

    def topk(self, logits, k: int):
        logits = np.ascontiguousarray(logits, dtype=np.float64)
        idx = np.empty(k, dtype=np.int32)
        self._L.oracle_topk(logits, logits.size, k, idx)
        return idx

    def topk_weights(self, p, idx, renorm: bool):
        p = np.ascontiguousarray(p, dtype=np.float64)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        w = np.empty(idx.size, dtype=np.float64)
        self._L.oracle_topk_weights(p, idx, idx.size, int(renorm), w)
        return w

    def shared_gate(self, g, dtype: str, x) -> float:
        g = _raw(g, dtype)
        x = np.ascontiguousarray(x, dtype=np.float64)
        return float(self._L.oracle_shared_gate(DTYPE_CODE[dtype], g.ctypes.data, g.size, x))

    def expert(self, record, hidden, inter, bits, x):
        record = np.ascontiguousarray(record, dtype=np.uint8)
        assert record.size >= self.record_bytes(hidden, inter, bits)
        x = np.ascontiguousarray(x, dtype=np.float64)
        h = np.empty(inter, dtype=np.float64)
        y = np.empty(hidden, dtype=np.float64)
        self._L.oracle_expert(record, hidden, inter, bits, x, h, y)
        return h, y

    def combine(self, h_res, y, w, y_shared, sigma):
        h_res = np.ascontiguousarray(h_res, dtype=np.float64)
        y = np.ascontiguousarray(y, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float64)
        y_shared = np.ascontiguousarray(y_shared, dtype=np.float64)
        out = np.empty_like(h_res)
        self._L.oracle_combine(h_res.size, w.size, h_res, y, w, y_shared, float(sigma), out)
        return out

    def set_threads(self, n: int) -> None:
        """Threads of the row loops; results are the same for any count."""
        self._L.oracle_set_threads(int(n))

    def max_threads(self) -> int:
        return int(self._L.oracle_max_threads())

    def rmsnorm(self, h, eps: float = 1e-6):
        h = np.ascontiguousarray(h, dtype=np.float64)
        x = np.empty_like(h)
        self._L.oracle_rmsnorm(h, h.size, eps, x)
        return x

    def bf16_to_f64(self, bits: int) -> float:
        return float(self._L.oracle_bf16_to_f64(bits))

    def gdn_step(self, q, k, v, alpha, beta, state):
        """One gated delta-rule decode step for [n_seq][n_heads] heads:
        S <- alpha S; u = S k; S <- S + beta (v - u) k^T; o = S q.  Returns
        (new state, o); the inputs are not modified."""
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        S = np.array(state, dtype=np.float64, copy=True, order="C")
        n_seq, n_heads, d_v, d_k = S.shape
        assert q.shape == k.shape == (n_seq, n_heads, d_k) and v.shape == (n_seq, n_heads, d_v)
        a = np.ascontiguousarray(alpha, dtype=np.float64).reshape(n_seq, n_heads)
        b = np.ascontiguousarray(beta, dtype=np.float64).reshape(n_seq, n_heads)
        o = np.empty((n_seq, n_heads, d_v))
        self._L.oracle_gdn_step(n_seq, n_heads, d_k, d_v, q, k, v, a, b, S, o)
        return S, o

    def gdn_block(self, rec_qko, rec_vab, hidden, n_heads, d_head, bits, h, state):
        """One linear-attention block for one token: x = RMSNorm(h), the
        quantised q/k/v/alpha/beta projections, unit-length q and k per head,
        sigmoid gates, the gated delta-rule step, and h + W_o o.  Returns dict
        (proj [3D + 2 n_heads], o [D], h_out [H], state [n_heads][d][d]); the
        inputs are not modified."""
        D = n_heads * d_head
        rq = np.ascontiguousarray(rec_qko, dtype=np.uint8).reshape(-1)
        rv = np.ascontiguousarray(rec_vab, dtype=np.uint8).reshape(-1)
        need = self.record_bytes(hidden, D, bits)
        assert rq.size >= need and rv.size >= need
        h = np.ascontiguousarray(h, dtype=np.float64)
        S = np.array(state, dtype=np.float64, copy=True, order="C").reshape(n_heads, d_head, d_head)
        proj = np.empty(3 * D + 2 * n_heads)
        o = np.empty(D)
        h_out = np.empty(hidden)
        self._L.oracle_gdn_block(hidden, n_heads, d_head, bits, rq, rv, h, S, proj, o, h_out)
        return dict(proj=proj, o=o, h_out=h_out, state=S)

    # -- composite -------------------------------------------------------
    def route(self, router, router_dtype, gate_vec, gate_dtype, x, top_k, renorm):
        """Router -> softmax -> top-K -> weights, plus the shared sigmoid gate."""
        logits = self.router(router, router_dtype, x)
        p = self.softmax(logits)
        idx = self.topk(logits, top_k)
        w = self.topk_weights(p, idx, renorm)
        sigma = self.shared_gate(gate_vec, gate_dtype, x)
        return dict(logits=logits, p=p, idx=idx, w=w, sigma=sigma)

    def layer(self, *, hidden, inter, n_experts, top_k, bits_routed, bits_shared,
              renorm, router, router_dtype, gate_vec, gate_dtype, experts,
              expert_stride, shared_record, x, h_res):
        """Whole layer with every routed record on the host (small shapes)."""
        router = _raw(router, router_dtype)
        gate_vec = _raw(gate_vec, gate_dtype)
        experts = np.ascontiguousarray(experts, dtype=np.uint8).reshape(-1)
        shared_record = np.ascontiguousarray(shared_record, dtype=np.uint8).reshape(-1)
        assert experts.size >= (n_experts - 1) * expert_stride + self.record_bytes(hidden, inter, bits_routed)
        x = np.ascontiguousarray(x, dtype=np.float64)
        h_res = np.ascontiguousarray(h_res, dtype=np.float64)
        K = top_k
        logits = np.empty(n_experts); p = np.empty(n_experts)
        idx = np.empty(K, dtype=np.int32); w = np.empty(K)
        sigma = C.c_double(0.0)
        h = np.empty((K + 1) * inter); y = np.empty((K + 1) * hidden); out = np.empty(hidden)
        self._L.oracle_layer(hidden, inter, n_experts, K, bits_routed, bits_shared, int(renorm),
                             DTYPE_CODE[router_dtype], router.ctypes.data,
                             DTYPE_CODE[gate_dtype], gate_vec.ctypes.data,
                             experts, expert_stride, shared_record, x, h_res,
                             logits, p, idx, w, C.byref(sigma), h, y, out)
        return dict(logits=logits, p=p, idx=idx, w=w, sigma=sigma.value,
                    h=h.reshape(K + 1, inter), y=y.reshape(K + 1, hidden), out=out)


_default: Oracle | None = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
