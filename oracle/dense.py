"""Dense NumPy brute force of the MoE layer -- TEST INFRASTRUCTURE ONLY.

Written separately from the C oracle: it unpacks every code with vectorised bit
operations, materialises each weight matrix as a dense fp64 array
(w = q*scale + bias), and then uses library primitives (matmul, exp, a stable
argsort).  Meant for tiny shapes, to cross-check the C oracle.
"""
from __future__ import annotations

import numpy as np


def _bf16(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def unpack_codes(words: np.ndarray, rows: int, cols: int, bits: int) -> np.ndarray:
    """[rows][cols] integer codes from packed words (little-endian fields)."""
    per = 32 // bits
    w = np.asarray(words, dtype=np.uint32).reshape(rows, cols // per)
    shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))
    fields = (w[:, :, None] >> shifts[None, None, :]) & np.uint32((1 << bits) - 1)
    return fields.reshape(rows, cols).astype(np.int64)


def dense_matrix(words, sb, rows, cols, bits, group=64) -> np.ndarray:
    q = unpack_codes(words, rows, cols, bits).astype(np.float64)
    sbw = np.asarray(sb, dtype=np.uint32).reshape(rows, cols // group)
    s = np.repeat(_bf16((sbw & np.uint32(0xFFFF)).astype(np.uint16)), group, axis=1)
    b = np.repeat(_bf16((sbw >> np.uint32(16)).astype(np.uint16)), group, axis=1)
    return q * s + b


def _sections(record, hidden, inter, bits):
    def up(n):
        return (n + 255) // 256 * 256
    gc = inter * hidden * bits // 8
    dc = hidden * inter * bits // 8
    gs = inter * (hidden // 64) * 4
    ds = hidden * (inter // 64) * 4
    sizes = [gc, gc, dc, gs, gs, ds]
    out, off = [], 0
    rec = np.asarray(record, dtype=np.uint8)
    for n in sizes:
        out.append(rec[off:off + n].view(np.uint32))
        off += up(n)
    return out


def expert_matrices(record, hidden, inter, bits):
    g, u, d, sg, su, sd = _sections(record, hidden, inter, bits)
    return (dense_matrix(g, sg, inter, hidden, bits),
            dense_matrix(u, su, inter, hidden, bits),
            dense_matrix(d, sd, hidden, inter, bits))


def expert(record, hidden, inter, bits, x):
    Wg, Wu, Wd = expert_matrices(record, hidden, inter, bits)
    a = Wg @ x
    u = Wu @ x
    h = a / (1.0 + np.exp(-a)) * u
    return h, Wd @ h


def layer(*, hidden, inter, n_experts, top_k, bits_routed, bits_shared, renorm,
          router, router_dtype, gate_vec, gate_dtype, experts, expert_stride,
          shared_record, x, h_res):
    x = np.asarray(x, dtype=np.float64)
    Wr = router.astype(np.float64) if router_dtype == "f32" else _bf16(router)
    g = gate_vec.astype(np.float64) if gate_dtype == "f32" else _bf16(gate_vec)
    logits = Wr @ x
    z = np.exp(logits - logits.max())
    p = z / z.sum()
    order = np.argsort(-logits, kind="stable")
    idx = order[:top_k].astype(np.int32)
    w = p[idx]
    if renorm:
        w = w / w.sum()
    sigma = 1.0 / (1.0 + np.exp(-(g @ x)))
    experts = np.asarray(experts, dtype=np.uint8).reshape(-1)
    hs, ys = [], []
    for e in idx:
        rec = experts[int(e) * expert_stride:]
        h, y = expert(rec, hidden, inter, bits_routed, x)
        hs.append(h); ys.append(y)
    h, y = expert(shared_record, hidden, inter, bits_shared, x)
    hs.append(h); ys.append(y)
    Y = np.stack(ys)
    out = np.asarray(h_res, dtype=np.float64) + w @ Y[:top_k] + sigma * Y[top_k]
    return dict(logits=logits, p=p, idx=idx, w=w, sigma=sigma, h=np.stack(hs), y=Y, out=out)


def gdn_block(rec_qko, rec_vab, hidden, n_heads, d_head, bits, h, state):
    """The linear-attention block on dense matrices: x = RMSNorm(h), the
    projections as matrix products, unit-length q and k per head, sigmoid
    gates, the delta rule in its closed matrix form
    S_new = alpha S (I - beta k k^T) + beta v k^T, o = S_new q, and h + W_o o."""
    D = n_heads * d_head
    Wq, Wk, Wo = expert_matrices(rec_qko, hidden, D, bits)
    Wv, Wab, _ = expert_matrices(rec_vab, hidden, D, bits)
    h = np.asarray(h, dtype=np.float64)
    x = h / np.sqrt(np.mean(h * h) + 1e-6)
    q = (Wq @ x).reshape(n_heads, d_head)
    k = (Wk @ x).reshape(n_heads, d_head)
    v = (Wv @ x).reshape(n_heads, d_head)
    ab = Wab[:2 * n_heads] @ x
    q = q / np.sqrt(np.sum(q * q, axis=1, keepdims=True) + 1e-6)
    k = k / np.sqrt(np.sum(k * k, axis=1, keepdims=True) + 1e-6)
    alpha = 1.0 / (1.0 + np.exp(-ab[:n_heads]))
    beta = 1.0 / (1.0 + np.exp(-ab[n_heads:]))
    S = np.asarray(state, dtype=np.float64).reshape(n_heads, d_head, d_head)
    eye = np.eye(d_head)
    Sn = np.stack([alpha[i] * S[i] @ (eye - beta[i] * np.outer(k[i], k[i]))
                   + beta[i] * np.outer(v[i], k[i]) for i in range(n_heads)])
    o = np.einsum("hij,hj->hi", Sn, q).reshape(D)
    return dict(o=o, h_out=h + Wo @ o, state=Sn, proj=np.concatenate([(Wq @ x), (Wk @ x), (Wv @ x), ab]))
