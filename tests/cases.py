"""Seeded test cases: inputs from the generator, gap enforcement and expected
values from the fp64 oracle (never from the HIP path).

Input recipe per workload:
  tiny       x ~ N(0,1) fp32 and h_res ~ N(0,1) fp32, independent
  q4/q2      h_res ~ N(0,1) fp32, x = bf16(RMSNorm(h_res)) (RMSNorm in fp64)
  stacks     h0 ~ N(0,1) fp32; per layer a bf16 N(0,1) update u_l, then
             h += u_l, x = RMSNorm(h) in fp32/fp64 (no bf16 rounding of x)
  batches    h_t = sqrt(rho) z0 + sqrt(1-rho) z_t, x_t = bf16(RMSNorm(h_t)),
             rho picked from {0, 0.05, ..., 0.95} so that the number of
             distinct routed experts comes closest to a target
The draw is repeated with attempt = 0, 1, ... until the gap between the K-th
and (K+1)-th largest fp64 logits is at least 1e-3, so that the expert indices
are decided the same way by any correct fp32 evaluation.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
from bit_dequant_expert_route_amd import synth

GAP = 1e-3
TOL = 2e-3


def err_metric(got, want):
    """max_i |g_i - o_i| / max(|o_i|, 1e-2 * rms(o)): elementwise relative error
    with a floor, so that outputs near zero do not make the ratio meaningless."""
    g = np.asarray(got, dtype=np.float64).reshape(-1)
    o = np.asarray(want, dtype=np.float64).reshape(-1)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), 1e-2 * rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(g - o) / den))


def logit_gap(logits, k):
    s = np.sort(np.asarray(logits, dtype=np.float64))[::-1]
    return float(s[k - 1] - s[k]) if s.size > k else float("inf")


@dataclasses.dataclass
class LayerCase:
    cfg: synth.LayerConfig
    seed: int
    attempt: int
    renorm: bool
    router: np.ndarray          # fp32 values or bf16 bits
    gate_vec: np.ndarray
    x: np.ndarray               # fp32 values or bf16 bits, as given to the GPU
    x64: np.ndarray             # the same values in fp64 (what the oracle sees)
    h_res: np.ndarray           # fp32
    route: dict                 # oracle routing (logits, p, idx, w, sigma)
    records: dict               # expert id -> record bytes (routed ones)
    shared: np.ndarray
    expect: dict                # oracle h, y, out for the routed + shared experts

    @property
    def bits_routed(self):
        return self.cfg.bits_routed


def _x_from_hres(orc, h_res, dtype):
    x64 = orc.rmsnorm(h_res.astype(np.float64), 1e-6)
    if dtype == "bf16":
        bits = synth.f64_to_bf16_rne(x64)
        return bits, synth.bf16_to_f32(bits).astype(np.float64)
    xf = x64.astype(np.float32)
    return xf, xf.astype(np.float64)


def make_layer_case(cfg: synth.LayerConfig, seed: int, renorm: bool = True,
                    orc: oracle.Oracle | None = None, records_from=None,
                    bits_shared: int | None = None, router_edit=None) -> LayerCase:
    """`records_from(expert_id) -> bytes` overrides the generator (tests that
    plant special experts).  `router_edit(router, logits) -> router` changes
    the router once the first draw's logits are known (tests that plant exact
    ties); the logit-gap rule is then not applied."""
    orc = orc or oracle.get()
    bits_shared = bits_shared or cfg.bits_shared
    router = synth.router_weights(cfg, seed)
    gate = synth.shared_gate_vector(cfg, seed)
    for attempt in range(1000):
        h_res = synth.residual(cfg, seed, attempt)
        if cfg.name == "tiny":
            x = synth.raw_x(cfg, seed, attempt)
            x64 = x.astype(np.float64)
        else:
            x, x64 = _x_from_hres(orc, h_res, cfg.x_dtype)
        logits = orc.router(router, cfg.router_dtype, x64)
        if router_edit is not None:
            router = router_edit(router, logits)
            break
        if logit_gap(logits, cfg.top_k) >= GAP:
            break
    else:
        raise RuntimeError("no draw with a large enough logit gap")
    route = orc.route(router, cfg.router_dtype, gate, cfg.gate_dtype, x64, cfg.top_k, renorm)
    gen = records_from or (lambda e: synth.make_record(seed, 0, e, cfg.hidden, cfg.inter, cfg.bits_routed))
    records = {int(e): gen(int(e)) for e in route["idx"]}
    shared = synth.make_record(seed, 0, synth.SHARED_GEN_ID, cfg.hidden, cfg.inter, bits_shared)
    hs, ys = [], []
    for e in route["idx"]:
        h, y = orc.expert(records[int(e)], cfg.hidden, cfg.inter, cfg.bits_routed, x64)
        hs.append(h); ys.append(y)
    h_s, y_s = orc.expert(shared, cfg.hidden, cfg.inter, bits_shared, x64)
    out = orc.combine(h_res.astype(np.float64), np.stack(ys), route["w"], y_s, route["sigma"])
    expect = dict(h=np.stack(hs), y=np.stack(ys), h_shared=h_s, y_shared=y_s, out=out)
    return LayerCase(cfg, seed, attempt, renorm, router, gate, x, x64, h_res, route,
                     records, shared, expect)


# ----------------------------------------------------------------------------
# stacks: the oracle walks the layers, redrawing a layer's update until its
# top-K gap is large enough
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class StackCase:
    cfg: synth.LayerConfig
    seed: int
    n_layers: int
    h0: np.ndarray              # fp32 [H]
    updates: np.ndarray         # bf16 bits [L][H] (the accepted draws)
    attempts: list
    routers: list               # per layer, as given to the GPU
    gates: list
    idx: np.ndarray             # [L][K] oracle selection
    w: np.ndarray               # [L][K]
    h: np.ndarray               # fp64 [H] after the last layer
    h_layers: list              # fp64 [H] after each layer


def layer_from_records(orc, cfg, seed, layer, router, gate, x64, h_res64, renorm,
                       bits_shared=None):
    """One layer on the oracle: routing, the selected experts (host generator
    records) and the shared expert, then the combine with h_res."""
    bits_shared = bits_shared or cfg.bits_shared
    route = orc.route(router, cfg.router_dtype, gate, cfg.gate_dtype, x64, cfg.top_k, renorm)
    ys = []
    for e in route["idx"]:
        rec = synth.make_record(seed, layer, int(e), cfg.hidden, cfg.inter, cfg.bits_routed)
        ys.append(orc.expert(rec, cfg.hidden, cfg.inter, cfg.bits_routed, x64)[1])
    shared = synth.make_record(seed, layer, synth.SHARED_GEN_ID, cfg.hidden, cfg.inter, bits_shared)
    y_s = orc.expert(shared, cfg.hidden, cfg.inter, bits_shared, x64)[1]
    out = orc.combine(h_res64, np.stack(ys), route["w"], y_s, route["sigma"])
    return route, out


def make_stack_case(cfg: synth.LayerConfig, seed: int, n_layers: int | None = None,
                    renorm: bool = True, orc: oracle.Oracle | None = None) -> StackCase:
    orc = orc or oracle.get()
    L = n_layers or cfg.n_layers
    h0 = synth.stack_h0(cfg, seed)
    h = h0.astype(np.float64)
    ups, atts, routers, gates, idxs, ws, hl = [], [], [], [], [], [], []
    for l in range(L):
        router = synth.router_weights(cfg, seed, l)
        gate = synth.shared_gate_vector(cfg, seed, l)
        for attempt in range(1000):
            u = synth.layer_update(cfg, seed, l, attempt)
            hr = h + synth.bf16_to_f32(u).astype(np.float64)
            x64 = orc.rmsnorm(hr, 1e-6)
            if logit_gap(orc.router(router, cfg.router_dtype, x64), cfg.top_k) >= GAP:
                break
        else:
            raise RuntimeError(f"layer {l}: no update with a large enough logit gap")
        route, h = layer_from_records(orc, cfg, seed, l, router, gate, x64, hr, renorm)
        ups.append(u); atts.append(attempt); routers.append(router); gates.append(gate)
        idxs.append(route["idx"]); ws.append(route["w"]); hl.append(h.copy())
    return StackCase(cfg, seed, L, h0, np.stack(ups), atts, routers, gates,
                     np.stack(idxs), np.stack(ws), h, hl)


# ----------------------------------------------------------------------------
# stacks with linear-attention layers: in those layers the block's output
# replaces the update, and the state carried in from earlier tokens is what
# is redrawn until the layer's top-K gap is large enough
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class GdnStackCase:
    cfg: synth.LayerConfig
    seed: int
    n_layers: int
    h0: np.ndarray              # fp32 [H]
    updates: np.ndarray         # bf16 bits [L][H] (zero rows in linear-attention layers)
    states0: list               # per layer: fp32 [heads][d][d] initial state, or None
    states: list                # per layer: fp64 state after the token, or None
    attempts: list
    routers: list
    gates: list
    idx: np.ndarray
    w: np.ndarray
    h: np.ndarray               # fp64 [H] after the last layer


def make_gdn_stack_case(cfg: synth.LayerConfig, seed: int, n_layers: int | None = None,
                        renorm: bool = True, orc: oracle.Oracle | None = None,
                        attention=None) -> GdnStackCase:
    """attention(l): whether layer l is a full-attention stand-in (no
    linear-attention block, a bf16 update instead); every fourth layer unless
    given."""
    orc = orc or oracle.get()
    attention = attention or synth.is_attention_layer
    L = n_layers or cfg.n_layers
    H, nh, dh, gb = cfg.hidden, cfg.gdn_heads, cfg.gdn_head_dim, cfg.gdn_bits
    h = synth.stack_h0(cfg, seed).astype(np.float64)
    h0 = h.astype(np.float32)
    ups, s0s, ss, atts, routers, gates, idxs, ws = [], [], [], [], [], [], [], []
    for l in range(L):
        router = synth.router_weights(cfg, seed, l)
        gate = synth.shared_gate_vector(cfg, seed, l)
        attn = attention(l)
        rq = rv = None
        if not attn:
            rq, rv = synth.gdn_records(seed, l, H, nh, dh, gb)
        for attempt in range(1000):
            if attn:
                u = synth.layer_update(cfg, seed, l, attempt)
                hr = h + synth.bf16_to_f32(u).astype(np.float64)
                s0 = s1 = None
            else:
                u = np.zeros(H, dtype=np.uint16)
                s0 = synth.gdn_state0(seed, l, nh, dh, attempt)
                blk = orc.gdn_block(rq, rv, H, nh, dh, gb, h, s0.astype(np.float64))
                hr, s1 = blk["h_out"], blk["state"]
            x64 = orc.rmsnorm(hr, 1e-6)
            if logit_gap(orc.router(router, cfg.router_dtype, x64), cfg.top_k) >= GAP:
                break
        else:
            raise RuntimeError(f"layer {l}: no draw with a large enough logit gap")
        route, h = layer_from_records(orc, cfg, seed, l, router, gate, x64, hr, renorm)
        ups.append(u); s0s.append(s0); ss.append(s1); atts.append(attempt)
        routers.append(router); gates.append(gate); idxs.append(route["idx"]); ws.append(route["w"])
    return GdnStackCase(cfg, seed, L, h0, np.stack(ups), s0s, ss, atts, routers, gates,
                        np.stack(idxs), np.stack(ws), h)


# ----------------------------------------------------------------------------
# correlated token batches
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class BatchCase:
    cfg: synth.LayerConfig
    seed: int
    rho: float
    distinct: int               # distinct routed experts over the batch
    attempts: list
    router: np.ndarray
    gate_vec: np.ndarray
    x: np.ndarray               # [T][H] bf16 bits (or fp32)
    h_res: np.ndarray           # [T][H] fp32
    idx: np.ndarray             # [T][K]
    w: np.ndarray               # [T][K]
    sigma: np.ndarray           # [T]
    out: np.ndarray             # [T][H] fp64


def _batch_draw(orc, cfg, seed, rho, router):
    xs, x64s, hs, atts, idxs = [], [], [], [], []
    for t in range(cfg.n_tokens):
        for attempt in range(1000):
            h = synth.token_residual(cfg, seed, rho, t, attempt)
            x, x64 = _x_from_hres(orc, h, cfg.x_dtype)
            logits = orc.router(router, cfg.router_dtype, x64)
            if logit_gap(logits, cfg.top_k) >= GAP:
                break
        else:
            raise RuntimeError(f"token {t}: no draw with a large enough logit gap")
        xs.append(x); x64s.append(x64); hs.append(h); atts.append(attempt)
        idxs.append(orc.topk(logits, cfg.top_k))
    return xs, x64s, hs, atts, idxs


def make_batch_case(cfg: synth.LayerConfig, seed: int, target_distinct: int | None = None,
                    renorm: bool = True, orc: oracle.Oracle | None = None) -> BatchCase:
    """rho in {0, 0.05, ..., 0.95} bringing the distinct routed count closest
    to target_distinct (ties to the smaller rho); without a target rho = 0."""
    orc = orc or oracle.get()
    router = synth.router_weights(cfg, seed)
    gate = synth.shared_gate_vector(cfg, seed)
    best = None
    rhos = [i * 0.05 for i in range(20)] if target_distinct else [0.0]
    for rho in rhos:
        draw = _batch_draw(orc, cfg, seed, rho, router)
        d = len({int(e) for idx in draw[4] for e in idx})
        score = abs(d - target_distinct) if target_distinct else 0
        if best is None or score < best[0]:
            best = (score, rho, d, draw)
    _, rho, d, (xs, x64s, hs, atts, _) = best
    idx, w, sig, outs = [], [], [], []
    for t in range(cfg.n_tokens):
        route, out = layer_from_records(orc, cfg, seed, 0, router, gate, x64s[t],
                                        hs[t].astype(np.float64), renorm)
        idx.append(route["idx"]); w.append(route["w"]); sig.append(route["sigma"]); outs.append(out)
    return BatchCase(cfg, seed, rho, d, atts, router, gate, np.stack(xs), np.stack(hs),
                     np.stack(idx), np.stack(w), np.array(sig), np.stack(outs))
