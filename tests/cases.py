"""Seeded test cases: inputs from the generator, gap enforcement and expected
values from the fp64 oracle (never from the HIP path).

Input recipe per workload (see the design notes):
  tiny       x ~ N(0,1) fp32 and h_res ~ N(0,1) fp32, independent
  q4/q2      h_res ~ N(0,1) fp32, x = bf16(RMSNorm(h_res)) (RMSNorm in fp64)
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
                    bits_shared: int | None = None) -> LayerCase:
    """`records_from(expert_id) -> bytes` overrides the generator (tests that
    plant special experts)."""
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
