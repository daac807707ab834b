"""Benchmark of the MoE expert hot path on one MI355X.

Workload (N=1): the Qwen3.5-397B-A17B-shaped MoE layer decode at batch 1 --
hidden 4096, expert intermediate 1024, 512 routed experts, top-4 plus one
sigmoid-gated shared expert, 4-bit groupwise-affine experts (group 64, bf16
scale/bias), bf16 router and x.  Synthetic weights and inputs (seeded).

A step is one replay of a HIP graph that holds R = 128 independent layer
decodes (a rotation set: distinct router, shared-gate vector, shared expert and
activation per instance over one 512-expert pool, 5 GB touched per replay), so
that no layer's weights are still in the 256 MB Infinity Cache when it runs.
`value` is the decode latency of one layer = step time / R.

Also reported: per-kernel durations from HIP events that each kernel's dispatch
records itself (the library's timing hook, one eager pass over the rotation
set), the roofline of the dominant kernel (shared + routed gate/up), and the
fp64 CPU oracle timed on a bounded sample on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode latency (us) and effective HBM GB/s (% of peak), 4-bit, batch 1"
PEAK_GBPS = 8000.0  # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", "--iters", dest="steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--instances", type=int, default=128)
    ap.add_argument("--workload", "--config", dest="workload", default="q4_layer",
                    choices=["q4_layer", "q2_layer", "q4_stack", "q4_stack_gdn", "q4_batch16", "gdn_step",
                             "q4_tier"])
    ap.add_argument("--tier-slots", type=int, default=128,
                    help="q4_tier: routed records the device cache holds")
    ap.add_argument("--tier-ar", type=float, default=0.95,
                    help="q4_tier: AR(1) coefficient of consecutive tokens' activations")
    ap.add_argument("--tier-tokens", type=int, default=256, help="q4_tier: timed tokens")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-stack", action="store_true",
                    help="q4_layer: skip the 60-layer stack figure reported beside the layer")
    ap.add_argument("--stack-steps", type=int, default=10,
                    help="q4_layer: timed tokens of the 60-layer stack figure")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile-passes", type=int, default=3)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (counter scaling for rocprofv3 --pmc)")
    ap.add_argument("--seed", type=int, default=0,
                    help="offset added to every seed of the synthetic weights and activations")
    ap.add_argument("--bits", type=int, choices=[2, 4], default=None,
                    help="width of routed and shared experts (default: the workload's)")
    ap.add_argument("--renorm", type=int, choices=[0, 1], default=1,
                    help="1: the K selected probabilities are renormalised to sum 1")
    ap.add_argument("--x-dtype", choices=["bf16", "f32"], default=None,
                    help="single-layer workloads: dtype of the layer input x (default: the workload's)")
    args = ap.parse_args()
    OPTS.update(seed=args.seed, renorm=bool(args.renorm))
    return args


# options the weight and input builders read (set from the command line)
OPTS = {"seed": 0, "renorm": True}


def workload_config(args):
    """The named workload's configuration with the command line's overrides
    (--bits, --x-dtype); an overridden workload gets a name that says so."""
    import dataclasses
    from bit_dequant_expert_route_amd import synth
    cfg = synth.CONFIGS["q4_layer" if args.workload == "q4_tier" else args.workload]
    over, tags = {}, []
    if args.bits and (args.bits != cfg.bits_routed or args.bits != cfg.bits_shared):
        over.update(bits_routed=args.bits, bits_shared=args.bits)
        tags.append(f"bits{args.bits}")
    if args.x_dtype and args.x_dtype != cfg.x_dtype:
        over["x_dtype"] = args.x_dtype
        tags.append(f"x{args.x_dtype}")
    if not over:
        return cfg
    return dataclasses.replace(cfg, name=cfg.name + "+" + "+".join(tags), **over)


def kernel_bytes(cfg):
    """Algorithmic bytes per launch of each kernel of one layer decode."""
    from bit_dequant_expert_route_amd import synth
    H, I, E, K = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k

    def mat(rows, cols, bits):
        return rows * cols * bits // 8 + rows * (cols // 64) * 4
    xb = H * (2 if cfg.x_dtype == "bf16" else 4)
    rb = 2 if cfg.router_dtype == "bf16" else 4
    # the shared expert's gate/up runs with the routed gate/up when both have
    # the same width, otherwise with the router
    shared_gu = 2 * mat(I, H, cfg.bits_shared) + I * 4
    same = cfg.bits_shared == cfg.bits_routed
    head = E * H * rb + H * rb + xb + E * 4 + 4 + (0 if same else shared_gu)
    gateup = K * 2 * mat(I, H, cfg.bits_routed) + xb + E * 4 + K * I * 4 + K * 8 + (shared_gu if same else 0)
    down = (K * mat(H, I, cfg.bits_routed) + mat(H, I, cfg.bits_shared) + K * I * 4 + I * 4
            + 2 * H * 4 + K * 8 + 4)
    weights = cfg.weight_bytes_per_token_layer()
    assert weights == E * H * rb + H * rb + K * synth.record_layout(H, I, cfg.bits_routed).total \
        + synth.record_layout(H, I, cfg.bits_shared).total
    return dict(head=head, gateup=gateup, down_combine=down, layer_weights=weights,
                layer_total=head + gateup + down)


def source_sha():
    """Hash of every kernel and library source (the counter summaries in
    profiles/ name the sources they were taken on)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_dequant_expert_route_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def profile_summary(workload, kernel):
    """The committed rocprofv3 counter summary of a kernel, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_sha") != source_sha():
        return None
    return d


def traffic_from_profiles(workload, kernel):
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, scaled by the copy
    probe) from the committed summary."""
    d = profile_summary(workload, kernel)
    return d.get("hbm_bytes_per_launch") if d else None


def valu_from_profiles(workload, kernel, live_us):
    """VALU issue bound of the kernel (SQ_INSTS_VALU x 4 cycles spread over the
    1,024 SIMDs at 2.4 GHz) from the committed summary, and its share of the
    kernel's live duration: which ceiling binds, next to the HBM roofline."""
    d = profile_summary(workload, kernel)
    if not d or d.get("valu_issue_us") is None:
        return None
    return {"instr_per_wave": d["valu_instr_per_wave"], "issue_bound_us": d["valu_issue_us"],
            "live_us": round(live_us, 3), "frac": round(d["valu_issue_us"] / live_us, 4)}


def build_rotation(cfg, R, seed0=1000):
    seed0 += OPTS["seed"]
    import torch
    from bit_dequant_expert_route_amd import moe, synth
    H, I, E = cfg.hidden, cfg.inter, cfg.n_experts
    rb = synth.record_layout(H, I, cfg.bits_routed).total
    sb = synth.record_layout(H, I, cfg.bits_shared).total
    pool = torch.empty(E * rb, dtype=torch.uint8, device="cuda")
    moe.fill_experts(pool, rb, E, seed0, 0, 0, H, I, cfg.bits_routed,
                     synth.dist_for_bits(cfg.bits_routed))
    shared = torch.empty(R * sb, dtype=torch.uint8, device="cuda")
    moe.fill_experts(shared, sb, R, seed0, 0, synth.SHARED_GEN_ID, H, I, cfg.bits_shared,
                     synth.dist_for_bits(cfg.bits_shared))
    g = torch.Generator(device="cuda")
    g.manual_seed(seed0)
    layers, xs, hres = [], [], []
    for i in range(R):
        router = (torch.randn(E, H, generator=g, device="cuda") * synth.ROUTER_STD).to(torch.bfloat16)
        gate = (torch.randn(H, generator=g, device="cuda") * synth.GATEVEC_STD).to(torch.bfloat16)
        h = torch.randn(H, generator=g, device="cuda")
        x = h / torch.sqrt(torch.mean(h * h) + 1e-6)
        x = x.to(torch.bfloat16) if cfg.x_dtype == "bf16" else x
        layers.append(moe.Layer(hidden=H, inter=I, n_experts=E, top_k=cfg.top_k,
                                bits_routed=cfg.bits_routed, bits_shared=cfg.bits_shared,
                                renorm=OPTS["renorm"], router=router, gate_vec=gate, experts=pool,
                                expert_stride=rb, shared_expert=shared[i * sb:(i + 1) * sb]))
        xs.append(x)
        hres.append(h)
    torch.cuda.synchronize()
    return layers, xs, hres, pool, shared


def cpu_baseline(cfg, budget_s):
    """fp64 oracle on the host: route + K routed experts + shared + combine for
    as many layer instances as fit the time budget, on all the oracle's
    threads, then on one thread for a third of that budget.  The instances
    are the timed rotation's first ones (same routers, gate vectors, x,
    residuals and records) when the GPU leg kept them, else fresh draws of
    the same recipe."""
    import oracle
    from bit_dequant_expert_route_amd import synth
    orc = oracle.get()
    H, I = cfg.hidden, cfg.inter
    rot = ROTATION_HOST if ROTATION_HOST.get("cfg") == cfg.name else None

    def inputs(i, first):
        if rot:
            d = rot["instances"][i % len(rot["instances"])]
            return (rot["seed0"], d["router"], d["gate"], d["x"], d["h_res"], d["shared_id"])
        seed = first + i
        h_res = synth.residual(cfg, seed)
        x64 = orc.rmsnorm(h_res.astype(np.float64))
        xb = synth.bf16_to_f32(synth.f64_to_bf16_rne(x64)).astype(np.float64)
        return (seed, synth.router_weights(cfg, seed), synth.shared_gate_vector(cfg, seed), xb,
                h_res.astype(np.float64), synth.SHARED_GEN_ID)

    def sample(budget, first):
        times = []
        t_end = time.perf_counter() + budget
        i = 0
        while time.perf_counter() < t_end or i == 0:
            seed, router, gate, xb, h_res, shared_id = inputs(i, first)
            # weight generation is excluded from the timed region
            logits = orc.router(router, cfg.router_dtype, xb)
            idx = orc.topk(logits, cfg.top_k)
            recs = [synth.make_record(seed, 0, int(e), H, I, cfg.bits_routed) for e in idx]
            shared = synth.make_record(seed, 0, shared_id, H, I, cfg.bits_shared)
            t0 = time.perf_counter()
            r = orc.route(router, cfg.router_dtype, gate, cfg.gate_dtype, xb, cfg.top_k, OPTS["renorm"])
            ys = [orc.expert(rec, H, I, cfg.bits_routed, xb)[1] for rec in recs]
            ysh = orc.expert(shared, H, I, cfg.bits_shared, xb)[1]
            orc.combine(h_res, np.stack(ys), r["w"], ysh, r["sigma"])
            times.append(time.perf_counter() - t0)
            i += 1
        return times

    threads = orc.max_threads()
    times = sample(budget_s, 5000)
    orc.set_threads(1)
    try:
        one = sample(budget_s / 3.0, 6000)
    finally:
        orc.set_threads(threads)
    which = (f"cycling over the first {len(rot['instances'])} layer instances of the timed rotation"
             if rot else "fresh draws of the workload's recipe")
    return dict(value=float(np.median(times) * 1e6), unit="us", cores=threads, kind="oracle",
                sample=f"{len(times)} single-token layer decodes of the {cfg.name} workload, {which} "
                       f"(fp64 oracle, OpenMP over output rows, weight generation excluded), median",
                value_1_core=float(np.median(one) * 1e6), sample_1_core=f"{len(one)} more decodes on one thread, median",
                cpu_model=cpu_model())


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gdn_bytes_per_layer(cfg):
    """HBM bytes of one linear-attention block for one token: the q/k/v
    projections and the 2 heads gate rows, the output projection, the state
    read and written."""
    H, D, nh, b = cfg.hidden, cfg.gdn_heads * cfg.gdn_head_dim, cfg.gdn_heads, cfg.gdn_bits

    def mat(rows, cols):
        return rows * cols * b // 8 + rows * (cols // 64) * 4
    state = nh * cfg.gdn_head_dim * cfg.gdn_head_dim * 4
    return 3 * mat(D, H) + mat(2 * nh, H) + mat(H, D) + 2 * state + (3 * D + 2 * nh) * 4 * 2 + D * 4 * 2


def bench_stack(cfg, args):
    """One token through the resident 60-layer stack (217 GB at 4 bits): a HIP
    graph of the whole stack, replayed; every layer has its own 512 experts, so
    nothing is cache-resident.  With cfg.gdn_heads, the linear-attention
    layers (45 of 60) open with their block (own projections and 4 MiB
    state).  Returns (ms per token, per-kernel live us)."""
    import torch
    from bit_dequant_expert_route_amd import moe, synth
    H, I, E, L = cfg.hidden, cfg.inter, cfg.n_experts, cfg.n_layers
    rb = synth.record_layout(H, I, cfg.bits_routed).total
    sb = synth.record_layout(H, I, cfg.bits_shared).total
    g = torch.Generator(device="cuda")
    S = 3000 + OPTS["seed"]
    g.manual_seed(S)
    layers, keep, gdn = [], [], []
    use_gdn = cfg.gdn_heads > 0
    D = cfg.gdn_heads * cfg.gdn_head_dim
    for l in range(L):
        if use_gdn and not synth.is_attention_layer(l):
            gb = synth.record_layout(H, D, cfg.gdn_bits).total
            recs = []
            for gid in (synth.GDN_QKO_GEN_ID, synth.GDN_VAB_GEN_ID):
                r = torch.empty(gb, dtype=torch.uint8, device="cuda")
                moe.fill_experts(r, gb, 1, S, l, gid, H, D, cfg.gdn_bits,
                                 synth.dist_for_bits(cfg.gdn_bits))
                recs.append(r)
            st = torch.randn(cfg.gdn_heads, cfg.gdn_head_dim, cfg.gdn_head_dim, generator=g,
                             device="cuda") * 0.1
            gdn.append(dict(n_heads=cfg.gdn_heads, d_head=cfg.gdn_head_dim, bits=cfg.gdn_bits,
                            rec_qko=recs[0], rec_vab=recs[1], state=st))
        else:
            gdn.append(None)
        pool = torch.empty(E * rb, dtype=torch.uint8, device="cuda")
        moe.fill_experts(pool, rb, E, S, l, 0, H, I, cfg.bits_routed, synth.dist_for_bits(cfg.bits_routed))
        shared = torch.empty(sb, dtype=torch.uint8, device="cuda")
        moe.fill_experts(shared, sb, 1, S, l, synth.SHARED_GEN_ID, H, I, cfg.bits_shared,
                         synth.dist_for_bits(cfg.bits_shared))
        router = (torch.randn(E, H, generator=g, device="cuda") * synth.ROUTER_STD).to(torch.bfloat16)
        gate = (torch.randn(H, generator=g, device="cuda") * synth.GATEVEC_STD).to(torch.bfloat16)
        layers.append(moe.Layer(hidden=H, inter=I, n_experts=E, top_k=cfg.top_k,
                                bits_routed=cfg.bits_routed, bits_shared=cfg.bits_shared,
                                renorm=OPTS["renorm"], router=router, gate_vec=gate, experts=pool,
                                expert_stride=rb, shared_expert=shared))
    stack = moe.GdnStack(layers, gdn) if use_gdn else moe.Stack(layers)
    ws = stack.workspace()
    updates = torch.randn(L, H, generator=g, device="cuda").to(torch.bfloat16)
    h = torch.randn(H, generator=g, device="cuda")
    K = cfg.top_k
    idx_log = torch.empty(L, K, dtype=torch.int32, device="cuda")
    w_log = torch.empty(L, K, device="cuda")
    decode = moe.stack_decode_gdn if use_gdn else moe.stack_decode
    decode(stack, updates, h, idx_log, w_log, ws)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        if use_gdn:
            moe.capture_begin(s)
            decode(stack, updates, h, idx_log, w_log, ws, stream=s)
            graph = moe.capture_end(s, keep=(stack, updates, h, idx_log, w_log, ws))
        else:
            graph = moe.graph_stack(stack, updates, h, idx_log, w_log, ws, s)
    for _ in range(args.warmup):
        graph.launch(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(args.steps):
        graph.launch(s)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    assert bool(torch.isfinite(h).all())
    n_launch = args.profile_passes * L * 7 + 4
    moe.profile_begin(n_launch)
    for _ in range(args.profile_passes):
        decode(stack, updates, h, idx_log, w_log, ws)
    rec = moe.profile_end(n_launch)
    graph.destroy()
    return ms, rec, dict(layers=L, distinct=None)


def stack_figure(args):
    """The 60-layer resident stack (217 GB of experts, one token through every
    layer, graph-replayed) measured in the same run as the layer: per-token
    latency, per layer, and its effective HBM rate over the layers' bytes."""
    import gc
    import torch
    from bit_dequant_expert_route_amd import synth
    gc.collect()
    torch.cuda.empty_cache()
    cfg = synth.CONFIGS["q4_stack"]
    sargs = argparse.Namespace(**vars(args))
    sargs.steps, sargs.warmup, sargs.profile_passes = args.stack_steps, 2, 1
    t0 = time.perf_counter()
    ms_token, rec, _ = bench_stack(cfg, sargs)
    wall = time.perf_counter() - t0
    per = {}
    for name, ms in rec:
        per.setdefault(name, []).append(ms)
    lb = kernel_bytes(cfg)["layer_total"] * cfg.n_layers
    gbps = lb / (ms_token * 1e-3) / 1e9
    out = {"workload": f"q4_stack: {cfg.n_layers} layers of the q4 layer shape, each with its own "
                       f"512 experts (217 GB resident), one token, h += u_l and RMSNorm between "
                       f"layers, one HIP graph per token",
           "us_per_token": round(ms_token * 1000.0, 2),
           "us_per_layer": round(ms_token * 1000.0 / cfg.n_layers, 3),
           "tokens_per_s": round(1000.0 / ms_token, 2),
           "hbm_bytes_per_token": lb, "effective_GBps": round(gbps, 1),
           "pct_hbm_peak": round(100.0 * gbps / PEAK_GBPS, 2),
           "steps": sargs.steps, "warmup": sargs.warmup,
           "kernels_us": {k: round(float(np.mean(v) * 1000.0), 3) for k, v in per.items()},
           "leg_wall_s": round(wall, 1)}
    gc.collect()
    torch.cuda.empty_cache()
    return out


def bench_batch(cfg, args):
    """Rotation set of R 16-token layer calls over one 512-expert pool; tokens of
    an instance are correlated (h_t = sqrt(0.5) z0 + sqrt(0.5) z_t) so that each
    call touches about 40 distinct routed experts."""
    import torch
    from bit_dequant_expert_route_amd import moe, synth
    H, I, E, T, K = cfg.hidden, cfg.inter, cfg.n_experts, cfg.n_tokens, cfg.top_k
    R = min(args.instances, 16)
    rb = synth.record_layout(H, I, cfg.bits_routed).total
    sb = synth.record_layout(H, I, cfg.bits_shared).total
    pool = torch.empty(E * rb, dtype=torch.uint8, device="cuda")
    S = 4000 + OPTS["seed"]
    moe.fill_experts(pool, rb, E, S, 0, 0, H, I, cfg.bits_routed, synth.dist_for_bits(cfg.bits_routed))
    shared = torch.empty(R * sb, dtype=torch.uint8, device="cuda")
    moe.fill_experts(shared, sb, R, S, 0, synth.SHARED_GEN_ID, H, I, cfg.bits_shared,
                     synth.dist_for_bits(cfg.bits_shared))
    g = torch.Generator(device="cuda")
    g.manual_seed(S)
    layers, xs, hres = [], [], []
    for i in range(R):
        router = (torch.randn(E, H, generator=g, device="cuda") * synth.ROUTER_STD).to(torch.bfloat16)
        gate = (torch.randn(H, generator=g, device="cuda") * synth.GATEVEC_STD).to(torch.bfloat16)
        z0 = torch.randn(1, H, generator=g, device="cuda")
        h = (0.5 ** 0.5) * z0 + (0.5 ** 0.5) * torch.randn(T, H, generator=g, device="cuda")
        x = (h / torch.sqrt(torch.mean(h * h, dim=1, keepdim=True) + 1e-6)).to(torch.bfloat16)
        layers.append(moe.Layer(hidden=H, inter=I, n_experts=E, top_k=K,
                                bits_routed=cfg.bits_routed, bits_shared=cfg.bits_shared,
                                renorm=OPTS["renorm"], router=router, gate_vec=gate, experts=pool,
                                expert_stride=rb, shared_expert=shared[i * sb:(i + 1) * sb]))
        xs.append(x.contiguous())
        hres.append(h.contiguous())
    out = torch.empty(T, H, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, device="cuda")
    ws = layers[0].workspace(T)
    distinct = []
    for i in range(R):
        moe.layer_decode(layers[i], xs[i], hres[i], out, idx, w, ws)
        distinct.append(len(set(idx.cpu().numpy().reshape(-1).tolist())))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        moe.capture_begin(s)
        for i in range(R):
            moe.layer_decode(layers[i], xs[i], hres[i], out, idx, w, ws, stream=s)
        graph = moe.capture_end(s, keep=(layers, xs, hres, out, idx, w, ws))
    for _ in range(args.warmup):
        graph.launch(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(args.steps):
        graph.launch(s)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps / R
    n_launch = args.profile_passes * R * (4 + 4 * T)
    moe.profile_begin(n_launch)
    for _ in range(args.profile_passes):
        for i in range(R):
            moe.layer_decode(layers[i], xs[i], hres[i], out, idx, w, ws)
    rec = moe.profile_end(n_launch)
    graph.destroy()
    return ms, rec, dict(instances=R, distinct=float(np.mean(distinct)))


GDN_LAYERS, GDN_HEADS, GDN_DK, GDN_DV = 45, 64, 128, 128


def bench_gdn(args):
    """The linear-attention decode step of every linear-attention layer (45,
    each with its own 64 x 128 x 128 fp32 state, 4 MiB) captured in one graph
    and replayed; returns (ms per layer step, live per-kernel records)."""
    import torch
    from bit_dequant_expert_route_amd import moe
    g = torch.Generator(device="cuda")
    g.manual_seed(4500 + OPTS["seed"])
    L, Hh, dk, dv = GDN_LAYERS, GDN_HEADS, GDN_DK, GDN_DV
    states = [torch.randn(1, Hh, dv, dk, generator=g, device="cuda") * 0.1 for _ in range(L)]
    def unit(t):
        return (t / t.norm(dim=-1, keepdim=True)).contiguous()
    qs = [unit(torch.randn(1, Hh, dk, generator=g, device="cuda")) for _ in range(L)]
    ks = [unit(torch.randn(1, Hh, dk, generator=g, device="cuda")) for _ in range(L)]
    vs = [torch.randn(1, Hh, dv, generator=g, device="cuda") for _ in range(L)]
    al = [0.9 + 0.1 * torch.rand(1, Hh, generator=g, device="cuda") for _ in range(L)]
    be = [torch.rand(1, Hh, generator=g, device="cuda") for _ in range(L)]
    outs = [torch.empty(1, Hh, dv, device="cuda") for _ in range(L)]

    def one_pass(stream=None):
        for i in range(L):
            moe.gdn_step(qs[i], ks[i], vs[i], al[i], be[i], states[i], outs[i], stream=stream)

    one_pass()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        moe.capture_begin(s)
        one_pass(s)
        graph = moe.capture_end(s, keep=(states, qs, ks, vs, al, be, outs))
    for _ in range(args.warmup):
        graph.launch(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(args.steps):
        graph.launch(s)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps / L
    assert all(bool(torch.isfinite(t).all()) for t in states)
    n_launch = args.profile_passes * L
    moe.profile_begin(n_launch)
    for _ in range(args.profile_passes):
        one_pass()
    rec = moe.profile_end(n_launch)
    graph.destroy()
    return ms, rec


def bench_layer(cfg, args):
    """Rotation set of R single-token layer decodes captured in one graph;
    returns (ms per layer, per-kernel live records, extras)."""
    import torch
    from bit_dequant_expert_route_amd import moe
    R = args.instances
    layers, xs, hres, pool, shared = build_rotation(cfg, R)
    K = cfg.top_k
    out = torch.empty(cfg.hidden, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, device="cuda")
    ws = layers[0].workspace(1)

    def one_pass(stream=None):
        for i in range(R):
            moe.layer_decode(layers[i], xs[i], hres[i], out, idx, w, ws, stream=stream)

    one_pass()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        moe.capture_begin(s)
        one_pass(s)
        graph = moe.capture_end(s, keep=(layers, xs, hres, out, idx, w, ws))
    for _ in range(args.warmup):
        graph.launch(s)
    torch.cuda.synchronize()
    # an event between replays: the whole span gives the value, each replay
    # its own latency (median, p90)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(s)
    for k in range(args.steps):
        graph.launch(s)
        ev[k + 1].record(s)
    torch.cuda.synchronize()
    ms_layer = ev[0].elapsed_time(ev[-1]) / args.steps / R
    per = [ev[k].elapsed_time(ev[k + 1]) * 1000.0 / R for k in range(args.steps)]
    # per-kernel durations (events recorded by each dispatch, eager launches)
    n_launch = args.profile_passes * R * 4
    moe.profile_begin(n_launch)
    for _ in range(args.profile_passes):
        one_pass()
    rec = moe.profile_end(n_launch)
    graph.destroy()
    extra = {"replay_us_per_layer_median": round(float(np.median(per)), 3),
             "replay_us_per_layer_p90": round(float(np.percentile(per, 90)), 3)}
    extra.update(launch_inclusive(layers, xs, hres, out, idx, w, ws, args))
    keep_for_cpu(cfg, layers, xs, hres)
    return ms_layer, rec, extra


# host copies of the first rotation instances, for the CPU oracle leg
ROTATION_HOST = {}
CPU_INSTANCES = 32


def keep_for_cpu(cfg, layers, xs, hres):
    """Copy the router, gate vector, x and residual of the first instances of
    the timed rotation to the host (after the timed region), so that the CPU
    leg decodes the same layers; their records are regenerated on the host,
    bit-identical to the device fill."""
    import torch
    from bit_dequant_expert_route_amd import synth

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
    insts = []
    for i in range(min(len(layers), CPU_INSTANCES)):
        x = host(xs[i])
        x64 = (synth.bf16_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)
        insts.append(dict(router=host(layers[i].router), gate=host(layers[i].gate_vec), x=x64,
                          h_res=host(hres[i]).astype(np.float64), shared_id=synth.SHARED_GEN_ID + i))
    ROTATION_HOST.update(cfg=cfg.name, seed0=1000 + OPTS["seed"], instances=insts)


def launch_inclusive(layers, xs, hres, out, idx, w, ws, args):
    """Two companion figures of the rotation measurement.
    one_layer_graph_us: one graph per layer instance, each replayed as its own
    launch over the same rotation (so the launch overhead is included and the
    data stay cold).  cache_warm_us_per_layer: one graph that calls the first
    instance R times with the same x; its 40 MB then sit in the memory-side
    cache, so this is a cache figure, not an HBM one."""
    import torch
    from bit_dequant_expert_route_amd import moe
    R = len(layers)
    s = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(s):
        for i in range(R):
            moe.capture_begin(s)
            moe.layer_decode(layers[i], xs[i], hres[i], out, idx, w, ws, stream=s)
            graphs.append(moe.capture_end(s))
        moe.capture_begin(s)
        for _ in range(R):
            moe.layer_decode(layers[0], xs[0], hres[0], out, idx, w, ws, stream=s)
        warm = moe.capture_end(s)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(args.steps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / args.steps / R

    def each():
        for g in graphs:
            g.launch(s)

    one = timed(each)
    hot = timed(lambda: warm.launch(s))
    for g in graphs:
        g.destroy()
    warm.destroy()
    return {"one_layer_graph_us": round(one, 3), "cache_warm_us_per_layer": round(hot, 3)}


def bench_tier(cfg, args):
    """One Qwen-shaped 4-bit layer whose 512 routed records (3.6 GB) sit in
    page-locked host memory behind a device cache of --tier-slots records,
    managed on the device (moe_tier_layer_decode: no host round trip; a miss
    is read from host memory by the expert kernels and written into its
    slot).  A stream of tokens with correlated activations (AR(1) over the
    residual: h_t = a h_{t-1} + sqrt(1 - a^2) z_t, x_t = bf16(RMSNorm(h_t)))
    is captured in one graph and replayed once, after an eager warm-up of the
    cache.  The same tokens are also timed on the resident layer, and with the
    cache emptied before every token (every routed expert a miss), which gives
    the rate at which the kernels read records from host memory.  Returns
    (ms per token, per-kernel live records, extras)."""
    import torch
    from bit_dequant_expert_route_amd import moe, synth
    H, I, E, K = cfg.hidden, cfg.inter, cfg.n_experts, cfg.top_k
    S, a, N = args.tier_slots, args.tier_ar, args.tier_tokens
    W = max(args.warmup, 1) * 16
    rb = synth.record_layout(H, I, cfg.bits_routed).total
    sb = synth.record_layout(H, I, cfg.bits_shared).total
    pool = torch.empty(E * rb, dtype=torch.uint8, device="cuda")
    seed = 5000 + OPTS["seed"]
    moe.fill_experts(pool, rb, E, seed, 0, 0, H, I, cfg.bits_routed, synth.dist_for_bits(cfg.bits_routed))
    host = torch.empty(E * rb, dtype=torch.uint8, pin_memory=True)
    host.copy_(pool)
    torch.cuda.synchronize()
    shared = torch.empty(sb, dtype=torch.uint8, device="cuda")
    moe.fill_experts(shared, sb, 1, seed, 0, synth.SHARED_GEN_ID, H, I, cfg.bits_shared,
                     synth.dist_for_bits(cfg.bits_shared))
    cache = torch.empty(S * rb, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    router = (torch.randn(E, H, generator=g, device="cuda") * synth.ROUTER_STD).to(torch.bfloat16)
    gate = (torch.randn(H, generator=g, device="cuda") * synth.GATEVEC_STD).to(torch.bfloat16)
    layer = moe.Layer(hidden=H, inter=I, n_experts=E, top_k=K, bits_routed=cfg.bits_routed,
                      bits_shared=cfg.bits_shared, renorm=OPTS["renorm"], router=router, gate_vec=gate,
                      experts=pool, expert_stride=rb, shared_expert=shared)
    tier = moe.Tier(host, E, rb, cache, S)
    hs = torch.empty(W + N, H, device="cuda")
    h = torch.randn(H, generator=g, device="cuda")
    for t in range(W + N):
        h = a * h + (1.0 - a * a) ** 0.5 * torch.randn(H, generator=g, device="cuda")
        hs[t] = h
    xs = (hs / torch.sqrt(torch.mean(hs * hs, dim=1, keepdim=True) + 1e-6)).to(torch.bfloat16)
    out = torch.empty(H, device="cuda")
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, device="cuda")
    ws = layer.workspace(1)
    st = torch.cuda.Stream()

    def graph_of(fn):
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            moe.capture_begin(st)
            fn(st)
            return moe.capture_end(st)

    def timed_once(gr):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        gr.launch(st)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / N

    timed_tokens = range(W, W + N)
    g_res = graph_of(lambda s_: [moe.layer_decode(layer, xs[t], hs[t], out, idx, w, ws, stream=s_)
                                 for t in timed_tokens])
    g_tier = graph_of(lambda s_: [tier.layer_decode(layer, xs[t], hs[t], out, idx, w, ws, stream=s_)
                                  for t in timed_tokens])

    def all_miss(s_):
        for t in timed_tokens:
            tier.reset(stream=s_)
            tier.layer_decode(layer, xs[t], hs[t], out, idx, w, ws, stream=s_)
    g_miss = graph_of(all_miss)
    g_res.launch(st)
    us_res = timed_once(g_res)
    us_miss = timed_once(g_miss)
    # the measured stream: an empty cache warmed by the first W tokens
    tier.reset()
    for t in range(W):
        tier.layer_decode(layer, xs[t], hs[t], out, idx, w, ws)
    torch.cuda.synchronize()
    h0, m0, b0 = tier.stats()
    us_tok = timed_once(g_tier)
    h1, m1, b1 = tier.stats()
    # per-kernel durations on a few more tokens (eager, dispatch-recorded events)
    n_launch = 4 * 8
    moe.profile_begin(n_launch)
    for t in range(W, W + 8):
        tier.layer_decode(layer, xs[t], hs[t], out, idx, w, ws)
    rec = moe.profile_end(n_launch)
    for gr in (g_res, g_tier, g_miss):
        gr.destroy()
    tier.close()
    hits, misses, read = h1 - h0, m1 - m0, b1 - b0
    # the kernels' rate of reading records from host memory: K records per
    # token beyond the resident time
    link = K * rb / ((us_miss - us_res) * 1e-6) / 1e9
    t_link = read / N / (link * 1e9) * 1e6   # the stream's host reads at that rate
    extra = {"tier_slots": S, "tier_ar": a, "tokens": N, "warmup_tokens": W,
             "hit_rate": round(hits / max(hits + misses, 1), 4),
             "misses_per_token": round(misses / N, 3),
             "host_bytes_read_per_token": int(read / N),
             "resident_us_per_token": round(us_res, 3),
             "all_miss_us_per_token": round(us_miss, 3),
             "host_read_GBps_by_kernels": round(link, 2),
             # the token's host reads at that rate, and what of the token's
             # time is not covered by them (routing before, down + combine
             # after: the hits' and the shared expert's work overlaps them)
             "transfer_us_per_token": round(t_link, 3),
             "outside_transfer_us_per_token": round(us_tok - t_link, 3),
             "link_busy_fraction": round(t_link / us_tok, 3),
             # transfer time that runs under compute: the resident token's
             # time plus the transfer, less the measured token time
             "hidden_transfer_us_per_token": round(us_res + t_link - us_tok, 3),
             "hidden_transfer_fraction": round((us_res + t_link - us_tok) / t_link, 3) if t_link > 0 else None}
    return us_tok / 1000.0, rec, extra


def read_peak_gbps():
    """Streaming-read rate of this GPU: a 4 GiB sum (read-bound), best of 3."""
    import torch
    a = torch.ones(1 << 29, dtype=torch.float64, device="cuda")  # 4 GiB
    a.sum()
    best = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        a.sum()
        e1.record()
        torch.cuda.synchronize()
        best = max(best, a.numel() * 8 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del a
    torch.cuda.empty_cache()
    return best


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only: the hot path is a single-GPU "
                                   "kernel sequence with no sharding or collectives; run with --gpus 1"}))
        sys.exit(2)
    import torch
    from bit_dequant_expert_route_amd import moe, synth

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": a.numel(), "dispatches": 3}))
        return

    if args.workload == "gdn_step":
        ms, rec = bench_gdn(args)
        us = ms * 1000.0
        state = GDN_HEADS * GDN_DV * GDN_DK * 4
        step_bytes = 2 * state + GDN_HEADS * (2 * GDN_DK + 2 * GDN_DV + 2) * 4
        kern = float(np.mean([m for _, m in rec]) * 1000.0)
        achieved = step_bytes / (kern * 1e-6) / 1e9
        line = {
            "metric": "linear-attention (gated delta rule) decode step latency per layer",
            "value": round(us, 3), "unit": "us", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms * GDN_LAYERS, 4),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": f"gdn_step: {GDN_LAYERS} layers x {GDN_HEADS} heads x "
                                   f"{GDN_DV}x{GDN_DK} fp32 state, one token (value = graph time / "
                                   f"{GDN_LAYERS})", "hbm_bytes_per_unit": step_bytes},
            "effective_GBps": round(step_bytes / (us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * step_bytes / (us * 1e-6) / 1e9 / PEAK_GBPS, 2),
            "kernels_us": {"gdn_step": round(kern, 3)},
            "roofline": {"bound": "hbm", "kernel": "k_gdn_step", "achieved": round(achieved, 1),
                         "peak": PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_GBPS, 4),
                         "traffic": traffic_from_profiles("gdn_step", "gdn"), "bytes_per_launch": step_bytes},
            "cpu_baseline": None,
        }
        valu = valu_from_profiles("gdn_step", "gdn", kern)
        if valu:
            line["valu_issue"] = {"kernel": "k_gdn_step", **valu}
        print(json.dumps(line), flush=True)
        return

    read_gbps = read_peak_gbps()
    cfg = workload_config(args)
    kb = kernel_bytes(cfg)
    if args.workload == "q4_tier":
        ms_tok, rec, extra = bench_tier(cfg, args)
        us_per_layer = ms_tok * 1000.0
        ms_per_step = ms_tok * extra["tokens"]
        unit_note = dict(extra)
        bytes_per_unit = kb["layer_total"]
    elif cfg.n_layers > 1:
        ms_token, rec, extra = bench_stack(cfg, args)
        us_per_layer = ms_token * 1000.0 / cfg.n_layers
        ms_per_step = ms_token
        unit_note = {"stack_us_per_token": round(ms_token * 1000.0, 2),
                     "stack_tokens_per_s": round(1000.0 / ms_token, 2)}
        bytes_per_unit = kb["layer_total"]
        if cfg.gdn_heads:
            n_gdn = sum(not synth.is_attention_layer(l) for l in range(cfg.n_layers))
            tok = cfg.n_layers * kb["layer_total"] + n_gdn * gdn_bytes_per_layer(cfg)
            bytes_per_unit = tok // cfg.n_layers
            unit_note.update({"linear_attention_layers": n_gdn, "hbm_bytes_per_token": tok})
    elif cfg.n_tokens > 1:
        ms_call, rec, extra = bench_batch(cfg, args)
        us_per_layer = ms_call * 1000.0
        ms_per_step = ms_call * extra["instances"]
        unit_note = {"tokens_per_call": cfg.n_tokens, "distinct_routed_experts": extra["distinct"],
                     "tokens_per_s": round(cfg.n_tokens * 1e6 / us_per_layer, 1)}
        # weights of the distinct experts + the shared one + the router, once
        bytes_per_unit = int(extra["distinct"] * cfg.record_bytes + cfg.shared_record_bytes
                             + cfg.n_experts * cfg.hidden * 2 + cfg.hidden * 2
                             + cfg.n_tokens * 40960)
    else:
        ms_layer, rec, extra = bench_layer(cfg, args)
        us_per_layer = ms_layer * 1000.0
        ms_per_step = ms_layer * args.instances
        unit_note = {"layer_instances_per_step": args.instances, **extra}
        bytes_per_unit = kb["layer_total"]

    per = {}
    for name, ms in rec:
        per.setdefault(name, []).append(ms)
    kern_us = {k: float(np.mean(v) * 1000.0) for k, v in per.items()}
    dom = "gateup"
    dom_bytes = kb[dom]
    dom_kernel = "k_gateup (shared + routed gate/up + SwiGLU)"
    if cfg.n_tokens > 1:
        # grouped gate/up: each distinct routed expert and the shared one once,
        # the tokens' x and the SwiGLU outputs of every (token, expert) pair
        H, I, T, K = cfg.hidden, cfg.inter, cfg.n_tokens, cfg.top_k
        gu = 2 * (I * H * cfg.bits_routed // 8 + I * (H // 64) * 4)
        dom_bytes = int(round((extra["distinct"] + 1) * gu + T * H * 2 + (T * K + T) * I * 4))
        dom_kernel = "k_gateup_grouped (distinct routed + shared experts, all tokens)"
    achieved = dom_bytes / (kern_us[dom] * 1e-6) / 1e9
    traffic = traffic_from_profiles(args.workload, dom)
    descr = {
        "q4_layer": "MoE layer decode, batch 1" if args.workload != "q4_tier" else
                    f"MoE layer decode, batch 1, routed experts in page-locked host memory behind a "
                    f"{args.tier_slots}-record device cache managed on the device (value = graph time "
                    f"per token over a correlated token stream)",
        "q2_layer": "MoE layer decode, batch 1",
        "q4_stack": f"{cfg.n_layers}-layer resident expert stack, one token (value = per-token time / {cfg.n_layers})",
        "q4_stack_gdn": f"{cfg.n_layers}-layer resident expert stack whose linear-attention layers open with "
                        f"their gated-delta-rule block ({cfg.gdn_heads} heads of {cfg.gdn_head_dim}, 4-bit "
                        f"projections, fp32 state), one token (value = per-token time / {cfg.n_layers})",
        "q4_batch16": f"MoE layer call on {cfg.n_tokens} correlated tokens (value = time per call)",
    }[cfg.name.split("+")[0]]
    line = {
        "metric": METRIC if args.workload != "q4_tier" else
                  "MoE-layer decode latency with the routed experts in host memory (us per token)",
        "value": round(us_per_layer, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {descr}, hidden {cfg.hidden}, "
                               f"expert intermediate {cfg.inter}, {cfg.n_experts} experts, "
                               f"top-{cfg.top_k} + 1 shared, {cfg.bits_routed}-bit experts (group 64, bf16 "
                               f"scale/bias), bf16 router, {cfg.x_dtype} x",
                   "hbm_bytes_per_unit": bytes_per_unit, **unit_note},
        "effective_GBps": round(bytes_per_unit / (us_per_layer * 1e-6) / 1e9, 1),
        "pct_hbm_peak": round(100.0 * bytes_per_unit / (us_per_layer * 1e-6) / 1e9 / PEAK_GBPS, 2),
        "measured_read_peak_GBps": round(read_gbps, 1),
        "pct_measured_read_peak": round(100.0 * bytes_per_unit / (us_per_layer * 1e-6) / 1e9 / read_gbps, 2),
        "kernels_us": {k: round(v, 3) for k, v in kern_us.items()},
        "roofline": {"bound": "hbm", "kernel": dom_kernel,
                     "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": dom_bytes},
        "cpu_baseline": None,
    }
    valu = valu_from_profiles(args.workload, dom, kern_us[dom])
    if valu:
        line["valu_issue"] = {"kernel": dom_kernel, **valu}
    if args.workload == "q4_layer" and not args.no_stack:
        line["stack_60_layers"] = stack_figure(args)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
