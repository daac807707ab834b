"""GPU parity of the resident expert stack (inter-layer step h += u_l,
x = RMSNorm(h) in fp32, then the layer) against the oracle walking the same
layers in fp64.  Per layer the selected experts must match as a set and their
weights per index; the final residual stream and each layer's weights meet
err_metric <= 2e-3.  The router's column tiles (moe_router_tile) must give the
same stack output bit for bit as reading the router rows."""
import numpy as np
import pytest
import torch

from bit_dequant_expert_route_amd import synth
from cases import TOL, err_metric, make_stack_case
from gpu_util import log, to_dev, upload_router

pytestmark = pytest.mark.gpu


def _build(cfg, case):
    from bit_dequant_expert_route_amd import moe
    rb = synth.record_layout(cfg.hidden, cfg.inter, cfg.bits_routed).total
    sb = synth.record_layout(cfg.hidden, cfg.inter, cfg.bits_shared).total
    layers, keep = [], []
    for l in range(case.n_layers):
        pool = torch.empty(cfg.n_experts * rb, dtype=torch.uint8, device="cuda")
        moe.fill_experts(pool, rb, cfg.n_experts, case.seed, l, 0, cfg.hidden, cfg.inter,
                         cfg.bits_routed, synth.dist_for_bits(cfg.bits_routed))
        shared = torch.empty(sb, dtype=torch.uint8, device="cuda")
        moe.fill_experts(shared, sb, 1, case.seed, l, synth.SHARED_GEN_ID, cfg.hidden, cfg.inter,
                         cfg.bits_shared, synth.dist_for_bits(cfg.bits_shared))
        layers.append(moe.Layer(hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts,
                                top_k=cfg.top_k, bits_routed=cfg.bits_routed,
                                bits_shared=cfg.bits_shared, renorm=True,
                                router=upload_router(case.routers[l], cfg.router_dtype),
                                gate_vec=upload_router(case.gates[l], cfg.gate_dtype),
                                experts=pool, expert_stride=rb, shared_expert=shared))
    stack = moe.Stack(layers)
    updates = to_dev(case.updates.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    return stack, updates, layers


def _check(case, h, idx_log, w_log):
    K = case.cfg.top_k
    for l in range(case.n_layers):
        g = [int(e) for e in idx_log[l]]
        r = [int(e) for e in case.idx[l]]
        assert sorted(g) == sorted(r), (l, g, r)
        w_by = np.array([w_log[l][g.index(e)] for e in r])
        assert err_metric(w_by, case.w[l]) <= TOL, (l, w_by, case.w[l])
    e = err_metric(h, case.h)
    assert e <= TOL, e
    return e


def _run(cfg, seed, n_layers=None, graph_replays=0, rows_too=False):
    from bit_dequant_expert_route_amd import moe
    case = make_stack_case(cfg, seed, n_layers)
    log(f"stack {cfg.name} seed {seed}: {case.n_layers} layers, update redraws {sum(case.attempts)}")
    stack, updates, layers = _build(cfg, case)
    ws = stack.workspace()
    K, L = cfg.top_k, case.n_layers
    h = to_dev(case.h0)
    idx_log = torch.empty(L, K, dtype=torch.int32, device="cuda")
    w_log = torch.empty(L, K, dtype=torch.float32, device="cuda")
    moe.stack_decode(stack, updates, h, idx_log, w_log, ws)
    torch.cuda.synchronize()
    eager = h.cpu().numpy()
    err = _check(case, eager, idx_log.cpu().numpy(), w_log.cpu().numpy())
    log(f"  eager: err(h) {err:.2e}")
    if rows_too:  # the same stack reading the router rows instead of its tiles
        rows = moe.Stack(layers, router_tiles=False)
        h_rows = to_dev(case.h0)
        moe.stack_decode(rows, updates, h_rows, idx_log, w_log, ws)
        torch.cuda.synchronize()
        assert np.array_equal(h_rows.cpu().numpy(), eager), "router rows and tiles differ"
        log("  router rows give the tiles' output bit for bit")
    if graph_replays:
        s = torch.cuda.Stream()
        h0 = to_dev(case.h0)
        with torch.cuda.stream(s):
            g = moe.graph_stack(stack, updates, h, idx_log, w_log, ws, s)
        for r in range(graph_replays):
            h.copy_(h0)
            idx_log.zero_()
            torch.cuda.synchronize()
            g.launch(s)
            torch.cuda.synchronize()
            got = h.cpu().numpy()
            assert np.array_equal(got, eager), f"replay {r} differs from the eager run"
            _check(case, got, idx_log.cpu().numpy(), w_log.cpu().numpy())
        g.destroy()
        log(f"  {graph_replays} graph replays equal the eager run bit for bit")
    return err


@pytest.mark.parametrize("seed", [3, 11])
def test_tiny_stack(seed):
    _run(synth.CONFIGS["tiny_stack"], seed, graph_replays=3 if seed == 3 else 0, rows_too=True)


@pytest.mark.parametrize("seed", [3, 23])
def test_q4_stack_60_layers(seed):
    """The 60-layer, 217 GB resident stack at its full size (one token)."""
    cfg = synth.CONFIGS["q4_stack"]
    import gc
    gc.collect()
    torch.cuda.empty_cache()  # the previous seed's 217 GB go back to the device
    free, total = torch.cuda.mem_get_info()
    need = cfg.n_layers * (cfg.n_experts * cfg.record_bytes + cfg.shared_record_bytes) + (4 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} GiB free")
    _run(cfg, seed, graph_replays=1 if seed == 3 else 0, rows_too=seed == 3)


STACK_EDGE = {
    # 2-bit experts throughout; a 2-bit layer with a 4-bit shared expert (the
    # shared gate/up runs in the router kernel, its down in its own launch);
    # rows that do not fill a wave
    "q2": synth.LayerConfig("stack_q2", 256, 128, 16, 2, 2, 2, "bf16", "bf16", "f32", n_layers=6),
    "mixed": synth.LayerConfig("stack_mixed", 256, 128, 16, 2, 2, 4, "f32", "f32", "f32", n_layers=6),
    "ragged": synth.LayerConfig("stack_ragged", 192, 320, 16, 2, 4, 4, "bf16", "bf16", "f32", n_layers=6),
}


@pytest.mark.parametrize("name", list(STACK_EDGE))
def test_stack_edges(name):
    _run(STACK_EDGE[name], 13, graph_replays=1, rows_too=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_router_tile_layout(dtype):
    """moe_router_tile: tile t, expert e holds columns 8t..8t+7 of row e."""
    from bit_dequant_expert_route_amd import moe
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    E, H = 48, 192
    r = torch.randn(E, H, generator=g, device="cuda").to(dtype)
    t = moe.router_tile(r)
    torch.cuda.synchronize()
    want = r.cpu().reshape(E, H // 8, 8).permute(1, 0, 2).contiguous()
    assert torch.equal(t.cpu(), want)
