"""The host-memory expert tier on the device: a stream of tokens through one
layer whose routed records live in page-locked host memory behind a small
device cache managed on the device.  Every output must equal the resident
path's bit for bit (same kernels, the slot's or the host record in place of
the resident one), the first token is also checked against the fp64 oracle,
and after every token the device's slot table and its hit/miss/byte counts
must follow the least-recently-used model.  A captured graph of a token
stream must replay to the same outputs and slot table as the eager calls."""
import numpy as np
import pytest
import torch

from bit_dequant_expert_route_amd import synth
from cases import make_layer_case
from gpu_util import expert_pool, log, make_layer, x_dev
from test_gpu_layer import check_layer
from test_tier import LRUModel

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
CFGS = {
    "tiny": synth.CONFIGS["tiny"],
    "mixed": C("tier_mixed", 256, 128, 16, 2, 2, 4, "f32", "f32", "f32"),
    "q4_e64": C("tier_q4_e64", 4096, 1024, 64, 4, 4, 4, "bf16", "bf16", "bf16"),
}


def _outputs(layer, x, h_res, run):
    K = layer.s.top_k
    out = torch.empty_like(h_res)
    idx = torch.empty(K, dtype=torch.int32, device="cuda")
    w = torch.empty(K, dtype=torch.float32, device="cuda")
    ws = layer.workspace(1)
    run(layer, x, h_res, out, idx, w, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), ws


def _setup(name, seed, n_slots, n_tokens):
    from bit_dequant_expert_route_amd import moe
    cfg = CFGS[name]
    bs = cfg.bits_shared
    case = make_layer_case(cfg, seed, True, bits_shared=bs)
    pool, stride = expert_pool(cfg, seed)
    layer = make_layer(cfg, case, pool, stride, bits_shared=bs)
    host = pool.cpu().pin_memory()
    cache = torch.empty(n_slots * stride, dtype=torch.uint8, device="cuda")
    tier = moe.Tier(host, cfg.n_experts, stride, cache, n_slots)
    # tokens: the case's own x first, then those of other draws over the same layer
    xs = [(x_dev(case), torch.from_numpy(case.h_res).cuda())]
    for j in range(1, n_tokens):
        c = make_layer_case(cfg, seed + 1000 * j, True, bits_shared=bs)
        xs.append((x_dev(c), torch.from_numpy(c.h_res).cuda()))
    return cfg, case, pool, layer, host, cache, tier, xs


@pytest.mark.parametrize("name,n_slots,n_tokens", [("tiny", 8, 24), ("mixed", 8, 12), ("q4_e64", 16, 12)])
def test_tier_stream_matches_resident(name, n_slots, n_tokens):
    from bit_dequant_expert_route_amd import moe
    cfg, case, pool, layer, host, cache, tier, xs = _setup(name, 61, n_slots, n_tokens)
    model = LRUModel(n_slots)
    rb = synth.record_layout(cfg.hidden, cfg.inter, cfg.bits_routed).total
    want_miss = 0
    for i, (x, h_res) in enumerate(xs):
        log(f"tier {name} token {i}")
        ro, ri, rw, _ = _outputs(layer, x, h_res, moe.layer_decode)
        to, ti, tw, ws = _outputs(layer, x, h_res, tier.layer_decode)
        assert np.array_equal(ri, ti), (i, ri, ti)
        assert np.array_equal(rw, tw), i
        assert np.array_equal(ro, to), i
        want_miss += sum(model.assign([int(e) for e in ti])[1])
        assert tier.slots() == model.owner, (i, tier.slots(), model.owner)
        if i == 0:
            view = moe.ws_view(layer, 1, ws)
            check_layer(case, dict(out=to, idx=ti, w=tw, logits=view["logits"][0].cpu().numpy(),
                                   sigma=float(view["sigma"][0]), h_routed=view["h_routed"][0].cpu().numpy(),
                                   h_shared=view["h_shared"][0].cpu().numpy()))
    hits, misses, read = tier.stats()
    K = cfg.top_k
    assert (hits, misses) == (n_tokens * K - want_miss, want_miss)
    assert read == misses * rb
    # every cached slot now holds its expert's record, byte for byte
    own = tier.slots()
    got = cache.cpu().numpy()
    pool_h = host.numpy()
    for s_, e in enumerate(own):
        if e >= 0:
            assert np.array_equal(got[s_ * pool.numel() // cfg.n_experts:][:rb],
                                  pool_h[e * (pool.numel() // cfg.n_experts):][:rb]), (s_, e)
    log(f"tier {name}: {hits} hits, {misses} misses over {n_tokens} tokens")
    tier.close()


def test_tier_graph_replay_equals_eager():
    """The tier path has no host round trip: a graph captured over a token
    stream replays to the eager outputs and slot table."""
    from bit_dequant_expert_route_amd import moe
    cfg, case, pool, layer, host, cache, tier, xs = _setup("tiny", 62, 8, 10)
    K = cfg.top_k
    outs = [torch.empty(cfg.hidden, device="cuda") for _ in xs]
    idxs = [torch.empty(K, dtype=torch.int32, device="cuda") for _ in xs]
    ws_ = [torch.empty(K, device="cuda") for _ in xs]
    wsp = layer.workspace(1)

    def run(stream=None):
        for i, (x, h_res) in enumerate(xs):
            tier.layer_decode(layer, x, h_res, outs[i], idxs[i], ws_[i], wsp, stream=stream)

    run()
    torch.cuda.synchronize()
    eager = [(o.cpu().numpy(), i.cpu().numpy()) for o, i in zip(outs, idxs)]
    slots_eager, stats_eager = tier.slots(), tier.stats()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        moe.capture_begin(s)
        run(stream=s)
        g = moe.capture_end(s, keep=(xs, outs, idxs, ws_, wsp))
    for rep in range(2):
        tier.reset()
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.launch(s)
        torch.cuda.synchronize()
        for i, (o, ix) in enumerate(zip(outs, idxs)):
            assert np.array_equal(o.cpu().numpy(), eager[i][0]), (rep, i)
            assert np.array_equal(ix.cpu().numpy(), eager[i][1]), (rep, i)
        assert tier.slots() == slots_eager and tier.stats() == stats_eager
    g.destroy()
    tier.close()
