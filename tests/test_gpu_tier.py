"""The host-memory expert tier on the device: a stream of tokens through one
layer whose routed records live in page-locked host memory behind a small
device cache.  Every output must equal the resident path's bit for bit (same
kernels, the cached record in place of the resident one), the first token is
also checked against the fp64 oracle, and the hit/miss counts and copied
bytes must follow the least-recently-used model."""
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


@pytest.mark.parametrize("name,n_slots,n_tokens", [("tiny", 8, 24), ("mixed", 8, 12), ("q4_e64", 16, 12)])
def test_tier_stream_matches_resident(name, n_slots, n_tokens):
    from bit_dequant_expert_route_amd import moe
    cfg = CFGS[name]
    seed = 61
    bs = cfg.bits_shared
    case = make_layer_case(cfg, seed, True, bits_shared=bs)
    pool, stride = expert_pool(cfg, seed)
    layer = make_layer(cfg, case, pool, stride, bits_shared=bs)
    host = pool.cpu().pin_memory()
    cache = torch.empty(n_slots * stride, dtype=torch.uint8, device="cuda")
    tier = moe.Tier(host, cfg.n_experts, stride, cache, n_slots)
    model = LRUModel(n_slots)
    rb = synth.record_layout(cfg.hidden, cfg.inter, cfg.bits_routed).total
    # tokens: the case's own x first, then those of other draws over the same layer
    xs = [(x_dev(case), torch.from_numpy(case.h_res).cuda())]
    for j in range(1, n_tokens):
        c = make_layer_case(cfg, seed + 1000 * j, True, bits_shared=bs)
        xs.append((x_dev(c), torch.from_numpy(c.h_res).cuda()))
    want_miss = 0
    for i, (x, h_res) in enumerate(xs):
        log(f"tier {name} token {i}")
        ro, ri, rw, _ = _outputs(layer, x, h_res, moe.layer_decode)
        to, ti, tw, ws = _outputs(layer, x, h_res, tier.layer_decode)
        assert np.array_equal(ri, ti), (i, ri, ti)
        assert np.array_equal(rw, tw), i
        assert np.array_equal(ro, to), i
        want_miss += sum(model.assign([int(e) for e in ti])[1])
        if i == 0:
            view = moe.ws_view(layer, 1, ws)
            check_layer(case, dict(out=to, idx=ti, w=tw, logits=view["logits"][0].cpu().numpy(),
                                   sigma=float(view["sigma"][0]), h_routed=view["h_routed"][0].cpu().numpy(),
                                   h_shared=view["h_shared"][0].cpu().numpy()))
    hits, misses, copied = tier.stats()
    K = cfg.top_k
    assert (hits, misses) == (n_tokens * K - want_miss, want_miss)
    assert copied == misses * rb
    log(f"tier {name}: {hits} hits, {misses} misses over {n_tokens} tokens")
    tier.close()


def test_tier_refuses_capture():
    from bit_dequant_expert_route_amd import moe
    cfg = CFGS["tiny"]
    case = make_layer_case(cfg, 62, True)
    pool, stride = expert_pool(cfg, 62)
    layer = make_layer(cfg, case, pool, stride)
    host = pool.cpu().pin_memory()
    cache = torch.empty(8 * stride, dtype=torch.uint8, device="cuda")
    tier = moe.Tier(host, cfg.n_experts, stride, cache, 8)
    x = x_dev(case)
    h_res = torch.from_numpy(case.h_res).cuda()
    out = torch.empty_like(h_res)
    idx = torch.empty(cfg.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.top_k, dtype=torch.float32, device="cuda")
    ws = layer.workspace(1)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    moe.capture_begin(s)
    with pytest.raises(moe.MoeError):
        tier.layer_decode(layer, x, h_res, out, idx, w, ws, stream=s)
    with torch.cuda.stream(s):
        out.fill_(0.0)  # the graph is not empty
    g = moe.capture_end(s, keep=(out,))
    g.destroy()
    tier.close()
