"""GPU parity of a multi-token layer call against the oracle run per token.
Each token's experts must match as a set, its weights per index, and its
output meet err_metric <= 2e-3.  The full-size case is a 16-token batch whose
tokens are correlated so that about 40 distinct routed experts are touched."""
import numpy as np
import pytest
import torch

from bit_dequant_expert_route_amd import synth
from cases import TOL, err_metric, make_batch_case
from gpu_util import expert_pool, log, to_dev, upload_router

pytestmark = pytest.mark.gpu


def _run(cfg, case):
    from bit_dequant_expert_route_amd import moe
    pool, rb = expert_pool(cfg, case.seed)
    sb = synth.record_layout(cfg.hidden, cfg.inter, cfg.bits_shared).total
    shared = torch.empty(sb, dtype=torch.uint8, device="cuda")
    moe.fill_experts(shared, sb, 1, case.seed, 0, synth.SHARED_GEN_ID, cfg.hidden, cfg.inter,
                     cfg.bits_shared, synth.dist_for_bits(cfg.bits_shared))
    layer = moe.Layer(hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts,
                      top_k=cfg.top_k, bits_routed=cfg.bits_routed, bits_shared=cfg.bits_shared,
                      renorm=True, router=upload_router(case.router, cfg.router_dtype),
                      gate_vec=upload_router(case.gate_vec, cfg.gate_dtype), experts=pool,
                      expert_stride=rb, shared_expert=shared)
    T, K = cfg.n_tokens, cfg.top_k
    if cfg.x_dtype == "bf16":
        x = to_dev(case.x.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    else:
        x = to_dev(case.x.astype(np.float32))
    h_res = to_dev(case.h_res)
    out = torch.empty_like(h_res)
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    ws = layer.workspace(T)
    moe.layer_decode(layer, x, h_res, out, idx, w, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _check(case, out, idx, w):
    worst = 0.0
    for t in range(case.cfg.n_tokens):
        g = [int(e) for e in idx[t]]
        r = [int(e) for e in case.idx[t]]
        assert sorted(g) == sorted(r), (t, g, r)
        w_by = np.array([w[t][g.index(e)] for e in r])
        assert err_metric(w_by, case.w[t]) <= TOL, (t, w_by, case.w[t])
        e = err_metric(out[t], case.out[t])
        assert e <= TOL, (t, e)
        worst = max(worst, e)
    return worst


@pytest.mark.parametrize("seed", [4, 5])
def test_tiny_batch(seed):
    cfg = synth.CONFIGS["tiny_batch"]
    case = make_batch_case(cfg, seed, target_distinct=8)
    log(f"tiny batch seed {seed}: rho {case.rho:.2f}, {case.distinct} distinct experts")
    err = _check(case, *_run(cfg, case))
    log(f"  worst err(out) {err:.2e}")


@pytest.mark.parametrize("seed", [4, 5, 6, 7])
def test_q4_batch16(seed):
    cfg = synth.CONFIGS["q4_batch16"]
    case = make_batch_case(cfg, seed, target_distinct=40)
    log(f"q4 batch of 16, seed {seed}: rho {case.rho:.2f}, {case.distinct} distinct routed experts")
    err = _check(case, *_run(cfg, case))
    log(f"  worst err(out) {err:.2e}")
