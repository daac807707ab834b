"""moe_layer_decode_noalloc (the library's own scratch array as the workspace)
against moe_layer_decode with a caller workspace, through the C ABI: the same
kernels on the same inputs, so the outputs must agree bit for bit.  Two calls
in a row on one GPU, the second with fewer tokens than the first, so that the
second runs on what the first left in the scratch array."""
import numpy as np
import pytest
import torch

from bit_dequant_expert_route_amd import synth
from gpu_util import expert_pool, log, to_dev, upload_router

pytestmark = pytest.mark.gpu


def _layer(cfg, seed):
    from bit_dequant_expert_route_amd import moe
    pool, rb = expert_pool(cfg, seed)
    sb = synth.record_layout(cfg.hidden, cfg.inter, cfg.bits_shared).total
    shared = torch.empty(sb, dtype=torch.uint8, device="cuda")
    moe.fill_experts(shared, sb, 1, seed, 0, synth.SHARED_GEN_ID, cfg.hidden, cfg.inter,
                     cfg.bits_shared, synth.dist_for_bits(cfg.bits_shared))
    return moe.Layer(hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts,
                     top_k=cfg.top_k, bits_routed=cfg.bits_routed, bits_shared=cfg.bits_shared,
                     renorm=True, router=upload_router(synth.router_weights(cfg, seed), cfg.router_dtype),
                     gate_vec=upload_router(synth.shared_gate_vector(cfg, seed), cfg.gate_dtype),
                     experts=pool, expert_stride=rb, shared_expert=shared)


def _inputs(cfg, T, seed):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, cfg.hidden)).astype(np.float32)
    x = h / np.sqrt(np.mean(h.astype(np.float64) ** 2, axis=1, keepdims=True) + 1e-6)
    xb = synth.f64_to_bf16_rne(x.astype(np.float64))
    return to_dev(xb.astype(np.uint16).view(np.int16)).view(torch.bfloat16), to_dev(h)


def _call(layer, x, h_res, noalloc):
    from bit_dequant_expert_route_amd import moe
    T, K = x.shape[0], layer.top_k
    out = torch.full_like(h_res, float("nan"))
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, K), float("nan"), device="cuda")
    if noalloc:
        moe.layer_decode_noalloc(layer, x, h_res, out, idx, w)
    else:
        moe.layer_decode(layer, x, h_res, out, idx, w, layer.workspace(T))
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def test_noalloc_equals_workspace_entry_point():
    cfg = synth.CONFIGS["q4_layer"]
    layer = _layer(cfg, 7)
    for T in (16, 1):  # the second call is smaller than the first
        log(f"q4 layer, {T} token(s): moe_layer_decode_noalloc vs moe_layer_decode")
        x, h_res = _inputs(cfg, T, 100 + T)
        got = _call(layer, x, h_res, True)
        want = _call(layer, x, h_res, False)
        assert np.array_equal(got[1], want[1]), (got[1], want[1])
        assert np.array_equal(got[2], want[2])
        assert np.array_equal(got[0], want[0])
        assert np.all(np.isfinite(got[0]))
