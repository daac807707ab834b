"""Helpers of the GPU tests: put a test case on the device and run the HIP path
through the C ABI binding."""
from __future__ import annotations

import sys

import numpy as np
import torch

from bit_dequant_expert_route_amd import synth


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


def upload_router(case_or_arr, dtype: str):
    a = case_or_arr
    if dtype == "bf16":
        return to_dev(a.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    return to_dev(a.astype(np.float32))


def expert_pool(cfg: synth.LayerConfig, seed: int, layer: int = 0, host: bool = False,
                bits: int | None = None):
    """All E routed records of a layer on the device, stride = record size.
    host=True builds them with the host generator and uploads them; otherwise
    the device fill kernel writes them."""
    from bit_dequant_expert_route_amd import moe
    bits = bits or cfg.bits_routed
    rb = synth.record_layout(cfg.hidden, cfg.inter, bits).total
    if host:
        recs = np.concatenate([synth.make_record(seed, layer, e, cfg.hidden, cfg.inter, bits)
                               for e in range(cfg.n_experts)])
        return to_dev(recs), rb
    pool = torch.empty(cfg.n_experts * rb, dtype=torch.uint8, device="cuda")
    moe.fill_experts(pool, rb, cfg.n_experts, seed, layer, 0, cfg.hidden, cfg.inter, bits,
                     synth.dist_for_bits(bits))
    return pool, rb


def make_layer(cfg, case, pool, stride, shared_dev=None, bits_shared=None):
    from bit_dequant_expert_route_amd import moe
    bits_shared = bits_shared or cfg.bits_shared
    if shared_dev is None:
        shared_dev = to_dev(case.shared)
    return moe.Layer(hidden=cfg.hidden, inter=cfg.inter, n_experts=cfg.n_experts,
                     top_k=cfg.top_k, bits_routed=cfg.bits_routed, bits_shared=bits_shared,
                     renorm=case.renorm, router=upload_router(case.router, cfg.router_dtype),
                     gate_vec=upload_router(case.gate_vec, cfg.gate_dtype), experts=pool,
                     expert_stride=stride, shared_expert=shared_dev)


def x_dev(case):
    if case.cfg.x_dtype == "bf16" and case.x.dtype == np.uint16:
        return to_dev(case.x.view(np.int16)).view(torch.bfloat16)
    return to_dev(case.x.astype(np.float32))
