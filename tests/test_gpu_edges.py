"""Edge cases of the layer path against the oracle: the smallest and largest
top-K (K = 1, K = E = 8), the largest expert count (E = 1024: the selection's
second register width), rows that do not fill a wave's lanes (H, I multiples
of 64 but not of 128, also for 2-bit bf16 x staged by lane pairs), the widest rows (H = 8192: four chunks per lane, also
with fp32 x staged in LDS), fp32 activations with bf16 weights, the 64-token
maximum, and run-to-run determinism."""
import dataclasses

import numpy as np
import pytest
import torch

from bit_dequant_expert_route_amd import synth
from cases import TOL, err_metric, make_batch_case, make_layer_case
from gpu_util import expert_pool, log, make_layer
from test_gpu_batch import _check as check_batch
from test_gpu_batch import _run as run_batch
from test_gpu_layer import _run_layer, check_layer

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
EDGE = {
    "k1": C("edge_k1", 256, 128, 16, 1, 4, 4, "bf16", "bf16", "bf16"),
    "e_eq_k": C("edge_e8k8", 256, 128, 8, 8, 4, 4, "bf16", "bf16", "bf16"),
    "e1024": C("edge_e1024", 128, 64, 1024, 4, 4, 4, "bf16", "bf16", "bf16"),
    "e600_k8": C("edge_e600k8", 128, 64, 600, 8, 2, 2, "f32", "f32", "f32"),
    "ragged4": C("edge_ragged4", 192, 320, 16, 2, 4, 4, "bf16", "bf16", "bf16"),
    "ragged2": C("edge_ragged2", 192, 320, 16, 2, 2, 2, "f32", "bf16", "f32"),
    # 2-bit rows of bf16 x with an odd count of 64-column chunks (3): the
    # lane pairs that stage the chunks' halves end inside a wave
    "ragged2b": C("edge_ragged2b", 192, 320, 16, 2, 2, 2, "bf16", "bf16", "bf16"),
    "wide4": C("edge_wide4", 8192, 64, 16, 2, 4, 4, "bf16", "bf16", "bf16"),
    "wide2": C("edge_wide2", 8192, 128, 16, 2, 2, 2, "bf16", "bf16", "bf16"),
    # fp32 x at the widest rows: x staged per workgroup fills the most LDS
    # (36 KB at 4 bits, 34 KB at 2 bits) and every thread holds eight float4
    "wide4f": C("edge_wide4f", 8192, 64, 16, 2, 4, 4, "bf16", "bf16", "f32"),
    "wide2f": C("edge_wide2f", 8192, 128, 16, 2, 2, 2, "bf16", "bf16", "f32"),
    "tall": C("edge_tall", 64, 8192, 16, 2, 4, 2, "f32", "f32", "f32"),
}


@pytest.mark.parametrize("name", list(EDGE))
@pytest.mark.parametrize("renorm", [True, False])
def test_edge_layer(name, renorm):
    cfg = EDGE[name]
    for seed in (21, 22):
        log(f"edge {name} renorm={renorm} seed={seed}")
        case = make_layer_case(cfg, seed, renorm)
        pool, stride = expert_pool(cfg, seed)
        layer = make_layer(cfg, case, pool, stride)
        errs = check_layer(case, _run_layer(cfg, case, layer))
        log(f"  errors {errs}")


def test_64_tokens():
    cfg = dataclasses.replace(synth.CONFIGS["tiny_batch"], name="tiny_batch64", n_tokens=64)
    case = make_batch_case(cfg, 6)
    err = check_batch(case, *run_batch(cfg, case))
    log(f"64 tokens: worst err(out) {err:.2e}")


def test_deterministic():
    """Two calls on the same inputs give the same bits (no atomics, fixed
    reduction order)."""
    from bit_dequant_expert_route_amd import moe
    cfg = synth.CONFIGS["q4_layer"]
    case = make_layer_case(cfg, 1, True)
    pool, stride = expert_pool(cfg, 1)
    layer = make_layer(cfg, case, pool, stride)
    a = _run_layer(cfg, case, layer)
    b = _run_layer(cfg, case, layer)
    for k in ("out", "idx", "w", "h_routed", "h_shared", "logits"):
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k
    assert a["sigma"] == b["sigma"]
