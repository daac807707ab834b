"""Multi-token layer calls at the shapes the grouped kernels specialise on,
against the oracle per token: 2-bit experts, a 2-bit layer with a 4-bit shared
expert and fp32 activations (the shared expert's own grouped launches), rows
that do not fill a wave (H, I multiples of 64 but not of 128), the largest K,
the largest expert count, the widest rows (four code chunks per lane), and
batches of more than 128 (token, expert) pairs, which take the separate
grouping launch."""
import pytest

from bit_dequant_expert_route_amd import synth
from cases import make_batch_case
from gpu_util import log
from test_gpu_batch import _check, _run

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
EDGE = {
    "q2": (C("batch_q2", 256, 128, 16, 2, 2, 2, "bf16", "bf16", "bf16", n_tokens=9), 6),
    "mixed": (C("batch_mixed", 256, 128, 16, 2, 2, 4, "f32", "f32", "f32", n_tokens=5), 5),
    "ragged": (C("batch_ragged", 192, 320, 16, 2, 4, 4, "bf16", "bf16", "bf16", n_tokens=6), 6),
    "k8": (C("batch_k8", 128, 64, 64, 8, 4, 4, "bf16", "bf16", "bf16", n_tokens=12), 30),
    "e1024": (C("batch_e1024", 128, 64, 1024, 4, 4, 4, "bf16", "bf16", "bf16", n_tokens=5), 12),
    "wide4": (C("batch_wide4", 8192, 64, 16, 2, 4, 4, "bf16", "bf16", "bf16", n_tokens=3), 4),
    "wide2": (C("batch_wide2", 8192, 128, 16, 2, 2, 2, "bf16", "bf16", "bf16", n_tokens=3), 4),
    # more than 128 (token, expert) pairs: the separate grouping launch
    # (up to 128 the gate/up kernel groups the pairs itself)
    "pairs256": (C("batch_pairs256", 128, 64, 64, 8, 4, 4, "bf16", "bf16", "bf16", n_tokens=32), 40),
    "pairs129": (C("batch_pairs129", 128, 64, 64, 3, 4, 4, "bf16", "bf16", "bf16", n_tokens=43), 40),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_batch_edge(name):
    cfg, target = EDGE[name]
    case = make_batch_case(cfg, 71, target_distinct=target)
    log(f"batch edge {name}: {cfg.n_tokens} tokens, {case.distinct} distinct experts")
    err = _check(case, *_run(cfg, case))
    log(f"  worst err(out) {err:.2e}")
