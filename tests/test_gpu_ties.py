"""Exact ties in the routing, on the GPU against the fp64 oracle.  The
gate/up kernel splits the selection over four waves, each taking a quarter of
the experts, and merges their candidates; equal logits must still go to the
lower expert index, as in one stable sort.  A router row copied onto another
expert gives two bitwise-equal logits (the same row, the same x, the same
reduction on both sides); the copy is placed in another quarter than the
original, at the K-th rank (only one of the two is selected) and at the first
rank (both are)."""
import numpy as np
import pytest
import torch

from bit_dequant_expert_route_amd import synth
from cases import make_layer_case
from gpu_util import expert_pool, log, make_layer
from test_gpu_layer import _run_layer, check_layer

pytestmark = pytest.mark.gpu

# 512 experts: four quarters of 128 in the split selection
CFG = synth.LayerConfig("ties", 256, 128, 512, 4, 4, 4, "bf16", "bf16", "bf16")
QUARTER = 128


def _tie(rank, partner_lower):
    """Copy the router row of the expert at `rank` (0 = largest logit) onto a
    lower-ranked expert of another quarter, below or above it in index."""
    def edit(router, logits):
        order = np.argsort(-logits, kind="stable")
        e = int(order[rank])
        q = e // QUARTER
        for cand in order[CFG.top_k + 4:]:
            c = int(cand)
            if c // QUARTER != q and (c < e) == partner_lower:
                r = router.copy()
                r[c] = router[e]
                log(f"tie: expert {c} copies expert {e} (rank {rank})")
                return r
        raise LookupError("no partner expert in another quarter")
    return edit


@pytest.mark.parametrize("rank", [0, CFG.top_k - 1])
@pytest.mark.parametrize("partner_lower", [True, False])
@pytest.mark.parametrize("renorm", [True, False])
def test_exact_tie(rank, partner_lower, renorm):
    done = 0
    for seed in range(31, 61):
        if done == 2:
            break
        try:
            case = make_layer_case(CFG, seed, renorm, router_edit=_tie(rank, partner_lower))
        except LookupError:  # (the expert sits in the last or first quarter)
            continue
        done += 1
        pool, stride = expert_pool(CFG, seed)
        layer = make_layer(CFG, case, pool, stride)
        got = _run_layer(CFG, case, layer)
        # the oracle's logits of the pair are equal, and so are the GPU's
        errs = check_layer(case, got)
        log(f"rank={rank} lower={partner_lower} renorm={renorm} seed={seed}: {errs}")
        del pool, layer
        torch.cuda.empty_cache()
    assert done == 2
