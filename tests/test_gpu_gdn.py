"""GPU parity of the gated delta-rule decode step (the linear-attention
layers' state update) against the fp64 oracle, through the C ABI: one step at
the pages' size (64 heads of 128x128), ragged and small shapes, several
sequences, and 16 consecutive steps carrying the state."""
import numpy as np
import pytest
import torch

import oracle
from bit_dequant_expert_route_amd import synth
from cases import TOL, err_metric
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def _gpu_steps(inputs_per_step, state0):
    from bit_dequant_expert_route_amd import moe
    S = to_dev(state0)
    outs = []
    for q, k, v, a, b in inputs_per_step:
        out = torch.empty(q.shape[:2] + (state0.shape[2],), device="cuda")
        moe.gdn_step(to_dev(q), to_dev(k), to_dev(v), to_dev(a), to_dev(b), S, out)
        outs.append(out)
    torch.cuda.synchronize()
    return S.cpu().numpy(), [o.cpu().numpy() for o in outs]


@pytest.mark.parametrize("n_seq,n_heads,d_k,d_v", [
    (1, 64, 128, 128),   # the pages' layer
    (3, 5, 128, 100),    # ragged rows, several sequences
    (2, 4, 16, 7),
    (1, 3, 64, 33),
    (1, 2, 256, 130),
])
def test_gdn_step(n_seq, n_heads, d_k, d_v):
    orc = oracle.get()
    q, k, v, a, b, S0 = synth.gdn_inputs(31, n_seq, n_heads, d_k, d_v)
    S, outs = _gpu_steps([(q, k, v, a, b)], S0)
    Sw, ow = orc.gdn_step(q, k, v, a, b, S0)
    es, eo = err_metric(S, Sw), err_metric(outs[0], ow)
    log(f"gdn {n_seq}x{n_heads} d_k={d_k} d_v={d_v}: err state {es:.2e} out {eo:.2e}")
    assert es <= TOL and eo <= TOL


def test_gdn_16_steps():
    """The state carried through 16 steps stays within the bound."""
    orc = oracle.get()
    n_seq, n_heads, d_k, d_v = 1, 64, 128, 128
    steps = [synth.gdn_inputs(32, n_seq, n_heads, d_k, d_v, step=t) for t in range(16)]
    S0 = steps[0][5]
    S, outs = _gpu_steps([s[:5] for s in steps], S0)
    Sw = S0.astype(np.float64)
    worst = 0.0
    for t, (q, k, v, a, b, _) in enumerate(steps):
        Sw, ow = orc.gdn_step(q, k, v, a, b, Sw)
        worst = max(worst, err_metric(outs[t], ow))
    es = err_metric(S, Sw)
    log(f"gdn 16 steps: err state {es:.2e}, worst out {worst:.2e}")
    assert es <= TOL and worst <= TOL
