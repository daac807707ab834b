"""Plant plausible mistakes in copies of the oracle source (on the CPU) and
check that the pin set catches every one of them."""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle import build as obuild
import oracle_pins

# (name, text in moe_oracle.c, replacement)
MUTANTS = [
    ("drop_bias", "* scale + bias;", "* scale;"),
    ("swap_scale_bias", "(uint16_t)(p & 0xFFFFu)", "(uint16_t)(p >> 16)"),
    ("reverse_fields", "(w >> (bits * (c % per_word)))", "(w >> (bits * (per_word - 1 - c % per_word)))"),
    ("group_index", "(size_t)(c / ORACLE_GROUP)]", "(size_t)(c / 32) % (size_t)(cols / ORACLE_GROUP)]"),
    ("row_stride", "(size_t)(cols / (32 / bits))", "(size_t)(cols / 8)"),
    ("softmax_unnormalised", "for (int i = 0; i < n; ++i) p[i] /= z;", ""),
    ("topk_ties_high", "logits[i] > logits[best]", "logits[i] >= logits[best]"),
    ("topk_ascending", "logits[i] > logits[best]", "logits[i] < logits[best]"),
    ("ignore_renorm", "if (renorm)", "if (0)"),
    ("weights_by_position", "w[j] = p[idx[j]];", "w[j] = p[j];"),
    ("gate_sign", "return 1.0 / (1.0 + exp(-acc));", "return 1.0 / (1.0 + exp(acc));"),
    ("silu_on_up", "double sig = 1.0 / (1.0 + exp(-a[r]));", "double sig = 1.0 / (1.0 + exp(-u[r]));"),
    ("no_silu", "h[r] = a[r] * sig * u[r];", "h[r] = a[r] * u[r];"),
    ("down_reads_x", "hidden, inter, bits, h, y);", "hidden, inter, bits, x, y);"),
    ("combine_no_sigma", "acc += sigma * y_shared[o];", "acc += y_shared[o];"),
    ("combine_no_residual", "double acc = h_res[o];", "double acc = 0.0;"),
    ("combine_transposed", "acc += w[j] * y[(size_t)j * hidden + o];", "acc += w[j] * y[(size_t)o * k + j];"),
    ("rms_no_mean", "sqrt(ss / (double)n + eps)", "sqrt(ss + eps)"),
    ("router_transposed", "size_t i = (size_t)e * hidden + c;", "size_t i = (size_t)c * n_experts + e;"),
    ("shared_bits_routed", "oracle_expert(shared_record, hidden, inter, bits_shared, x,",
     "oracle_expert(shared_record, hidden, inter, bits_routed, x,"),
    # (with H and I multiples of 64 every section is already a multiple of 256
    # bytes, so the rounding itself is never exercised; the total is)
    ("record_total_short", "L.total = L.down_sb + up256(ds);", "L.total = L.down_sb;"),
    ("sb_section_swapped", "L.up_sb = L.gate_sb + up256(gs);", "L.up_sb = L.gate_sb;"),
    ("gdn_no_decay", "for (size_t i = 0; i < (size_t)d_v * d_k; ++i) S[i] *= a;", ""),
    ("gdn_delta_sign", "const double c = b * (vh[i] - u);", "const double c = b * (u - vh[i]);"),
    ("gdn_no_delta", "const double c = b * (vh[i] - u);", "const double c = b * vh[i];"),
    ("gdn_key_for_query", "for (int j = 0; j < d_k; ++j) o += row[j] * qh[j];",
     "for (int j = 0; j < d_k; ++j) o += row[j] * kh[j];"),
    ("gdn_transposed_gemv", "for (int j = 0; j < d_k; ++j) u += row[j] * kh[j];",
     "for (int j = 0; j < d_k && j < d_v; ++j) u += S[(size_t)j * d_k + i] * kh[j];"),
    ("gdn_block_no_qnorm", "q[(size_t)hd * d_head + j] = qh[j] * rq;", "q[(size_t)hd * d_head + j] = qh[j];"),
    ("gdn_block_no_knorm", "k[(size_t)hd * d_head + j] = kh[j] * rk;", "k[(size_t)hd * d_head + j] = kh[j];"),
    ("gdn_block_gates_swapped", "alpha[hd] = 1.0 / (1.0 + exp(-proj[3 * D + hd]));",
     "alpha[hd] = 1.0 / (1.0 + exp(-proj[3 * D + n_heads + hd]));"),
    ("gdn_block_no_residual", "h_out[i] = h[i] + y[i];", "h_out[i] = y[i];"),
    ("gdn_block_unnormalised_x", "oracle_rmsnorm(h, hidden, 1e-6, x);",
     "memcpy(x, h, sizeof(double) * (size_t)hidden);"),
    ("gdn_block_v_from_k", "proj + 2 * D, alpha, beta, state, o);", "proj + D, alpha, beta, state, o);"),
    ("gdn_block_out_reads_q", "hidden, D, bits, o, y);", "hidden, D, bits, q, y);"),
]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutated = src.replace(old, new, 1)
    path = os.path.join(workdir, f"{name}.c")
    open(path, "w").write(mutated)
    lib = obuild.compile_oracle(path, os.path.join(workdir, f"lib_{name}.so"), extra=["-w"])
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(exc).__name__))
    assert failed, f"mutant {name} passed every pin"
