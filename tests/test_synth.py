"""The seeded input generator: published SplitMix64 outputs, bf16 rounding,
distributions and the record layout."""
from fractions import Fraction

import numpy as np
import pytest

from bit_dequant_expert_route_amd import synth


def test_splitmix64_known_answer():
    # first outputs of SplitMix64 from state 1234567, as published with the
    # reference implementation of the generator (Vigna, prng.di.unimi.it)
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [synth.sm(1234567, i) for i in range(5)] == want
    assert list(synth.sm_stream(1234567, 5)) == want
    assert list(synth.sm_stream(1234567, 3, start=2)) == want[2:]


def _nearest_bf16_exact(v: float) -> int:
    """Brute force: scan the bf16 neighbours of v with exact rationals."""
    b0 = (np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16)
    cands = []
    for b in range(max(int(b0) - 2, 0), int(b0) + 3):
        val = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        if not np.isfinite(val):
            continue
        cands.append((abs(Fraction(float(val)) - Fraction(v)), b & 1, b))
    cands.sort()
    best = cands[0]
    ties = [c for c in cands if c[0] == best[0]]
    return min(ties, key=lambda c: c[1])[2]  # even mantissa wins a tie


def test_bf16_rne_against_brute_force():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(300) * 0.02, rng.uniform(-0.08, 0.04, 300),
                        rng.standard_normal(100) * 1e5])
    got = synth.f64_to_bf16_rne(v)
    for x, g in zip(v, got):
        assert int(g) == _nearest_bf16_exact(float(x)), x


def test_bf16_rne_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert synth.f64_to_bf16_rne(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
    assert synth.f64_to_bf16_rne(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82
    assert synth.f64_to_bf16_rne(np.array([-0.0, 0.0]))[0] == 0x8000


def test_codes_are_uniform_and_deterministic():
    k = synth.section_key(1, 0, 7, synth.SEC_GATE_CODES)
    w = synth.gen_codes(k, 1 << 16)
    assert np.array_equal(w, synth.gen_codes(k, 1 << 16))
    nib = np.concatenate([(w >> np.uint32(4 * i)) & np.uint32(15) for i in range(8)])
    counts = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(counts - 1 / 16) < 0.002)
    assert synth.gen_codes(k, 5)[4] == w[4]  # prefix property
    k2 = synth.section_key(1, 0, 8, synth.SEC_GATE_CODES)
    assert not np.array_equal(synth.gen_codes(k2, 64), w[:64])


@pytest.mark.parametrize("dist", [synth.Q4_DIST, synth.Q2_DIST])
def test_scale_bias_ranges(dist):
    sb = synth.gen_sb(synth.section_key(2, 3, 4, synth.SEC_DOWN_SB), 20000, dist)
    s = synth.bf16_to_f32((sb & np.uint32(0xFFFF)).astype(np.uint16))
    b = synth.bf16_to_f32((sb >> np.uint32(16)).astype(np.uint16))
    tol = 2.0 ** -8
    assert s.min() >= dist.scale_lo * (1 - tol) and s.max() <= dist.scale_hi * (1 + tol)
    assert b.min() >= dist.bias_lo * (1 + tol) and b.max() <= 0.0
    mid_s = (dist.scale_lo + dist.scale_hi) / 2
    assert abs(s.mean() - mid_s) < 0.01 * mid_s


def test_record_layout_matches_oracle(orc):
    for H, I, bits in ((4096, 1024, 4), (4096, 1024, 2), (256, 128, 4), (192, 320, 2)):
        lay = synth.record_layout(H, I, bits)
        assert lay.total == orc.record_bytes(H, I, bits)
        assert lay.total % 256 == 0
    assert synth.CONFIGS["q4_layer"].record_bytes == 7077888
    assert synth.CONFIGS["q2_layer"].record_bytes == 3932160
    assert synth.CONFIGS["tiny"].record_bytes == 55296
    assert synth.CONFIGS["q4_layer"].weight_bytes_per_token_layer() == 39591936
    assert synth.CONFIGS["q2_layer"].weight_bytes_per_token_layer() == 23863296
    assert synth.CONFIGS["tiny"].weight_bytes_per_token_layer() == 16 * 256 * 4 + 256 * 4 + 3 * 55296


def test_make_record_sections():
    rec = synth.make_record(5, 2, 9, 256, 128, 4)
    lay = synth.record_layout(256, 128, 4)
    gate = rec[lay.gate_codes:lay.gate_codes + 128 * 128].view(np.uint32)
    assert np.array_equal(gate, synth.gen_codes(synth.section_key(5, 2, 9, 0), 128 * 32))
    assert np.array_equal(rec, synth.make_record(5, 2, 9, 256, 128, 4))
