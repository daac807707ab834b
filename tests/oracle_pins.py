"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each `pin_*` takes an `oracle.Oracle` and raises AssertionError when the oracle
disagrees with: a number printed on the pages (tests/golden/page_facts.json),
a closed form, an exact rational computation, a special case that reduces to a
library routine (numpy / scipy), or brute force on a tiny input.  The same set
is run against deliberately broken copies of the oracle (test_oracle_mutants)
to show that each plausible mistake is caught by at least one pin.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import scipy.special

from bit_dequant_expert_route_amd import synth
from oracle import dense

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# small helpers (test-local; none of them is shared with the oracle or the
# HIP library)
# ----------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack [rows][cols] codes: column c goes to word c*b/32 at bit b*(c mod 32/b)."""
    rows, cols = codes.shape
    per = 32 // bits
    words = np.zeros((rows, cols // per), dtype=np.uint64)
    for c in range(cols):
        words[:, c // per] |= codes[:, c].astype(np.uint64) << np.uint64(bits * (c % per))
    return words.astype(np.uint32).reshape(-1)


def bf16_bits_exact(v: float) -> int:
    """bf16 pattern of a value that bf16 represents exactly."""
    b = synth.f64_to_bf16_rne(np.array([v]))[0]
    assert float(synth.bf16_to_f32(np.array([b]))[0]) == v
    return int(b)


def make_sb(scales_bits: np.ndarray, biases_bits: np.ndarray) -> np.ndarray:
    return (scales_bits.astype(np.uint32) | (biases_bits.astype(np.uint32) << np.uint32(16))).reshape(-1)


def random_qmatrix(rng, rows, cols, bits, dist=None):
    dist = dist or synth.dist_for_bits(bits)
    codes = rng.integers(0, 1 << bits, size=(rows, cols))
    ng = cols // 64
    s = synth.f64_to_bf16_rne(rng.uniform(dist.scale_lo, dist.scale_hi, size=(rows, ng)))
    b = synth.f64_to_bf16_rne(rng.uniform(dist.bias_lo, dist.bias_hi, size=(rows, ng)) - 1e-3)
    return codes, s, b, pack_codes(codes, bits), make_sb(s, b)


def bf16v(bits):
    return synth.bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def build_record(Wg, Wu, Wd, hidden, inter, bits):
    """Assemble a record from (codes, sbits, bbits) triples of gate, up, down."""
    lay = synth.record_layout(hidden, inter, bits)
    rec = np.zeros(lay.total, dtype=np.uint8)
    for (codes, s, b), off_c, off_s in ((Wg, lay.gate_codes, lay.gate_sb),
                                        (Wu, lay.up_codes, lay.up_sb),
                                        (Wd, lay.down_codes, lay.down_sb)):
        cw = pack_codes(codes, bits).view(np.uint8)
        rec[off_c:off_c + cw.size] = cw
        sw = make_sb(s, b).view(np.uint8)
        rec[off_s:off_s + sw.size] = sw
    return rec


def random_record(rng, hidden, inter, bits):
    trip = []
    for rows, cols in ((inter, hidden), (inter, hidden), (hidden, inter)):
        codes, s, b, _, _ = random_qmatrix(rng, rows, cols, bits)
        trip.append((codes, s, b))
    return build_record(*trip, hidden, inter, bits), trip


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64); b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------
# format
# ----------------------------------------------------------------------------
def pin_record_bytes_pages(orc):
    """6.75 MB per 4-bit expert and ~27 MB for the 4 routed experts of a layer,
    as printed on the pages, at hidden 4096 / intermediate 1024 / group 64."""
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    H = facts["hidden"]["value"]
    rb = orc.record_bytes(H, 1024, 4)
    assert rb == int(facts["expert_record_mb_4bit"]["value"] * 2 ** 20), rb
    four = facts["active_routed_experts"]["value"] * rb
    assert abs(four / 2 ** 20 - facts["four_experts_mb_per_layer"]["value"]) < 0.5
    # closed forms: codes I*H*b/8 per gate/up, H*I*b/8 for down, 4 bytes per group
    assert orc.record_bytes(4096, 1024, 2) == 3 * (1024 * 4096 // 4) + 3 * (1024 * 64 * 4)
    assert orc.record_bytes(256, 128, 4) == 3 * (128 * 256 // 2) + 3 * (128 * 4 * 4)
    assert orc.record_bytes(64, 64, 2) == 3 * 1024 + 3 * 256


def pin_onehot_decode(orc):
    """x = e_c gives y_r = q[r][c]*s + b exactly: recovers every code and the
    placement of scale (low half) and bias (high half) per 64-column group."""
    rng = np.random.default_rng(11)
    for bits, rows, cols in ((4, 5, 192), (2, 3, 256)):
        codes, s, b, words, sb = random_qmatrix(rng, rows, cols, bits)
        for c in range(cols):
            x = np.zeros(cols); x[c] = 1.0
            y = orc.qmatvec(words, sb, rows, cols, bits, x)
            want = codes[:, c] * bf16v(s[:, c // 64]) + bf16v(b[:, c // 64])
            assert np.array_equal(y, want), (bits, c)


def pin_zero_codes(orc):
    """All-zero codes: y_r = sum_g b[r][g] * (sum of x over group g), exactly in
    rationals (x dyadic)."""
    rng = np.random.default_rng(12)
    rows, cols, bits = 4, 256, 4
    codes = np.zeros((rows, cols), dtype=np.int64)
    _, s, b, _, _ = random_qmatrix(rng, rows, cols, bits)
    x = rng.integers(-64, 64, size=cols) / 16.0
    y = orc.qmatvec(pack_codes(codes, bits), make_sb(s, b), rows, cols, bits, x)
    bv = bf16v(b)
    for r in range(rows):
        exact = sum(Fraction(bv[r, g]) * sum(Fraction(v) for v in x[64 * g:64 * g + 64])
                    for g in range(cols // 64))
        assert abs(Fraction(y[r]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 60)


def pin_integer_dot(orc):
    """scale 1, bias 0: y is the integer dot product of codes and integer x."""
    rng = np.random.default_rng(13)
    for bits in (4, 2):
        rows, cols = 6, 128
        codes = rng.integers(0, 1 << bits, size=(rows, cols))
        one = bf16_bits_exact(1.0)
        s = np.full((rows, cols // 64), one, dtype=np.uint16)
        b = np.zeros((rows, cols // 64), dtype=np.uint16)
        x = rng.integers(-1000, 1000, size=cols)
        y = orc.qmatvec(pack_codes(codes, bits), make_sb(s, b), rows, cols, bits, x.astype(np.float64))
        want = [int(sum(int(codes[r, c]) * int(x[c]) for c in range(cols))) for r in range(rows)]
        assert [int(v) for v in y] == want and np.all(y == np.round(y))


def pin_constant_closed_form(orc):
    """codes 15, scale 2^-7, bias -2^-4, x = 1: each weight is 7/128, so each of
    the 64-column groups adds 3.5."""
    rows, cols = 2, 256
    codes = np.full((rows, cols), 15)
    s = np.full((rows, 4), bf16_bits_exact(2.0 ** -7), dtype=np.uint16)
    b = np.full((rows, 4), bf16_bits_exact(-2.0 ** -4), dtype=np.uint16)
    y = orc.qmatvec(pack_codes(codes, 4), make_sb(s, b), rows, cols, 4, np.ones(cols))
    assert np.all(y == 3.5 * 4)


def pin_exact_rational(orc):
    """Against the exact rational value of sum_c (q s + b) x_c, within the fp64
    summation bound; also the three regroupings the pages give are equal in
    exact arithmetic: (q s + b) x = q (s x) + b x = (q x) s + b x."""
    rng = np.random.default_rng(14)
    rows, cols, bits = 3, 128, 4
    codes, s, b, words, sb = random_qmatrix(rng, rows, cols, bits)
    x = synth.bf16_to_f32(synth.f64_to_bf16_rne(rng.standard_normal(cols))).astype(np.float64)
    y = orc.qmatvec(words, sb, rows, cols, bits, x)
    sv, bv = bf16v(s), bf16v(b)
    for r in range(rows):
        terms = []
        for c in range(cols):
            q = Fraction(int(codes[r, c])); sc = Fraction(sv[r, c // 64]); bi = Fraction(bv[r, c // 64]); xc = Fraction(x[c])
            t1 = (q * sc + bi) * xc
            t2 = q * (sc * xc) + bi * xc
            t3 = (q * xc) * sc + bi * xc
            assert t1 == t2 == t3
            terms.append(t1)
        exact = sum(terms)
        bound = Fraction(cols * 3) * Fraction(1, 2 ** 53) * sum(abs(t) for t in terms)
        assert abs(Fraction(y[r]) - exact) <= bound


def pin_dense_matvec(orc):
    """Brute force: materialised fp64 matrix (numpy unpack) @ x."""
    rng = np.random.default_rng(15)
    for bits, rows, cols in ((4, 8, 128), (4, 64, 256), (2, 16, 320), (2, 8, 64)):
        _, _, _, words, sb = random_qmatrix(rng, rows, cols, bits)
        x = rng.standard_normal(cols)
        W = dense.dense_matrix(words, sb, rows, cols, bits)
        y = orc.qmatvec(words, sb, rows, cols, bits, x)
        assert rel_err(y, W @ x) < 1e-13
        assert np.array_equal(orc.dequant_matrix(words, sb, rows, cols, bits), W)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
def pin_softmax(orc):
    rng = np.random.default_rng(16)
    logits = rng.standard_normal(512) * 3
    p = orc.softmax(logits)
    assert abs(p.sum() - 1.0) < 1e-14 and np.all(p > 0) and np.all(p < 1)
    assert rel_err(p, scipy.special.softmax(logits)) < 1e-13
    assert rel_err(orc.softmax(logits + 123.25), p) < 1e-12
    assert int(np.argmax(p)) == int(np.argmax(logits))


def pin_topk(orc):
    rng = np.random.default_rng(17)
    for E, K in ((512, 4), (16, 2), (8, 8), (64, 1)):
        logits = rng.standard_normal(E)
        idx = orc.topk(logits, K)
        assert list(idx) == list(np.argsort(-logits, kind="stable")[:K])
    ties = np.array([0.5, 2.0, 1.0, 2.0, 2.0, -1.0, 1.0])
    assert list(orc.topk(ties, 4)) == [1, 3, 4, 2]


def pin_topk_weights(orc):
    rng = np.random.default_rng(18)
    logits = rng.standard_normal(64)
    p = scipy.special.softmax(logits)
    idx = np.argsort(-logits, kind="stable")[:4].astype(np.int32)
    w0 = orc.topk_weights(p, idx, False)
    assert np.array_equal(w0, p[idx])
    w1 = orc.topk_weights(p, idx, True)
    assert abs(w1.sum() - 1.0) < 1e-15
    assert rel_err(w1, p[idx] / p[idx].sum()) < 1e-15


def pin_shared_gate(orc):
    rng = np.random.default_rng(19)
    g = rng.standard_normal(256).astype(np.float32) * 0.02
    x = rng.standard_normal(256)
    sg = orc.shared_gate(g, "f32", x)
    assert abs(sg - scipy.special.expit(g.astype(np.float64) @ x)) < 1e-15
    assert orc.shared_gate(np.zeros(64, np.float32), "f32", np.ones(64)) == 0.5
    gb = synth.f64_to_bf16_rne(rng.standard_normal(256) * 0.02)
    assert abs(orc.shared_gate(gb, "bf16", x) - scipy.special.expit(bf16v(gb) @ x)) < 1e-15


def pin_router(orc):
    rng = np.random.default_rng(20)
    E, H = 24, 192
    wf = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    wb = synth.f64_to_bf16_rne(rng.standard_normal((E, H)) * 0.02)
    x = rng.standard_normal(H)
    assert rel_err(orc.router(wf, "f32", x), wf.astype(np.float64) @ x) < 1e-13
    assert rel_err(orc.router(wb, "bf16", x), bf16v(wb) @ x) < 1e-13
    # one-hot x picks column c of W
    e5 = np.zeros(H); e5[5] = 1.0
    assert np.array_equal(orc.router(wb, "bf16", e5), bf16v(wb)[:, 5])


# ----------------------------------------------------------------------------
# expert, combine, layer
# ----------------------------------------------------------------------------
def pin_expert_onehot_swiglu(orc):
    """x = e_c makes a and u single dequantised weights; h = silu(a) * u with
    silu(a) = a * expit(a) (scipy), and y = W_down h (numpy matmul)."""
    rng = np.random.default_rng(21)
    H, I, bits = 128, 64, 4
    rec, (G, U, D) = random_record(rng, H, I, bits)
    c = 77
    x = np.zeros(H); x[c] = 1.0
    h, y = orc.expert(rec, H, I, bits, x)
    a = G[0][:, c] * bf16v(G[1][:, c // 64]) + bf16v(G[2][:, c // 64])
    u = U[0][:, c] * bf16v(U[1][:, c // 64]) + bf16v(U[2][:, c // 64])
    hh = a * scipy.special.expit(a) * u
    assert rel_err(h, hh) < 1e-14
    Wd = D[0] * np.repeat(bf16v(D[1]), 64, axis=1) + np.repeat(bf16v(D[2]), 64, axis=1)
    assert rel_err(y, Wd @ hh) < 1e-13


def pin_expert_dense(orc):
    rng = np.random.default_rng(22)
    for H, I, bits in ((256, 128, 4), (128, 192, 2)):
        rec, _ = random_record(rng, H, I, bits)
        x = rng.standard_normal(H)
        h, y = orc.expert(rec, H, I, bits, x)
        hd, yd = dense.expert(rec, H, I, bits, x)
        assert rel_err(h, hd) < 1e-12 and rel_err(y, yd) < 1e-12


def pin_combine(orc):
    rng = np.random.default_rng(23)
    H, K = 64, 3
    h_res = rng.standard_normal(H); y = rng.standard_normal((K, H)); ys = rng.standard_normal(H)
    w = np.array([0.5, 0.25, 0.125]); sig = 0.75
    out = orc.combine(h_res, y, w, ys, sig)
    # dyadic weights: one-at-a-time terms are exact, only the additions round
    want = h_res + 0.5 * y[0] + 0.25 * y[1] + 0.125 * y[2] + 0.75 * ys
    assert rel_err(out, want) < 1e-15
    assert np.array_equal(orc.combine(h_res, np.zeros((K, H)), w, np.zeros(H), sig), h_res)


def pin_rmsnorm(orc):
    n = 4096
    c = 3.0
    x = orc.rmsnorm(np.full(n, c), 1e-6)
    assert np.allclose(x, c / np.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)
    rng = np.random.default_rng(24)
    h = rng.standard_normal(n) * 5
    x = orc.rmsnorm(h, 1e-6)
    ms = np.mean(h * h)
    assert abs(np.mean(x * x) - ms / (ms + 1e-6)) < 1e-13
    assert rel_err(orc.rmsnorm(h * 8.0, 0.0), orc.rmsnorm(h, 0.0)) < 1e-15


def _tiny_layer_inputs(rng, E=8, K=2, H=128, I=64, bits_r=4, bits_s=4, same_experts=False):
    recs = []
    first = None
    for e in range(E):
        if same_experts and first is not None:
            recs.append(first)
            continue
        r, _ = random_record(rng, H, I, bits_r)
        recs.append(r)
        first = r
    stride = recs[0].size
    experts = np.concatenate(recs)
    shared, _ = random_record(rng, H, I, bits_s)
    router = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    gate = (rng.standard_normal(H) * 0.02).astype(np.float32)
    x = rng.standard_normal(H)
    h_res = rng.standard_normal(H)
    return dict(hidden=H, inter=I, n_experts=E, top_k=K, bits_routed=bits_r,
                bits_shared=bits_s, router=router, router_dtype="f32", gate_vec=gate,
                gate_dtype="f32", experts=experts, expert_stride=stride,
                shared_record=shared, x=x, h_res=h_res)


def pin_layer_dense(orc):
    """Whole layer: C oracle against the NumPy brute force, both renorm modes
    and a shared expert whose width differs from the routed ones."""
    rng = np.random.default_rng(25)
    for renorm, bits_r, bits_s in ((True, 4, 4), (False, 4, 2), (True, 2, 4)):
        args = _tiny_layer_inputs(rng, bits_r=bits_r, bits_s=bits_s)
        a = orc.layer(renorm=renorm, **args)
        d = dense.layer(renorm=renorm, **args)
        assert list(a["idx"]) == list(d["idx"])
        for k in ("logits", "p", "w", "h", "y", "out"):
            assert rel_err(a[k], d[k]) < 1e-12, k
        assert abs(a["sigma"] - d["sigma"]) < 1e-15


def pin_threads_bitwise(orc):
    """The row loops run on several threads, each row summed by one thread in
    its fixed order: every output is bitwise the same on one thread."""
    rng = np.random.default_rng(26)
    # one width and small records: the planted oracle mistakes that misread a
    # record's size (tests/test_oracle_mutants.py) then stay inside its buffer
    args = _tiny_layer_inputs(rng, E=8, K=2, H=128, I=64, bits_r=4, bits_s=4)
    n = orc.max_threads()
    many = orc.layer(renorm=True, **args)
    orc.set_threads(1)
    try:
        one = orc.layer(renorm=True, **args)
    finally:
        orc.set_threads(n)
    assert list(many["idx"]) == list(one["idx"])
    for k in ("logits", "p", "w", "h", "y", "out"):
        assert np.array_equal(np.asarray(many[k]), np.asarray(one[k])), k
    assert many["sigma"] == one["sigma"]


def pin_layer_all_selected(orc):
    """E = K: every expert is selected and (with renorm) the layer is the dense
    softmax mixture h_res + sum_e p_e y_e + sigma y_s (einsum brute force)."""
    rng = np.random.default_rng(26)
    args = _tiny_layer_inputs(rng, E=4, K=4)
    a = orc.layer(renorm=True, **args)
    assert sorted(a["idx"]) == [0, 1, 2, 3]
    ys = []
    for e in range(4):
        rec = args["experts"][e * args["expert_stride"]:(e + 1) * args["expert_stride"]]
        ys.append(dense.expert(rec, 128, 64, 4, args["x"])[1])
    logits = args["router"].astype(np.float64) @ args["x"]
    p = scipy.special.softmax(logits)
    sig = scipy.special.expit(args["gate_vec"].astype(np.float64) @ args["x"])
    ysh = dense.expert(args["shared_record"], 128, 64, 4, args["x"])[1]
    want = args["h_res"] + np.einsum("e,eh->h", p, np.stack(ys)) + sig * ysh
    assert rel_err(a["out"], want) < 1e-12


def pin_layer_identical_experts(orc):
    """All routed experts identical + renorm: out = h_res + y + sigma y_s."""
    rng = np.random.default_rng(27)
    args = _tiny_layer_inputs(rng, E=6, K=3, same_experts=True)
    a = orc.layer(renorm=True, **args)
    y = a["y"][0]
    for k in range(3):
        assert np.array_equal(a["y"][k], y)
    want = args["h_res"] + y + a["sigma"] * a["y"][3]
    assert rel_err(a["out"], want) < 1e-14


def pin_layer_zero_experts(orc):
    """Zero codes and zero bias everywhere: every expert output is exactly 0 and
    the layer returns the residual unchanged."""
    rng = np.random.default_rng(28)
    args = _tiny_layer_inputs(rng)
    args["experts"] = np.zeros_like(args["experts"])
    args["shared_record"] = np.zeros_like(args["shared_record"])
    a = orc.layer(renorm=True, **args)
    assert np.array_equal(a["out"], args["h_res"]) and not np.any(a["y"])


# ----------------------------------------------------------------------------
# gated delta-rule decode step
# ----------------------------------------------------------------------------
def _gdn_inputs(rng, n_seq=2, n_heads=3, d_k=8, d_v=6):
    S = rng.standard_normal((n_seq, n_heads, d_v, d_k))
    q = rng.standard_normal((n_seq, n_heads, d_k))
    k = rng.standard_normal((n_seq, n_heads, d_k))
    v = rng.standard_normal((n_seq, n_heads, d_v))
    return S, q, k, v


def pin_gdn_identity(orc):
    """alpha = 1, beta = 0: the state is unchanged (exactly) and o = S q
    (numpy matmul)."""
    rng = np.random.default_rng(11)
    S, q, k, v = _gdn_inputs(rng)
    ones, zeros = np.ones(S.shape[:2]), np.zeros(S.shape[:2])
    Sn, o = orc.gdn_step(q, k, v, ones, zeros, S)
    assert np.array_equal(Sn, S)
    assert np.allclose(o, np.einsum("shij,shj->shi", S, q), rtol=1e-13, atol=1e-13)


def pin_gdn_column_write(orc):
    """alpha = 1, beta = 1, k = e_j: column j of the state becomes v and the
    other columns keep their values (the delta rule writes v at key j)."""
    rng = np.random.default_rng(12)
    S, q, _, v = _gdn_inputs(rng)
    j = 5
    k = np.zeros(q.shape)
    k[..., j] = 1.0
    Sn, o = orc.gdn_step(q, k, v, np.ones(S.shape[:2]), np.ones(S.shape[:2]), S)
    others = [c for c in range(S.shape[3]) if c != j]
    assert np.array_equal(Sn[..., others], S[..., others])
    assert np.allclose(Sn[..., j], v, rtol=0, atol=1e-15)
    assert np.allclose(o, np.einsum("shij,shj->shi", Sn, q), rtol=1e-13, atol=1e-13)


def pin_gdn_reset(orc):
    """alpha = 0: the old state is forgotten, S = beta v k^T and o = beta v (k . q)."""
    rng = np.random.default_rng(13)
    S, q, k, v = _gdn_inputs(rng)
    beta = rng.uniform(0.1, 0.9, S.shape[:2])
    Sn, o = orc.gdn_step(q, k, v, np.zeros(S.shape[:2]), beta, S)
    want = beta[..., None, None] * v[..., :, None] * k[..., None, :]
    assert np.allclose(Sn, want, rtol=1e-14, atol=1e-15)
    kq = np.einsum("shj,shj->sh", k, q)
    assert np.allclose(o, beta[..., None] * v * kq[..., None], rtol=1e-12, atol=1e-13)


def pin_gdn_matrix_form(orc):
    """The closed matrix form of the gated delta rule,
    S_new = alpha S (I - beta k k^T) + beta v k^T, evaluated with numpy
    matrix products (a different evaluation order)."""
    rng = np.random.default_rng(14)
    S, q, k, v = _gdn_inputs(rng, n_seq=2, n_heads=4, d_k=16, d_v=12)
    alpha = rng.uniform(0.5, 1.0, S.shape[:2])
    beta = rng.uniform(0.0, 1.0, S.shape[:2])
    Sn, o = orc.gdn_step(q, k, v, alpha, beta, S)
    eye = np.eye(S.shape[3])
    for s_ in range(S.shape[0]):
        for h in range(S.shape[1]):
            kk = np.outer(k[s_, h], k[s_, h])
            want = alpha[s_, h] * S[s_, h] @ (eye - beta[s_, h] * kk) + beta[s_, h] * np.outer(v[s_, h], k[s_, h])
            assert np.allclose(Sn[s_, h], want, rtol=1e-12, atol=1e-12)
            assert np.allclose(o[s_, h], want @ q[s_, h], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# linear-attention block around the decode step
# ----------------------------------------------------------------------------
def _gdn_block_inputs(rng, H=128, n_heads=2, d_head=32, bits=4):
    D = n_heads * d_head
    rq, _ = random_record(rng, H, D, bits)
    rv, _ = random_record(rng, H, D, bits)
    h = rng.standard_normal(H)
    S = 0.1 * rng.standard_normal((n_heads, d_head, d_head))
    return rq, rv, h, S


def pin_gdn_block_dense(orc):
    """The whole block against its dense NumPy brute force (matrices
    materialised, products by matmul, the delta rule in closed matrix form),
    at 4 and 2 bits."""
    for bits, seed in ((4, 21), (2, 22)):
        rng = np.random.default_rng(seed)
        H, nh, dh = 128, 2, 32
        rq, rv, h, S = _gdn_block_inputs(rng, H, nh, dh, bits)
        got = orc.gdn_block(rq, rv, H, nh, dh, bits, h, S)
        want = dense.gdn_block(rq, rv, H, nh, dh, bits, h, S)
        for key in ("proj", "o", "h_out", "state"):
            assert rel_err(got[key], want[key]) < 1e-12, (bits, key, rel_err(got[key], want[key]))


def pin_gdn_block_gates_and_unit_keys(orc):
    """With zero gate rows (codes and biases 0) both gates are sigmoid(0) =
    1/2 exactly; then, from the block's own projections, the new state must be
    S/2 (I - k^ k^T/2) + v k^T/2 with k^ = k / sqrt(|k|^2 + 1e-6) per head, and
    o = S_new q^: unit-length keys and queries, checked with numpy."""
    rng = np.random.default_rng(23)
    H, nh, dh, bits = 128, 2, 32, 4
    D = nh * dh
    rq, _ = random_record(rng, H, D, bits)
    trip = []
    for rows, cols in ((D, H), (D, H), (H, D)):
        codes, s, b, _, _ = random_qmatrix(rng, rows, cols, bits)
        trip.append((codes, s, b))
    codes, s, b = trip[1]
    codes[:2 * nh] = 0
    b[:2 * nh] = 0
    rv = build_record(trip[0], (codes, s, b), trip[2], H, D, bits)
    h = rng.standard_normal(H)
    S = 0.1 * rng.standard_normal((nh, dh, dh))
    got = orc.gdn_block(rq, rv, H, nh, dh, bits, h, S)
    proj = got["proj"]
    assert np.array_equal(proj[3 * D:], np.zeros(2 * nh))
    q = proj[:D].reshape(nh, dh)
    k = proj[D:2 * D].reshape(nh, dh)
    v = proj[2 * D:3 * D].reshape(nh, dh)
    qh = q / np.sqrt(np.sum(q * q, axis=1, keepdims=True) + 1e-6)
    kh = k / np.sqrt(np.sum(k * k, axis=1, keepdims=True) + 1e-6)
    eye = np.eye(dh)
    for i in range(nh):
        want = 0.5 * S[i] @ (eye - 0.5 * np.outer(kh[i], kh[i])) + 0.5 * np.outer(v[i], kh[i])
        assert np.allclose(got["state"][i], want, rtol=1e-12, atol=1e-13)
        assert np.allclose(got["o"][i * dh:(i + 1) * dh], want @ qh[i], rtol=1e-12, atol=1e-13)


def pin_gdn_block_zero_output_projection(orc):
    """A zero output projection (codes and biases 0) leaves the residual
    stream exactly as it was, whatever the state does."""
    rng = np.random.default_rng(24)
    H, nh, dh, bits = 128, 2, 32, 4
    D = nh * dh
    trip = []
    for rows, cols in ((D, H), (D, H), (H, D)):
        codes, s, b, _, _ = random_qmatrix(rng, rows, cols, bits)
        trip.append((codes, s, b))
    codes, s, b = trip[2]
    rq = build_record(trip[0], trip[1], (np.zeros_like(codes), s, np.zeros_like(b)), H, D, bits)
    rv, _ = random_record(rng, H, D, bits)
    h = rng.standard_normal(H)
    S = 0.1 * rng.standard_normal((nh, dh, dh))
    got = orc.gdn_block(rq, rv, H, nh, dh, bits, h, S)
    assert np.array_equal(got["h_out"], h)
    assert not np.allclose(got["state"], S)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
