"""Host checks of the top-K selection's building blocks, without a GPU.

1. The comparator network every lane runs on its eight keys (the table in
   csrc/moe_sortnet.h that the kernels compile in) sorts in descending order:
   exhaustively over all 2^8 zero-one inputs (by the zero-one principle that
   proves it sorts any input), and on random 64-bit keyed words with ties.
2. The order-preserving key of a logit (larger float, larger unsigned key;
   NaN ranks as -inf; -0 and +0 tie), modelled bit for bit on float32.
3. The selection procedure on those keys, modelled as the kernels run it --
   lane l sorts the words of experts 8l..8l+7, then K rounds take the wave
   maximum of the lanes' first keys, the lowest lane holding it, and shift
   that lane's list; and the four-wave split (each quarter selects its K,
   the 4K candidate words are merged by their 64-bit value, or entry by
   entry by counting the larger words) -- against a
   brute-force stable sort by (logit descending, expert ascending), on
   logits drawn from a small set of values so that ties are frequent."""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NET_H = os.path.join(ROOT, "bit_dequant_expert_route_amd", "csrc", "moe_sortnet.h")


def network():
    text = open(NET_H).read()
    body = text[text.index("kSort8Net"):]
    body = body[body.index("{") + 1: body.index("};")]
    pairs = [(int(a), int(b)) for a, b in re.findall(r"\{\s*(\d+)\s*,\s*(\d+)\s*\}", body)]
    n = int(re.search(r"kSort8Comparators\s*=\s*(\d+)", text).group(1))
    assert len(pairs) == n
    return pairs


def apply(net, vals):
    v = list(vals)
    for i, j in net:
        if v[j] > v[i]:
            v[i], v[j] = v[j], v[i]
    return v


def test_network_shape():
    net = network()
    assert len(net) == 19
    # depth 6: comparators fall into six layers of disjoint wires
    depth = [0] * 8
    for i, j in net:
        d = max(depth[i], depth[j]) + 1
        depth[i] = depth[j] = d
    assert max(depth) == 6


def test_network_sorts_all_zero_one_inputs():
    net = network()
    for m in range(256):
        bits = [(m >> k) & 1 for k in range(8)]
        assert apply(net, bits) == sorted(bits, reverse=True), bits


def test_network_sorts_keyed_words_with_ties():
    net = network()
    rng = np.random.default_rng(0)
    for _ in range(20000):
        keys = rng.integers(0, 4, size=8)          # many equal keys
        e = rng.permutation(8)
        words = [(int(k) << 32) | (0xFFFFFFFF - int(x)) for k, x in zip(keys, e)]
        assert apply(net, words) == sorted(words, reverse=True)


def logit_key(f):
    """The kernels' key: NaN -> key of -inf, -0 -> +0, then flip."""
    f = np.float32(f)
    if np.isnan(f):
        f = np.float32(-np.inf)
    f = np.float32(f + np.float32(0.0))
    b = int(np.array(f, dtype=np.float32).view(np.uint32))
    return (~b) & 0xFFFFFFFF if b & 0x80000000 else b | 0x80000000


def test_logit_key_orders_like_floats():
    vals = [-np.inf, -3e38, -1.0, -1e-38, -1e-45, -0.0, 0.0, 1e-45, 1e-38, 0.5, 1.0, 3e38, np.inf]
    keys = [logit_key(v) for v in vals]
    for a in range(len(vals)):
        for b in range(len(vals)):
            assert (keys[a] < keys[b]) == (vals[a] < vals[b]), (vals[a], vals[b])
            assert (keys[a] == keys[b]) == (vals[a] == vals[b])
    assert logit_key(np.nan) == logit_key(-np.inf)
    rng = np.random.default_rng(1)
    x = rng.standard_normal(5000).astype(np.float32)
    k = np.array([logit_key(v) for v in x], dtype=np.uint64)
    assert np.array_equal(np.argsort(x, kind="stable"), np.argsort(k, kind="stable"))


def word(logit, e):
    return (logit_key(logit) << 32) | (0xFFFFFFFF - e)


def select_lane_lists(net, logits, K):
    """One wave, E <= 512: lane l holds experts 8l..8l+7 (absent ones are 0)."""
    E = len(logits)
    lanes = []
    for l in range(64):
        ws = [word(logits[8 * l + i], 8 * l + i) if 8 * l + i < E else 0 for i in range(8)]
        lanes.append(apply(net, ws))
    out = []
    for _ in range(K):
        heads = [lst[0] >> 32 for lst in lanes]
        m = max(heads)
        src = heads.index(m)                      # the lowest lane holding it
        out.append(0xFFFFFFFF - (lanes[src][0] & 0xFFFFFFFF))
        lanes[src] = lanes[src][1:] + [0]
    return out


def select_split(logits, K, npl):
    """Four waves: wave w takes experts [w R, (w + 1) R), R = 64 npl, lane l
    of it the npl consecutive experts w R + npl l + i; each wave selects its
    top K, then the 4 K words are merged by their 64-bit value."""
    E = len(logits)
    R = 64 * npl
    cands = []
    for w in range(4):
        ws = [word(logits[e], e) for e in range(w * R, min((w + 1) * R, E))]
        cands += sorted(ws, reverse=True)[:K]
    cands.sort(reverse=True)
    return [0xFFFFFFFF - (c & 0xFFFFFFFF) for c in cands[:K]]


def split_candidates(logits, K, npl):
    """The 4 K candidate words the four waves leave in LDS: each wave's top K
    words in descending order, a wave with fewer than K experts padding its
    list with 0 words."""
    E = len(logits)
    R = 64 * npl
    cands = []
    for w in range(4):
        ws = sorted((word(logits[e], e) for e in range(w * R, min((w + 1) * R, E))), reverse=True)[:K]
        cands += ws + [0] * (K - len(ws))
    return cands


def merge_one(cands, k, E):
    """Entry k of the merge by rank count (topk_merge_one): lane j's word is
    entry k if exactly k of the words are larger; the lowest such lane is
    read; a 0 word, an expert out of range or no such lane gives -2."""
    ranks = [sum(1 for o in cands if o > c) for c in cands]
    lanes = [j for j, r in enumerate(ranks) if r == k]
    if not lanes:
        return -2
    c = cands[lanes[0]]
    ex = 0xFFFFFFFF - (c & 0xFFFFFFFF)
    return ex if (c >> 32) != 0 and ex < E else -2


def brute(logits, K):
    order = sorted(range(len(logits)), key=lambda e: (-float(np.float32(logits[e]) + 0.0)
                                                      if not np.isnan(logits[e]) else np.inf, e))
    return order[:K]


@pytest.mark.parametrize("E,K", [(512, 4), (16, 2), (8, 8), (300, 8), (64, 1), (256, 4), (1024, 8), (600, 8)])
def test_selection_with_ties(E, K):
    net = network()
    rng = np.random.default_rng(E * 10 + K)
    for trial in range(60):
        pool = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, np.nan], dtype=np.float32)
        logits = rng.choice(pool, size=E).astype(np.float32)
        if trial % 3 == 0:
            logits = rng.standard_normal(E).astype(np.float32)
        want = brute(logits, K)
        if E <= 512:  # the one-wave selection's eight-per-lane layout
            assert select_lane_lists(net, logits, K) == want
        assert select_split(logits, K, 2 if E <= 512 else 4) == want
        cands = split_candidates(logits, K, 2 if E <= 512 else 4)
        assert [merge_one(cands, k, E) for k in range(K)] == want
