"""Host bookkeeping of the expert tier (moe_tier_create / _assign / _stats),
checked against a plain least-recently-used model; no device is touched (the
tier only records addresses until a decode call)."""
import random

import pytest

moe = pytest.importorskip("bit_dequant_expert_route_amd.moe")

HOST, CACHE, STRIDE = 0x10000, 0x100000, 256


class LRUModel:
    """Slots hold experts; a call takes one tick; a miss takes the slot with
    the oldest last use among those this call has not used (never-used slots
    first, lowest index on ties)."""

    def __init__(self, n_slots):
        self.owner = [-1] * n_slots
        self.used = [0] * n_slots
        self.tick = 0

    def assign(self, ids):
        self.tick += 1
        slots, miss = [], []
        for e in ids:
            if e in self.owner:
                s = self.owner.index(e)
                miss.append(0)
            else:
                cand = [j for j in range(len(self.owner)) if self.used[j] < self.tick]
                s = min(cand, key=lambda j: (self.used[j], j))
                self.owner[s] = e
                miss.append(1)
            self.used[s] = self.tick
            slots.append(s)
        return slots, miss


@pytest.mark.parametrize("n_experts,n_slots,k,seed", [(32, 8, 4, 1), (512, 64, 4, 2), (16, 8, 8, 3)])
def test_assign_matches_lru_model(n_experts, n_slots, k, seed):
    rng = random.Random(seed)
    t = moe.Tier(None, n_experts, STRIDE, CACHE, n_slots, host_ptr=HOST)
    model = LRUModel(n_slots)
    hot = list(range(0, n_experts, max(1, n_experts // (2 * n_slots))))
    total = model_misses = 0
    for step in range(300):
        pool = hot if rng.random() < 0.7 else list(range(n_experts))
        ids = rng.sample(pool, k) if len(pool) >= k else rng.sample(range(n_experts), k)
        slots, miss = t.assign(ids)
        want_slots, want_miss = model.assign(ids)
        assert (slots, miss) == (want_slots, want_miss), (step, ids, slots, want_slots)
        assert len(set(slots)) == len(ids)  # distinct slots within a call
        total += len(ids)
        model_misses += sum(want_miss)
    hits, misses, copied = t.stats()
    assert (hits, misses) == (total - model_misses, model_misses)
    assert 0 < misses < total
    assert copied == 0  # assign alone copies nothing
    t.close()


def test_repeat_is_hit_and_eviction_order():
    t = moe.Tier(None, 16, STRIDE, CACHE, 8, host_ptr=HOST)
    s1, m1 = t.assign([0, 1, 2, 3, 4, 5, 6, 7])
    assert m1 == [1] * 8 and s1 == list(range(8))
    s2, m2 = t.assign([3, 9])  # 3 hits; 9 evicts the oldest slot not used now
    assert m2 == [0, 1] and s2[0] == s1[3] and s2[1] == 0
    s3, m3 = t.assign([0])  # 0 was evicted by 9
    assert m3 == [1] and s3[0] == 1
    assert t.stats()[:2] == (1, 10)
    t.close()


def test_tier_validation():
    with pytest.raises(moe.MoeError):
        moe.Tier(None, 16, STRIDE, CACHE, 4, host_ptr=HOST)  # fewer slots than the largest K
    with pytest.raises(moe.MoeError):
        moe.Tier(None, 16, STRIDE, CACHE, 17, host_ptr=HOST)  # more slots than experts
    with pytest.raises(moe.MoeError):
        moe.Tier(None, 16, STRIDE + 16, CACHE, 8, host_ptr=HOST)  # stride not 256-aligned
    with pytest.raises(moe.MoeError):
        moe.Tier(None, 16, STRIDE, CACHE + 8, 8, host_ptr=HOST)  # cache not 256-aligned
    t = moe.Tier(None, 16, STRIDE, CACHE, 8, host_ptr=HOST)
    with pytest.raises(moe.MoeError):
        t.assign([16])
    with pytest.raises(moe.MoeError):
        t.assign(list(range(9)))  # more ids than slots
    t.close()
