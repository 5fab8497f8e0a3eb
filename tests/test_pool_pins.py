"""The expert slot pool's replacement policy: the reference (oracle/pool_oracle.py)
pinned by closed-form traces, then the library's pool (csrc/pool.hip, in its
host-only mode: no device) checked against the reference decision by
decision on long seeded traces.  No GPU."""
import numpy as np
import pytest

from oracle.pool_oracle import SlotPool

A, B, C, D = 0, 1, 2, 3


def test_compulsory_misses_only_when_everything_fits(rng):
    p = SlotPool(64)
    keys = set()
    for _ in range(50):
        layer = int(rng.integers(0, 4))
        ex = rng.choice(16, 5, replace=False).tolist()
        p.require(layer, ex)
        keys |= {(layer, e) for e in ex}
    assert p.misses == len(keys) and p.evictions == 0
    assert p.hits == 250 - len(keys)


def test_single_slot_misses_on_every_change():
    p = SlotPool(1)
    for e in (A, B, A, B, B, A):
        p.require(0, [e])
    assert (p.hits, p.misses) == (1, 5)


def test_least_frequent_is_evicted_not_least_recent():
    """A is used 3 times, then B once (more recently); C must replace B (an
    LRU policy would replace A)."""
    p = SlotPool(2)
    for e in (A, A, A, B):
        p.require(0, [e])
    sa, sb = p.slot_of(0, A), p.slot_of(0, B)
    p.require(0, [C])
    assert p.slot_of(0, C) == sb and p.slot_of(0, A) == sa and p.slot_of(0, B) == -1


def test_equal_counts_fall_back_to_recency():
    p = SlotPool(2)
    p.require(0, [A])
    p.require(0, [B])
    p.require(0, [C])            # A and B used once each: A is older
    assert p.slot_of(0, A) == -1 and p.slot_of(0, C) == 0 and p.slot_of(0, B) == 1


def test_keys_of_the_current_call_are_not_evicted():
    """Calls [A, B] then [C, A]: C replaces one of A, B (equal count and
    tick: the lower slot, A's); then A misses and must replace B, not C."""
    p = SlotPool(2)
    assert p.require(0, [A, B]) == [(A, 0), (B, 1)]
    assert p.require(0, [C, A]) == [(C, 0), (A, 1)]
    assert p.slot_of(0, B) == -1


def test_layers_are_separate_keys():
    p = SlotPool(4)
    p.require(0, [A, B])
    p.require(1, [A, B])
    assert p.misses == 4 and p.slot_of(1, A) == 2


def test_too_many_distinct_experts_refused():
    p = SlotPool(3)
    with pytest.raises(ValueError):
        p.require(0, [A, B, C, D])
    p.require(0, [A, A, B, B, C])   # repeats count once
    assert p.misses == 3 and p.hits == 2


# planted mistakes, each caught by a pin above


def _plant(monkeypatch, fn):
    monkeypatch.setattr(SlotPool, "require", fn)


def _require_evict_most_frequent(self, layer, experts):
    self.tick += 1
    loads = []
    for e in experts:
        key = (layer, int(e))
        if key in self.where:
            self.hits += 1
            self.count[key] += 1
            self.last[key] = self.tick
            continue
        self.misses += 1
        free = [s for s in range(self.n_slots) if self.slot_key[s] is None]
        if free:
            slot = free[0]
        else:
            cands = [(-self.count[k], self.last[k], s) for s, k in enumerate(self.slot_key)
                     if self.last[k] < self.tick]   # wrong: the most frequent
            _, _, slot = min(cands)
            old = self.slot_key[slot]
            del self.where[old], self.count[old], self.last[old]
        self.slot_key[slot] = key
        self.where[key] = slot
        self.count[key] = 1
        self.last[key] = self.tick
        loads.append((int(e), slot))
    return loads


def test_planted_most_frequent_eviction_is_caught(monkeypatch):
    _plant(monkeypatch, _require_evict_most_frequent)
    with pytest.raises(AssertionError):
        test_least_frequent_is_evicted_not_least_recent()


# ---------------------------------------------------------------------------
# the library's pool against the reference


def _trace(rng, n_layers, E, calls, k, zipf):
    """Requests of k distinct experts per call, cycling over the layers, with
    a Zipf-skewed expert popularity per layer (seeded permutations)."""
    perms = [rng.permutation(E) for _ in range(n_layers)]
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** -zipf
    p /= p.sum()
    out = []
    for c in range(calls):
        layer = c % n_layers
        ex = perms[layer][rng.choice(E, k, replace=False, p=p)]
        out.append((layer, [int(e) for e in ex]))
    return out


@pytest.mark.parametrize("n_slots,zipf", [(40, 1.1), (128, 1.1), (300, 0.0), (12, 0.5)])
def test_library_pool_matches_reference(rng, n_slots, zipf):
    import int4_group_quantized_moe_amd as moe
    d = moe.make_desc(1, 256, 64, 10, 128, 128, bits=4)
    n_layers, E, k = 6, 64, 10
    pool = moe.MoePool(d, n_layers, n_slots, host_only=True)
    ref = SlotPool(n_slots)
    for layer, ex in _trace(rng, n_layers, E, 600, k, zipf):
        loads = ref.require(layer, ex)
        missed = pool.require(layer, ex, stream=0)
        assert missed == len(loads)
        for e, s in loads:
            assert pool.slot(layer, e) == s
    st = pool.stats()
    assert (st["hits"], st["misses"], st["evictions"]) == (ref.hits, ref.misses, ref.evictions)
    assert st["lookups"] == 600 * k and st["bytes_copied"] == 0
    # every resident key agrees
    for layer in range(n_layers):
        for e in range(E):
            assert pool.slot(layer, e) == ref.slot_of(layer, e)


def test_library_pool_rejects_bad_requests():
    import int4_group_quantized_moe_amd as moe
    d = moe.make_desc(1, 256, 64, 10, 128, 128, bits=4)
    pool = moe.MoePool(d, 2, 3, host_only=True)
    for layer, ex in ((2, [0]), (0, [64]), (0, [-1]), (0, [0, 1, 2, 3])):
        with pytest.raises(moe.MoeError):
            pool.require(layer, ex, stream=0)
    assert pool.stats()["requests"] == 0
    assert pool.require(0, [5, 5, 6], stream=0) == 2
