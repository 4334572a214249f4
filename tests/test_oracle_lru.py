"""Pins of the oracle's shared LRU slot cache (no GPU).

* Brute force: with every miss filled (B_H <= B_P) and enough victims, the
  cache must behave as a textbook LRU (collections.OrderedDict): [FT]
  "语义感知专家缓存" -- a hit refreshes recency, a fill admits, eviction takes
  the least recently needed.  For q < m the brute force admits only the
  first q misses, as the split of [FT] "q* 策略" prescribes.
* Invariants after every call: residency tables are mutual inverses, hits and
  fills are resident, the host set is not and is left untouched ([FT] "q*
  策略"), no hit slot is a victim, victims are the q smallest keys.
* The cache example printed on the pages (tests/golden).
"""
from collections import OrderedDict

import numpy as np
import pytest

from oracle import lru, qsplit
from tests.conftest import golden


class TextbookLRU:
    def __init__(self, C, seeded):
        self.C = C
        self.od = OrderedDict((i, None) for i in seeded)   # front = least recent

    def step(self, uniq, q_cap):
        hits = [i for i in uniq if i in self.od]
        misses = [i for i in uniq if i not in self.od]
        for i in hits:
            self.od.move_to_end(i)
        q = min(q_cap(len(misses)), self.C - len(hits))
        evicted = []
        for i in misses[:q]:
            if len(self.od) >= self.C:
                old, _ = self.od.popitem(last=False)
                evicted.append(old)
            else:
                evicted.append(-1)
            self.od[i] = None
        return hits, misses[:q], misses[q:], evicted


def _random_trace(rng, steps, L, E, T, k):
    out = []
    for _ in range(steps):
        layer = int(rng.integers(0, L))
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        out.append((layer, ids))
    return out


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("bp,bh", [(900, 475), (118, 475), (527, 773)])
def test_lru_matches_textbook(seed, bp, bh):
    rng = np.random.default_rng(seed)
    L, E = int(rng.integers(1, 4)), int(rng.integers(3, 5))
    C = int(rng.integers(1, 7))
    T, k = int(rng.integers(1, 3)), int(rng.integers(1, min(E, 3) + 1))
    seeded = list(rng.choice(L * E, size=min(C, L * E) // 2, replace=False))
    oc = lru.ExpertCache(L, E, C, bp, bh)
    oc.seed(seeded)
    tb = TextbookLRU(C, seeded)
    for layer, ids in _random_trace(rng, 200, L, E, T, k):
        r = oc.step(layer, ids)
        uniq = sorted(set((layer * E + ids).reshape(-1).tolist()))
        hits, fills, host, evicted = tb.step(uniq, lambda m: qsplit.q_star(m, bp, bh))
        assert r.uniq == uniq and r.hits == hits
        assert r.fill_id == fills and r.host_id == host
        assert r.fill_evicted == evicted
        resident = set(i for i in oc.slot_id if i >= 0)
        assert resident == set(tb.od.keys())


def _check_invariants(oc, r, layer, ids, before):
    slot_id, ts, id_slot, _ = oc.tables()
    for s, i in enumerate(slot_id):
        if i >= 0:
            assert id_slot[i] == s
    for i, s in enumerate(id_slot):
        if s >= 0:
            assert slot_id[s] == i
    assert (slot_id >= 0).sum() <= oc.C
    for i in r.hits + r.fill_id:
        assert id_slot[i] >= 0
    for i in r.host_id:
        assert id_slot[i] < 0                       # host set not admitted
    old_slot_id, old_ts = before
    hit_slots = set(old_slot_id.tolist().index(i) for i in r.hits)
    assert not (hit_slots & set(r.fill_slot))        # hits are never victims
    # victims are the q smallest (stamp, slot) keys among the other slots
    keys = sorted((int(old_ts[s]), s) for s in range(oc.C)
                  if s not in hit_slots and old_slot_id[s] != lru.RESERVED)
    assert [s for _, s in keys[:r.q]] == r.fill_slot
    # stamps unique among occupied slots
    occ = ts[slot_id >= 0]
    assert len(set(occ.tolist())) == len(occ)
    # rewrite: each pick points at its expert's slot or at the host (-1)
    E = oc.E
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            lid = layer * E + int(ids[t, j])
            if lid in r.host_id:
                assert r.pick_slot[t, j] == -1
            else:
                assert slot_id[r.pick_slot[t, j]] == lid


@pytest.mark.parametrize("seed", range(6))
def test_lru_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    L, E, C, T, k = 3, 8, 7, 3, 2
    oc = lru.ExpertCache(L, E, C, 118, 475)
    oc.seed([0, 9, 17])
    if seed % 2:
        oc.reserve(5, 2)
    for layer, ids in _random_trace(rng, 150, L, E, T, k):
        before = (np.array(oc.slot_id), np.array(oc.ts, np.uint64))
        r = oc.step(layer, ids)
        _check_invariants(oc, r, layer, ids, before)
        if seed % 2:
            assert oc.slot_id[5] == lru.RESERVED and oc.slot_id[6] == lru.RESERVED


def test_page_cache_example():
    """12 routed experts, 8 of them cached, 4 missing at 11.8:47.5 -> 1 fill, 3 on the host."""
    g = golden("qstar_worked_examples.json")["cache_example"]
    E = 16
    oc = lru.ExpertCache(1, E, 12, g["bp"], g["bh"])
    oc.seed(list(range(g["cached"])))                  # experts 0..7 cached, 4 slots empty
    ids = np.arange(g["routed"]).reshape(6, 2)          # routes to experts 0..11
    r = oc.step(0, ids)
    assert len(r.hits) == g["cached"] and len(r.misses) == g["missing"]
    assert r.q == g["fills"] and len(r.host_id) == g["host"]
    assert r.fill_id == [8] and r.host_id == [9, 10, 11]
    assert r.fill_slot == [8] and r.fill_evicted == [-1]   # empty slots go first


def test_all_hits_no_fill_and_no_victim_cases():
    oc = lru.ExpertCache(1, 8, 4, 118, 475)
    oc.seed([0, 1, 2, 3])
    r = oc.step(0, np.array([[0, 1], [2, 3]]))
    assert r.q_star == 0 and r.q == 0 and r.host_id == [] and r.fill_id == []
    # every slot is a hit, one miss: q* = 1 but no free victim -> host
    r = oc.step(0, np.array([[0, 1], [2, 3], [4, 0]]))
    assert r.q_star == 1 and r.q == 0 and r.host_id == [4]
    assert (r.pick_slot[2] == [-1, oc.id_slot[0]]).all()


def test_lru_refresh_order_by_hand():
    """C = 2, all misses filled: trace [a], [b], [a], [c] evicts b, not a."""
    oc = lru.ExpertCache(1, 4, 2, 900, 475)
    for ids in ([[0]], [[1]], [[0]]):
        oc.step(0, np.array(ids))
    r = oc.step(0, np.array([[2]]))
    assert r.fill_evicted == [1]
    assert sorted(i for i in oc.slot_id if i >= 0) == [0, 2]


def test_cross_layer_sharing():
    """The LRU spans layers: an expert of layer 1 can evict one of layer 0."""
    oc = lru.ExpertCache(2, 4, 1, 900, 475)
    oc.step(0, np.array([[3]]))
    r = oc.step(1, np.array([[3]]))
    assert r.fill_id == [7] and r.fill_evicted == [3]


def test_tiny_config_all_hit_consequence():
    """Tiny workload: 4 seeded slots all hit, no victim -> q = 0, all misses on host."""
    oc = lru.ExpertCache(1, 8, 4, 118, 475)
    oc.seed([0, 1, 2, 3])
    ids = np.array([[i % 8, (i + 4) % 8] for i in range(32)])
    r = oc.step(0, ids)
    assert r.hits == [0, 1, 2, 3] and r.q_star == 1 and r.q == 0
    assert r.host_id == [4, 5, 6, 7]


# ---------------------------------------------------------------- prefill hand-over and on-demand loading
@pytest.mark.parametrize("seed", range(8))
def test_fill_all_matches_textbook(seed):
    """On-demand loading fills every miss that has room: the textbook LRU
    with q capped only by the free or evictable slots, whatever the
    bandwidth ratio (here one that would keep most misses on the host)."""
    rng = np.random.default_rng(300 + seed)
    L, E, C, T, k = 2, 6, int(rng.integers(2, 9)), 3, 2
    oc = lru.ExpertCache(L, E, C, 1, 1000)
    tb = TextbookLRU(C, [])
    for layer, ids in _random_trace(rng, 120, L, E, T, k):
        r = oc.step(layer, ids, fill_all=True)
        uniq = sorted(set((layer * E + ids).reshape(-1).tolist()))
        hits, fills, host, evicted = tb.step(uniq, lambda m: m)
        assert r.q_star == len(r.misses)
        assert (r.hits, r.fill_id, r.host_id, r.fill_evicted) == (hits, fills, host, evicted)


def _prefill_then_textbook(rng, L, E, C, n_buf, n_layers_run, pre_resident):
    """Reserve n_buf full-layer buffers, run prefill over layers
    0..n_layers_run-1 (layer l in buffer l % n_buf), finish; return the
    oracle cache and the textbook LRU that must agree with it from there."""
    first = C - n_buf * E
    oc = lru.ExpertCache(L, E, C, 900, 475)
    oc.seed(pre_resident)
    oc.reserve(first, n_buf * E)
    held = {}
    order = []
    for l in range(n_layers_run):
        b = l % n_buf
        held[b] = l
        if b in order:
            order.remove(b)
        order.append(b)
    loaded = [(b, held[b]) for b in order]
    oc.finish_prefill(first, n_buf, loaded)
    # textbook: the decode residents that kept their slots (seeded order),
    # then the buffers' experts, least recently loaded first, ascending e
    od = OrderedDict((int(i), None) for i in pre_resident)
    for b, l in loaded:
        for e in range(E):
            od.pop(l * E + e, None)
            od[l * E + e] = None
    tb = TextbookLRU(C, [])
    tb.od = od
    return oc, tb, loaded


@pytest.mark.parametrize("seed", range(10))
def test_prefill_survivors_seed_the_lru(seed):
    rng = np.random.default_rng(400 + seed)
    E = int(rng.integers(2, 5))
    L = int(rng.integers(2, 6))
    n_buf = int(rng.integers(1, 4))
    C = n_buf * E + int(rng.integers(0, 5))
    run = int(rng.integers(0, L + 1))
    first = C - n_buf * E
    pre = list(rng.choice(L * E, size=min(first, L * E), replace=False))
    oc, tb, loaded = _prefill_then_textbook(rng, L, E, C, n_buf, run, pre)
    slot_id, ts, id_slot, _ = oc.tables()
    assert set(i for i in slot_id if i >= 0) == set(tb.od.keys())
    for b, l in loaded:                              # every held expert is resident
        for e in range(E):
            s = id_slot[l * E + e]
            assert s >= 0 and slot_id[s] == l * E + e
            assert s == first + b * E + e or s < first  # its buffer slot, or the decode slot it had
    assert not (slot_id == lru.RESERVED).any()
    for s, i in enumerate(slot_id):
        if i >= 0:
            assert id_slot[i] == s
    # the recency order the stamps give is the textbook's
    occ = sorted((int(ts[s]), s) for s in range(C) if slot_id[s] >= 0)
    assert [int(slot_id[s]) for _, s in occ] == list(tb.od.keys())
    # and decode from there behaves as the textbook LRU
    for layer, ids in _random_trace(rng, 80, L, E, 2, min(2, E)):
        r = oc.step(layer, ids, fill_all=True)
        uniq = sorted(set((layer * E + ids).reshape(-1).tolist()))
        hits, fills, host, evicted = tb.step(uniq, lambda m: m)
        assert (r.hits, r.fill_id, r.host_id, r.fill_evicted) == (hits, fills, host, evicted)


def test_prefill_survivor_already_resident_keeps_its_slot():
    """Worked by hand: slot 0 holds id 9 (layer 2, expert 1), slot 1 holds
    id 2 (layer 0, expert 2); buffers at slots 2-5 (layer 0) and 6-9
    (layer 2, loaded last)."""
    L, E, C = 3, 4, 10
    oc = lru.ExpertCache(L, E, C, 900, 475)
    oc.seed([9, 2])
    oc.reserve(2, 8)
    t0 = oc.tick
    oc.finish_prefill(2, 2, [(0, 0), (1, 2)])
    slot_id, ts, id_slot, tick = oc.tables()
    assert slot_id.tolist() == [9, 2, 0, 1, -1, 3, 8, -1, 10, 11]
    assert id_slot[2] == 1 and id_slot[9] == 0
    base = t0 << 16
    assert ts.tolist() == [base | 6, base | 3, base | 1, base | 2, 0, base | 4, base | 5, 0, base | 7, base | 8]
    assert tick == t0 + 1


def test_finish_with_nothing_loaded_releases_the_buffers():
    oc = lru.ExpertCache(2, 4, 9, 900, 475)
    oc.seed([5])
    oc.reserve(1, 8)
    oc.finish_prefill(1, 2, [])
    slot_id, ts, _, _ = oc.tables()
    assert slot_id.tolist() == [5] + [-1] * 8 and ts.tolist() == [1] + [0] * 8


# ---------------------------------------------------------------- resize at a safe point
@pytest.mark.parametrize("seed", range(12))
def test_resize_matches_textbook(seed):
    """Shrinking keeps the most recent residents that fit, growing adds room;
    the recency order survives, and steps after it agree with a textbook
    LRU of the new capacity holding the same entries in the same order."""
    rng = np.random.default_rng(500 + seed)
    L, E, T, k = 2, 5, 2, 2
    C = int(rng.integers(2, 9))
    oc = lru.ExpertCache(L, E, C, 1, 1)
    tb = TextbookLRU(C, [])
    for n_resize in range(4):
        for layer, ids in _random_trace(rng, 30, L, E, T, k):
            r = oc.step(layer, ids, fill_all=True)
            uniq = sorted(set((layer * E + ids).reshape(-1).tolist()))
            hits, fills, host, evicted = tb.step(uniq, lambda m: m)
            assert (r.hits, r.fill_id, r.host_id, r.fill_evicted) == (hits, fills, host, evicted)
        new_C = int(rng.integers(1, 10))
        moves = oc.resize(new_C)
        keys = list(tb.od.keys())
        tb = TextbookLRU(new_C, keys[max(0, len(keys) - new_C):])
        slot_id, ts, id_slot, _ = oc.tables()
        assert len(slot_id) == new_C
        occ = sorted((int(ts[s]), s) for s in range(new_C) if slot_id[s] >= 0)
        assert [int(slot_id[s]) for _, s in occ] == list(tb.od.keys())
        for s, i in enumerate(slot_id):
            if i >= 0:
                assert id_slot[i] == s
        assert (id_slot >= 0).sum() == (slot_id >= 0).sum()
        assert all(dst < new_C <= src for src, dst in moves)


def test_resize_by_hand():
    """Slots 0-5 hold ids 10..15 with recency 12 < 14 < 10 < 15 < 11 < 13
    (stamps 3, 5, 1, 6, 2, 4 in slot order); shrink to 3 keeps the three most
    recent: 15 (slot 5), 11 (slot 1), 13 (slot 3) -> 11 stays in slot 1,
    13 moves to slot 0, 15 to slot 2."""
    oc = lru.ExpertCache(2, 8, 6, 1, 1)
    oc.slot_id = [10, 11, 12, 13, 14, 15]
    oc.ts = [3, 5, 1, 6, 2, 4]
    oc.id_slot = [-1] * 16
    for s, i in enumerate(oc.slot_id):
        oc.id_slot[i] = s
    moves = oc.resize(3)
    assert moves == [(3, 0), (5, 2)]
    slot_id, ts, id_slot, _ = oc.tables()
    assert slot_id.tolist() == [13, 11, 15] and ts.tolist() == [6, 5, 4]
    moves = oc.resize(5)                             # grow: nothing moves, two empty slots
    assert moves == [] and oc.slot_id == [13, 11, 15, -1, -1] and oc.ts == [6, 5, 4, 0, 0]
    with pytest.raises(ValueError):
        oc.reserve(3, 2)
        oc.resize(4)
