"""Pins of the expert-cache policy model (oracle/cache.py) against facts
fixed outside it: a textbook page-replacement count, the stack-distance
characterisation of LRU, LRU's inclusion property, closed forms at the
extreme cache sizes, and hand-worked slot tables for the call and preload
rules (QuarkStar README, "Running Models Larger Than Available Memory")."""
import numpy as np
import pytest

from oracle.cache import ExpertCacheModel

# The reference string of the LRU page-replacement example in Silberschatz,
# Galvin and Gagne, "Operating System Concepts" (chapter on virtual memory):
# with 3 frames LRU takes 12 page faults (FIFO 15, OPT 9).
TEXTBOOK = [7, 0, 1, 2, 0, 3, 0, 4, 2, 3, 0, 3, 2, 1, 2, 0, 1, 7, 0, 1]


def _run(seq, slots):
    m = ExpertCacheModel(slots)
    hits = [m.use((0, e)) for e in seq]
    return m, hits


def test_textbook_lru_fault_count():
    m, hits = _run(TEXTBOOK, 3)
    assert m.stats["misses"] == 12
    assert m.stats["hits"] == 8
    # every fault after the first three evicts
    assert m.stats["evictions"] == 12 - 3


def _stack_distance_hits(seq, slots):
    """A reference is an LRU hit with S slots iff the key was referenced
    before and fewer than S distinct other keys were referenced since."""
    out = []
    for t, x in enumerate(seq):
        prev = [i for i in range(t) if seq[i] == x]
        if not prev:
            out.append(False)
            continue
        between = set(seq[prev[-1] + 1:t])
        out.append(len(between) < slots)
    return out


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("slots", [1, 2, 3, 5, 8])
def test_stack_distance(seed, slots):
    rng = np.random.default_rng(seed)
    # Zipf-like reuse, as the routing workloads have
    seq = [int(x) for x in np.minimum(rng.zipf(1.3, 300), 40)]
    _, hits = _run(seq, slots)
    assert hits == _stack_distance_hits(seq, slots)


@pytest.mark.parametrize("seed", range(4))
def test_inclusion_property(seed):
    """LRU is a stack algorithm: what S slots hold, S + 1 slots hold too, at
    every point of any sequence, so hits never drop as the cache grows."""
    rng = np.random.default_rng(100 + seed)
    seq = [int(x) for x in rng.integers(0, 25, 400)]
    models = [ExpertCacheModel(s) for s in range(0, 12)]
    for e in seq:
        for m in models:
            m.use((0, e))
        sets = [set(m.where) for m in models]
        for a, b in zip(sets, sets[1:]):
            assert a <= b
    hits = [m.stats["hits"] for m in models]
    assert hits == sorted(hits)


def test_extreme_sizes():
    rng = np.random.default_rng(7)
    seq = [int(x) for x in rng.integers(0, 30, 200)]
    m0, h0 = _run(seq, 0)
    assert not any(h0) and m0.stats["admissions"] == 0
    distinct = len(set(seq))
    big, _ = _run(seq, distinct)
    assert big.stats["misses"] == distinct             # compulsory misses only
    assert big.stats["hits"] == len(seq) - distinct
    assert big.stats["evictions"] == 0
    one, h1 = _run(seq, 1)
    assert h1 == [t > 0 and seq[t - 1] == x for t, x in enumerate(seq)]


def test_call_uses_order_and_dedup():
    # 3 layers, layer 0 resident; T = 2 tokens, k = 2
    ids = np.array([[[5, 1], [1, 5]],       # layer 0: resident, no uses
                    [[3, 4], [4, 2]],       # layer 1: 3, 4, 2
                    [[6, 6], [0, 6]]])      # layer 2 (duplicate within a token too): 6, 0
    uses = ExpertCacheModel.call_uses(ids, layer0=0, resident_layers=1)
    assert uses == [(1, 3), (1, 4), (1, 2), (2, 6), (2, 0)]
    # a call starting at layer 2 of the same stack
    assert ExpertCacheModel.call_uses(ids[1:], layer0=2, resident_layers=1) == [(2, 3), (2, 4), (2, 2),
                                                                                (3, 6), (3, 0)]


def test_hand_worked_slot_table():
    m = ExpertCacheModel(3)
    m.call([[[3, 4]], [[3, 1]]], layer0=1, resident_layers=1)   # uses (1,3) (1,4) (2,3) (2,1)
    # free slots lowest first: (1,3)->0, (1,4)->1, (2,3)->2; then (2,1) evicts the LRU (1,3)
    assert m.table().tolist() == [[2, 1], [1, 4], [2, 3]]
    assert m.stats == {"hits": 0, "misses": 4, "admissions": 4, "evictions": 1, "preloaded": 0}
    m.call([[[4, 9]]], layer0=1, resident_layers=1)             # (1,4) hit, (1,9) evicts (2,3)
    assert m.table().tolist() == [[2, 1], [1, 4], [1, 9]]
    assert m.stats["hits"] == 1 and m.stats["evictions"] == 2


def test_preload_rules():
    m = ExpertCacheModel(3)
    m.preload([(1, 7), (1, 8), (1, 7), (2, 0), (2, 5)])   # the duplicate is skipped; (2,5) finds no slot
    assert m.table().tolist() == [[1, 7], [1, 8], [2, 0]]
    assert m.stats["preloaded"] == 3 and m.stats["misses"] == 0
    # the coldest preloaded, (2,0), is the least recent: a miss evicts it first
    m.use((3, 3))
    assert m.table().tolist() == [[1, 7], [1, 8], [3, 3]]
    m.use((3, 4))                                          # then (1,8), then (1,7)
    assert m.table().tolist() == [[1, 7], [3, 4], [3, 3]]
    # preload evicts nothing once full
    m.preload([(4, 1)])
    assert m.stats["preloaded"] == 3 and (4, 1) not in m.where
