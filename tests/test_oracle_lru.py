"""Pins of the oracle's LRU slot pools, waves and statistics (CPU)."""
import numpy as np
import pytest

from oracle import lru


@pytest.mark.parametrize("cls", [lru.LinkedListPool, lru.TimestampPool])
def test_hand_traced_sequence(cls):
    # K = 3, one token of two picks per plan; traced by hand:
    pool = cls(3)
    r = pool.plan([5, 2])                       # sorted misses 2, 5 -> empty slots 0, 1
    assert r.hits == [] and r.fills == [(2, 0), (5, 1)] and r.evictions == []
    assert pool.order() == [2, 0, 1]
    r = pool.plan([2, 7])                       # 2 hits (slot 0); 7 -> empty slot 2
    assert r.hits == [2] and r.fills == [(7, 2)] and r.evictions == []
    assert pool.order() == [1, 0, 2]
    r = pool.plan([5, 9])                       # 5 hits (slot 1); 9 evicts 2 from slot 0
    assert r.hits == [5] and r.fills == [(9, 0)] and r.evictions == [(2, 0)]
    assert pool.order() == [2, 1, 0]
    r = pool.plan([9, 2])                       # 9 hits; 2 evicts 7 from slot 2
    assert r.hits == [9] and r.fills == [(2, 2)] and r.evictions == [(7, 2)]
    assert pool.order() == [1, 0, 2]
    r = pool.plan([3, 1])                       # sorted 1, 3: 1 evicts 5 (slot 1), 3 evicts 9 (slot 0)
    assert r.hits == [] and r.fills == [(1, 1), (3, 0)] and r.evictions == [(5, 1), (9, 0)]
    assert r.slot_of == {3: 0, 1: 1}


@pytest.mark.parametrize("cls", [lru.LinkedListPool, lru.TimestampPool])
def test_hits_are_refreshed_before_any_eviction(cls):
    pool = cls(2)
    pool.plan([1, 2])                           # 1 -> slot 0, 2 -> slot 1; slot 0 is least recent
    r = pool.plan([3, 1])                       # 1 must survive: the victim is 2's slot
    assert r.hits == [1] and r.fills == [(3, 1)] and r.evictions == [(2, 1)]


@pytest.mark.parametrize("cls", [lru.LinkedListPool, lru.TimestampPool])
def test_duplicates_and_first_occurrence(cls):
    pool = cls(4)
    pool.plan([4])
    r = pool.plan([6, 4, 6, 5, 4])
    assert r.uniq == [6, 4, 5] and r.hits == [4]
    assert r.fills == [(5, 1), (6, 2)]          # sorted misses take slots in recency order


@pytest.mark.parametrize("cls", [lru.LinkedListPool, lru.TimestampPool])
def test_too_many_distinct_is_an_error(cls):
    with pytest.raises(lru.PlanError):
        cls(2).plan([1, 2, 3])


def _random_run(rng, E, K, n_plans, per_plan, sticky=0.7):
    prev = []
    out = []
    for _ in range(n_plans):
        n = int(rng.integers(1, per_plan + 1))
        keys = []
        for _ in range(n):
            if prev and rng.random() < sticky:
                keys.append(int(rng.choice(prev)))
            else:
                keys.append(int(rng.integers(0, E)))
        out.append(keys)
        prev = keys
    return out


def test_two_implementations_agree_on_random_traces():
    rng = np.random.default_rng(7)
    for trial in range(40):
        E = int(rng.integers(2, 64))
        K = int(rng.integers(1, E + 4))
        a, b = lru.LinkedListPool(K), lru.TimestampPool(K)
        for keys in _random_run(rng, E, K, 60, max(1, min(K, 12))):
            if len(set(keys)) > K:
                keys = keys[:K]
                keys = list(dict.fromkeys(keys))[:K]
            ra, rb = a.plan(keys), b.plan(keys)
            assert (ra.hits, ra.fills, ra.evictions, ra.slot_of) == (rb.hits, rb.fills, rb.evictions, rb.slot_of)
            assert a.order() == b.order()


def test_invariants_per_plan():
    rng = np.random.default_rng(8)
    pool = lru.LinkedListPool(16)
    for keys in _random_run(rng, 50, 16, 300, 10):
        r = pool.plan(keys)
        assert len(r.hits) + len(r.fills) == len(r.uniq)
        for s, k in enumerate(pool.key_of):
            if k >= 0:
                assert pool.where[k] == s
        for k, s in pool.where.items():
            assert pool.key_of[s] == k
        assert sorted(pool.order()) == list(range(16))
        assert [e for e, _ in r.fills] == sorted(e for e, _ in r.fills)


def test_enough_slots_means_misses_equal_first_touches():
    rng = np.random.default_rng(9)
    E = 40
    sim = lru.CacheSim(E, E, 4, n_layers=3, block_bytes=10)
    seen = set()
    first = 0
    for step in range(50):
        for layer in range(3):
            ids = np.stack([rng.choice(E, 4, replace=False) for _ in range(2)])
            for e in ids.reshape(-1):
                if (layer, int(e)) not in seen:
                    seen.add((layer, int(e)))
                    first += 1
            sim.decode(layer, ids, step)
    tot = sim.stats.b["small"]
    assert tot["misses"] == first and tot["evictions"] == 0
    # shared pool over all layers with L*E slots: same count
    sim2 = lru.CacheSim(E, 3 * E, 4, n_layers=3, shared_pool=True)
    rng = np.random.default_rng(9)
    for step in range(50):
        for layer in range(3):
            ids = np.stack([rng.choice(E, 4, replace=False) for _ in range(2)])
            sim2.decode(layer, ids, step)
    assert sim2.stats.b["small"]["misses"] == first


def test_waves():
    assert lru.waves(32, 8, 92) == [(0, 11), (11, 22), (22, 32)]
    assert lru.waves(4, 8, 92) == [(0, 4)]
    assert lru.waves(11, 8, 88) == [(0, 11)]
    assert lru.waves(12, 8, 88) == [(0, 11), (11, 12)]
    with pytest.raises(lru.PlanError):
        lru.waves(2, 8, 7)


def test_shared_pool_keys_and_cross_layer_eviction():
    sim = lru.CacheSim(n_experts=4, n_slots=2, top_k=1, n_layers=2, shared_pool=True)
    sim.decode(0, np.array([[3]]))           # key 3 -> slot 0
    sim.decode(1, np.array([[3]]))           # key 7 -> slot 1
    _, recs = sim.decode(1, np.array([[0]]))  # key 4 evicts layer 0's expert 3 (key 3)
    assert recs[0]["fills"] == [(0, 0)] and recs[0]["evictions"] == [(3, 0)]


def test_stats_buckets_and_union():
    sim = lru.CacheSim(n_experts=64, n_slots=64, top_k=2, n_layers=1, block_bytes=100)
    sim.decode(0, np.array([[1, 2]] * 8))     # 16 ids = 8 * top_k -> small
    sim.decode(0, np.array([[1, 3]] * 9))     # 18 ids -> large
    s, l = sim.stats.b["small"], sim.stats.b["large"]
    assert (s["plans"], s["misses"], s["hits"], s["bytes_h2d"], s["union_max"]) == (1, 2, 0, 200, 2)
    assert (l["plans"], l["misses"], l["hits"], l["picks"], l["pick_hits"]) == (1, 1, 1, 18, 9)


def test_coalesce():
    assert lru.coalesce([(2, 0), (3, 1), (4, 2), (7, 3), (9, 4), (10, 5)]) == [(2, 0, 3), (7, 3, 1), (9, 4, 2)]
    assert lru.coalesce([(1, 5), (2, 4)]) == [(1, 5, 1), (2, 4, 1)]
    assert lru.coalesce([]) == []


def test_prefill_plan_leaves_pools_alone():
    sim = lru.CacheSim(n_experts=70, n_slots=8, top_k=2, n_layers=1, block_bytes=1)
    sim.decode(0, np.array([[3, 40]]))
    before = sim.pools[0].order(), list(sim.pools[0].key_of)
    ids = np.array([[e, (e + 1) % 70] for e in range(0, 70, 2)])
    batches = sim.prefill(0, ids, batch=32)
    assert [len(b) for b, _ in batches] == [32, 32, 6]
    flat = [e for b, _ in batches for e in b]
    assert flat == sorted(set(ids.reshape(-1).tolist()))
    res = {e: r for b, rs in batches for e, r in zip(b, rs)}
    assert res[3] and res[40] and not res[4]
    assert (sim.pools[0].order(), list(sim.pools[0].key_of)) == before
    assert sim.stats.b["prefill"]["hits"] == 2 and sim.stats.b["prefill"]["misses"] == 68


def test_waves_union_hand_worked():
    # K = 4, top-2: tokens (0,1) (1,2) (0,2) (3,4) (4,3).  The first three share experts 0..2
    # (union 3 <= 4); adding (3,4) would make 5, so the second wave starts there.  The count rule
    # packs floor(4/2) = 2 tokens a wave: 3 waves.
    toks = [(0, 1), (1, 2), (0, 2), (3, 4), (4, 3)]
    assert lru.waves_union(toks, 4) == [(0, 3), (3, 5)]
    assert lru.waves(5, 2, 4) == [(0, 2), (2, 4), (4, 5)]
    assert lru.waves_union([], 4) == []
    with pytest.raises(lru.PlanError):
        lru.waves_union([(0, 1, 2)], 2)


def test_waves_union_properties():
    rng = np.random.default_rng(5)
    for trial in range(300):
        E = int(rng.integers(4, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        K = int(rng.integers(k, 3 * k + 6))
        b = int(rng.integers(1, 40))
        hot = rng.choice(E, size=min(E, k + int(rng.integers(0, 6))), replace=False)
        toks = [rng.choice(hot if rng.random() < 0.7 and len(hot) >= k else E, size=k, replace=False)
                for _ in range(b)]
        w = lru.waves_union(toks, K)
        # contiguous, in order, covering every token
        assert w[0][0] == 0 and w[-1][1] == b and all(w[i][1] == w[i + 1][0] for i in range(len(w) - 1))
        for t0, t1 in w:
            assert t1 > t0
            assert len(set(int(e) for t in range(t0, t1) for e in toks[t])) <= K       # fits
            if t1 < b:                                                               # maximal
                assert len(set(int(e) for t in range(t0, t1 + 1) for e in toks[t])) > K
        # never more waves than the count rule; one wave whenever b * k <= K
        assert len(w) <= len(lru.waves(b, k, K))
        if b * k <= K:
            assert w == [(0, b)]


def test_waves_union_equals_count_rule_on_disjoint_tokens():
    # tokens with pairwise disjoint experts: every union is k per token, so the greedy
    # rule packs exactly floor(K / k) tokens a wave, as the count rule does
    for k, K, b in ((2, 7, 9), (8, 92, 32), (3, 9, 10), (1, 5, 12)):
        toks = [tuple(range(t * k, (t + 1) * k)) for t in range(b)]
        assert lru.waves_union(toks, K) == lru.waves(b, k, K)


def test_cachesim_union_rule_plans_each_wave_within_the_pool():
    rng = np.random.default_rng(9)
    E, k, K, b = 32, 4, 10, 16
    ids = np.stack([rng.choice(E // 2, size=k, replace=False) for _ in range(b)])
    for rule, n_expected in (("count", len(lru.waves(b, k, K))), ("union", None)):
        sim = lru.CacheSim(E, K, k, 1, wave_rule=rule)
        slots, recs = sim.decode(0, ids)
        assert (slots >= 0).all()
        if n_expected is not None:
            assert len(recs) == n_expected
        for r in recs:
            assert len(r["hits"]) + len(r["fills"]) <= K
    assert len(recs) <= len(lru.waves(b, k, K))


def test_lfu_pool_hand_traced():
    # K = 3.  Counts survive eviction; victims by (count, plan of last use, slot).
    p = lru.LFUPool(3)
    r = p.plan([1, 2]);  assert r.fills == [(1, 0), (2, 1)] and r.evictions == []
    r = p.plan([1]);     assert r.hits == [1] and r.fills == []          # count(1) = 2
    r = p.plan([3]);     assert r.fills == [(3, 2)]                      # the last empty slot
    # residents 1 (count 2), 2 (count 1, used in plan 0), 3 (count 1, plan 2): 2 goes
    r = p.plan([4]);     assert r.fills == [(4, 1)] and r.evictions == [(2, 1)]
    # 2 comes back with count 2; 5 is new.  Candidates 3 (1, plan 2), 4 (1, plan 3), 1 (2, plan 1):
    # the ascending misses 2, 5 take the slots of 3 and then 4
    r = p.plan([2, 5]);  assert r.fills == [(2, 2), (5, 1)] and r.evictions == [(3, 2), (4, 1)]
    # candidates 1 (2, plan 1), 2 (2, plan 4), 5 (1, plan 4): the least frequent, 5, goes
    r = p.plan([6]);     assert r.fills == [(6, 1)] and r.evictions == [(5, 1)]
    with pytest.raises(lru.PlanError):
        p.plan([7, 8, 9, 10])


def test_lfu_pool_never_evicts_a_named_key_and_fills_room_first():
    rng = np.random.default_rng(17)
    for trial in range(50):
        K = int(rng.integers(2, 12))
        p = lru.LFUPool(K)
        seen = set()
        for step in range(60):
            n = int(rng.integers(1, K + 1))
            keys = [int(x) for x in rng.choice(3 * K, size=n)]
            r = p.plan(keys)
            uniq = lru.distinct_first_occurrence(keys)
            assert all(p.resident(k) for k in uniq)                        # the plan's keys all stay
            assert sorted(r.hits + [k for k, _ in r.fills]) == sorted(uniq)
            assert not any(k in uniq for k, _ in r.evictions)
            if len(seen | set(uniq)) <= K:                                 # room: no evictions
                assert r.evictions == []
            seen |= set(uniq)
            assert sorted(p.where.values()) == sorted(set(p.where.values()))   # one key per slot


def test_cachesim_lfu_policy_equals_lru_when_everything_fits():
    rng = np.random.default_rng(21)
    ids = np.stack([rng.choice(12, size=3, replace=False) for _ in range(40)])
    a = lru.CacheSim(12, 12, 3, 1, policy="lfu")
    b = lru.CacheSim(12, 12, 3, 1)
    for t in range(40):
        ra = a.decode(0, ids[t:t + 1])[1][0]
        rb = b.decode(0, ids[t:t + 1])[1][0]
        assert ra["hits"] == rb["hits"] and ra["fills"] == rb["fills"] and ra["evictions"] == []


# --- adaptive per-layer capacity (95 GiB page, "Decode") ------------------------------------

def _adaptive_sim(E, K0, k, L, **ad):
    return lru.CacheSim(E, K0, k, L, adaptive=ad)


def test_adaptive_hand_traced_two_layers():
    """Two layers of 3 slots (global slots 0-2 and 3-5), top-1, a rebalance every 2 steps,
    one slot per move, floor 2.  Worked by hand from the stated rule."""
    sim = _adaptive_sim(8, 3, 1, 2, period=2, delta=1, pairs=1, floor=2)
    ad = sim.adaptive
    rec = lambda step, l, e: sim.decode(l, [[e]], step)[1][0]
    r = rec(0, 0, 0); assert r["fills"] == [(0, 0)] and r["evictions"] == []
    r = rec(0, 1, 0); assert r["fills"] == [(0, 3)]
    r = rec(1, 0, 0); assert r["hits"] == [0] and r["fills"] == []
    r = rec(1, 1, 1); assert r["fills"] == [(1, 4)]
    # step 2 opens with a rebalance: layer 0 hit 1 of 2 picks, layer 1 hit 0 of 2
    r = rec(2, 0, 0)
    assert ad.target == [2, 4] and ad.rebalances == 1
    assert r["hits"] == [0] and r["fills"] == [] and r["evictions"] == []
    assert ad.lists[0] == [2, 0] and ad.free == [1]           # empty slot 1 released
    r = rec(2, 1, 2)
    assert r["fills"] == [(2, 1)]                             # layer 1 takes slot 1 first
    assert ad.lists[1] == [5, 3, 4, 1] and ad.free == []
    r = rec(3, 0, 5); assert r["fills"] == [(5, 2)] and ad.lists[0] == [0, 2]
    r = rec(3, 1, 6); assert r["fills"] == [(6, 5)]
    # step 4: the same ranking, but layer 0 would drop below the floor: no move
    r = rec(4, 0, 0)
    assert ad.target == [2, 4] and ad.rebalances == 2 and r["hits"] == [0]
    # a full layer above its target evicts its least recently used expert to shrink
    ad.target = [1, 5]
    r = rec(5, 0, 0)
    assert r["hits"] == [0] and r["evictions"] == [(5, 2)] and ad.lists[0] == [0] and ad.free == [2]


def test_adaptive_without_moves_is_per_layer_lru():
    rng = np.random.default_rng(7)
    E, K, k, L = 24, 10, 3, 4
    plain = lru.CacheSim(E, K, k, L)
    for ad in (dict(period=1, delta=0, pairs=2, floor=3), dict(period=3, delta=2, pairs=0, floor=3)):
        sim = _adaptive_sim(E, K, k, L, **ad)
        ref = lru.CacheSim(E, K, k, L)
        for step in range(30):
            for l in range(L):
                ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(int(rng.integers(1, 6)))])
                s1, r1 = sim.decode(l, ids, step)
                s0, r0 = ref.decode(l, ids, step)
                # global slot numbers: layer l's pool starts at l*K
                assert np.array_equal(s1, s0 + l * K)
                for a, b in zip(r1, r0):
                    assert a["hits"] == b["hits"]
                    assert a["fills"] == [(e, s + l * K) for e, s in b["fills"]]
                    assert a["evictions"] == [(key, s + l * K) for key, s in b["evictions"]]
    del plain


def test_adaptive_invariants_random():
    rng = np.random.default_rng(11)
    E, K0, k, L = 32, 12, 4, 6
    sim = _adaptive_sim(E, K0, k, L, period=2, delta=2, pairs=2, floor=6)
    ad = sim.adaptive
    # layers of different locality: layer l routes among 6 + 5*l experts
    for step in range(80):
        for l in range(L):
            pool = 6 + 5 * l
            b = int(rng.integers(1, 4))
            ids = np.stack([rng.choice(pool, size=k, replace=False) for _ in range(b)])
            sim.decode(l, ids, step)
            held = [s for lst in ad.lists for s in lst]
            assert sorted(held + ad.free) == list(range(L * K0))          # slots conserved
            assert sum(ad.target) == L * K0 and min(ad.target) >= 6 and max(ad.target) <= E
            assert all(ad.key_of[s] == -1 for s in ad.free)
            for li in range(L):
                assert len(ad.where[li]) <= len(ad.lists[li])
                for key, s in ad.where[li].items():
                    assert ad.key_of[s] == key and s in ad.lists[li]
    assert ad.target[0] < K0 < ad.target[-1]          # capacity went from local to diffuse layers


# ----------------------------------------------------------------------------- RAM tier (two-tier store)

def test_ram_tier_hand_traced():
    # R = 3: 5 M, 7 M, 5 H, 9 M, 11 M (evicts 7, the least recent), 7 M (evicts 5), 9 H
    t = lru.RamTier(3)
    got = [t.access(k) for k in (5, 7, 5, 9, 11, 7, 9)]
    assert got == [False, False, True, False, False, False, True]
    assert (t.hits, t.misses, t.evictions) == (2, 5, 2)
    assert t.lru == [11, 7, 9]


def test_ram_tier_matches_the_stack_distance_rule():
    """LRU's inclusion property: an access hits iff its key was seen before and fewer than R
    distinct other keys were accessed since its previous access (brute force over the history)."""
    rng = np.random.default_rng(51)
    for R in (1, 2, 5, 16):
        seq = rng.integers(0, 24, size=400)
        t = lru.RamTier(R)
        for i, k in enumerate(seq):
            prev = [j for j in range(i) if seq[j] == k]
            want = bool(prev) and len(set(seq[prev[-1] + 1:i].tolist()) - {k}) < R
            assert t.access(int(k)) == want, (R, i)
        assert t.hits + t.misses == len(seq) and t.evictions == max(0, t.misses - R)


def test_cachesim_ram_tier_sees_every_upload():
    """Each demand upload (a fill, or a prefill batch's upload) is one RAM access; with room for
    every key the RAM misses are the distinct keys ever uploaded."""
    rng = np.random.default_rng(52)
    E, K, k, L = 32, 8, 2, 3
    for R, shared in ((8, False), (1000, False), (12, True)):
        sim = lru.CacheSim(E, 3 * K if shared else K, k, L, shared_pool=shared, ram_blocks=R)
        uploaded = set()
        n_up = 0
        for step in range(30):
            for layer in range(L):
                ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(int(rng.integers(1, 9)))])
                _slots, recs = sim.decode(layer, ids, step)
                for r in recs:
                    n_up += len(r["fills"])
                    uploaded |= {layer * E + e for e, _s in r["fills"]}
            if step % 10 == 9:
                for batch, res in sim.prefill(0, rng.integers(0, E, size=40)):
                    ups = [e for e, rr in zip(batch, res) if not rr]
                    n_up += len(ups)
                    uploaded |= set(ups)
        assert sim.ram.hits + sim.ram.misses == n_up
        if R >= L * E:
            assert sim.ram.misses == len(uploaded) and sim.ram.evictions == 0
        else:
            assert sim.ram.misses >= len(uploaded) and sim.ram.evictions == sim.ram.misses - R


def test_ram_tier_recency_follows_use():
    """A block the slots keep hitting stays recent in RAM: R = 2, keys 1 and 2 read, key 1 used
    (touched) again, then key 3 read evicts key 2, not key 1.  A touch of an absent key reads
    nothing."""
    t = lru.RamTier(2)
    t.access(1)
    t.access(2)
    t.touch(1)
    t.touch(9)
    assert not t.present(9)
    t.access(3)
    assert t.lru == [1, 3] and (t.hits, t.misses, t.evictions) == (0, 3, 1)


def test_cachesim_ram_tier_keeps_what_the_slots_use():
    """Per-layer pool of K = 2, RAM of 3 blocks, one layer: expert 0 is hit every call while the
    other picks cycle, so its block stays in RAM (touched by every hit) and a later upload of it
    is a RAM hit."""
    sim = lru.CacheSim(8, 2, 1, 1, ram_blocks=3)
    for e in (0, 1, 0, 2, 0, 3, 0, 4):
        sim.decode(0, np.array([[e]]))
    # slots: 0 stays resident (hit on every other call), 1..4 rotate through the other slot
    assert sim.ram.misses == 5 and sim.ram.hits == 0
    assert 0 in sim.ram.lru
    sim2 = lru.CacheSim(8, 2, 2, 1, ram_blocks=3)
    sim2.decode(0, np.array([[0, 1]]))
    sim2.decode(0, np.array([[2, 3]]))        # evicts 0 and 1 from the slots; RAM evicts 0
    sim2.decode(0, np.array([[0, 2]]))        # 2 hits in the slots (touched), 0 read again
    assert (sim2.ram.hits, sim2.ram.misses, sim2.ram.evictions) == (0, 5, 2)
    sim2.decode(0, np.array([[3, 2]]))        # 3 uploaded again: still in RAM
    assert sim2.ram.hits == 1
