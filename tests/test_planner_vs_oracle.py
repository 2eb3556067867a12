"""The library's host slot table (C++, libmoe_planner.so, no GPU) against the
oracle's LRU simulation: slots, hits, fills, evictions, waves, stats, bit-exact."""
import numpy as np
import pytest

import expert_offload_lru_amd as moe
from oracle import lru


def _sticky_ids(rng, b, k, E, prev, stick):
    out = np.empty((b, k), dtype=np.int32)
    for t in range(b):
        chosen = []
        while len(chosen) < k:
            if prev is not None and rng.random() < stick:
                e = int(prev[t][rng.integers(0, k)])
            else:
                e = int(min(E - 1, int(E * rng.random() ** 1.8)))
            if e not in chosen:
                chosen.append(e)
        out[t] = chosen
    return out


def _compare_run(E, K, k, L, b, steps, shared, seed, stick=0.7, union=False, lfu=False, adaptive=None,
                 layer_E=None):
    """adaptive: dict(period, delta, pairs, floor) or None; layer_E: experts each layer routes
    among (layers of different locality), default E for all."""
    rng = np.random.default_rng(seed)
    sim = lru.CacheSim(E, K, k, L, shared_pool=shared, block_bytes=1000, wave_rule="union" if union else "count",
                       policy="lfu" if lfu else "lru", adaptive=adaptive)
    flags = (moe.POOL_SHARED if shared else 0) | (moe.WAVES_UNION if union else 0) | (moe.POLICY_LFU if lfu else 0)
    flags |= moe.ADAPTIVE_CAPACITY if adaptive else 0
    pl = moe.Planner(E, K, k, L, flags=flags, block_bytes=1000)
    if adaptive:
        pl.set_adaptive(**adaptive)
    prev = [None] * L
    for step in range(steps):
        for layer in range(L):
            ids = _sticky_ids(rng, b, k, layer_E[layer] if layer_E else E, prev[layer], stick)
            prev[layer] = ids
            slots_o, recs_o = sim.decode(layer, ids, step)
            slots_c, recs_c = pl.decode(layer, ids)
            assert np.array_equal(slots_o, slots_c), (step, layer)
            assert len(recs_o) == len(recs_c)
            for ro, rc in zip(recs_o, recs_c):
                assert (ro["t0"], ro["t1"], ro["wave"]) == (rc["t0"], rc["t1"], rc["wave"])
                assert ro["hits"] == rc["hits"]
                assert ro["fills"] == rc["fills"]
                assert ro["evictions"] == rc["evictions"]
            if adaptive:
                ad = sim.adaptive
                assert pl.capacity(layer) == (len(ad.lists[layer]), ad.target[layer]), (step, layer)
                assert ad.lists[layer] == pl.order(layer)
            elif not lfu and (not shared or layer == 0):
                assert sim.pool(layer).order() == pl.order(layer)
    st = pl.stats()
    for name in ("small", "large"):
        o = sim.stats.b[name]
        c = st[name]
        for key in ("plans", "hits", "misses", "evictions", "picks", "pick_hits", "union_sum", "union_max"):
            assert o[key] == c[key], (name, key)
        assert c["bytes_h2d"] == o["bytes_h2d"]
    assert st["waves"] == sim.stats.waves
    return st


def test_tiny_single_layer():
    _compare_run(E=16, K=8, k=2, L=1, b=1, steps=64, shared=False, seed=1)


def test_per_layer_pools_batch_one():
    _compare_run(E=128, K=92, k=8, L=6, b=1, steps=40, shared=False, seed=2)


def test_batch_four_and_thirty_two_waves():
    _compare_run(E=128, K=92, k=8, L=3, b=4, steps=30, shared=False, seed=3)
    st = _compare_run(E=128, K=92, k=8, L=3, b=32, steps=20, shared=False, seed=4)
    assert st["large"]["plans"] == 3 * 20 * 3          # 3 waves per call


def test_shared_pool_across_48_layers():
    _compare_run(E=64, K=300, k=10, L=48, b=1, steps=6, shared=True, seed=5, stick=0.5)


def test_all_hit_all_miss_and_k_equals_topk():
    _compare_run(E=8, K=8, k=8, L=2, b=1, steps=10, shared=False, seed=6)        # all hits after the first
    _compare_run(E=200, K=10, k=10, L=2, b=1, steps=20, shared=False, seed=7, stick=0.0)
    _compare_run(E=12, K=3, k=3, L=1, b=5, steps=20, shared=False, seed=8)       # one token per wave


def test_adversarial_duplicates_across_tokens():
    rng = np.random.default_rng(9)
    E, K, k = 10, 6, 3
    sim = lru.CacheSim(E, K, k, 1)
    pl = moe.Planner(E, K, k, 1)
    for _ in range(100):
        base = rng.choice(E, k, replace=False)
        ids = np.stack([np.roll(base, int(rng.integers(0, k))) for _ in range(2)]).astype(np.int32)
        so, ro = sim.decode(0, ids)
        sc, rc = pl.decode(0, ids)
        assert np.array_equal(so, sc)
        assert [r["fills"] for r in ro] == [r["fills"] for r in rc]


def test_coalesced_runs_match_oracle():
    pl = moe.Planner(32, 16, 4, 1)
    pl.decode(0, np.array([[5, 6, 7, 9]], dtype=np.int32))
    assert pl.last_runs() == [tuple(r) for r in lru.coalesce([(5, 0), (6, 1), (7, 2), (9, 3)])] == [(5, 0, 3), (9, 3, 1)]


def test_errors_leave_state_unchanged():
    pl = moe.Planner(10, 4, 2, 2)
    pl.decode(0, np.array([[1, 2]], dtype=np.int32))
    before = pl.order(0)
    assert pl.decode_rc(0, np.array([[1, 12]], dtype=np.int32)) == moe.ERR_INVALID
    assert pl.decode_rc(0, np.array([[1, -1]], dtype=np.int32)) == moe.ERR_INVALID
    assert pl.decode_rc(5, np.array([[1, 2]], dtype=np.int32)) == moe.ERR_INVALID
    assert pl.order(0) == before
    with pytest.raises(moe.MoeError) as ei:
        moe.Planner(10, 1, 2, 1)
    assert ei.value.code == moe.ERR_CACHE_TOO_SMALL


def test_rollback_empties_filled_slots():
    pl = moe.Planner(10, 4, 2, 1)
    pl.decode(0, np.array([[3, 4]], dtype=np.int32))       # slots 0, 1
    pl.decode(0, np.array([[5, 6]], dtype=np.int32))       # slots 2, 3
    pl.rollback_last()
    # 5 and 6 are gone; their slots are least recently used, so the next misses take them first
    slots, recs = pl.decode(0, np.array([[7, 3]], dtype=np.int32))
    assert recs[0]["hits"] == [3]
    assert recs[0]["fills"][0][1] in (2, 3) and recs[0]["evictions"] == []


def test_prefill_lookup_matches_oracle_and_keeps_state():
    rng = np.random.default_rng(10)
    E, K, k = 128, 92, 8
    sim = lru.CacheSim(E, K, k, 1, block_bytes=5)
    pl = moe.Planner(E, K, k, 1, block_bytes=5)
    for _ in range(30):
        ids = np.stack([rng.choice(E, k, replace=False)]).astype(np.int32)
        sim.decode(0, ids)
        pl.decode(0, ids)
    order = pl.order(0)
    prompt = np.stack([rng.choice(E, k, replace=False) for _ in range(300)]).astype(np.int32)
    ex, sl = pl.prefill(0, prompt)
    batches = sim.prefill(0, prompt)
    assert ex == [e for b, _ in batches for e in b]
    assert [s >= 0 for s in sl] == [r for _, rs in batches for r in rs]
    assert pl.order(0) == order
    st = pl.stats()["prefill"]
    o = sim.stats.b["prefill"]
    assert (st["hits"], st["misses"], st["bytes_d2d"], st["bytes_h2d"]) == (o["hits"], o["misses"], o["bytes_d2d"],
                                                                           o["bytes_h2d"])


def test_union_waves_match_oracle():
    # b = 32 at K = 92: sticky routing makes the unions much smaller than 8 per token
    st_u = _compare_run(E=128, K=92, k=8, L=3, b=32, steps=20, shared=False, seed=4, union=True)
    st_c = _compare_run(E=128, K=92, k=8, L=3, b=32, steps=20, shared=False, seed=4)
    assert st_u["waves"] < st_c["waves"]
    _compare_run(E=40, K=12, k=4, L=2, b=9, steps=30, shared=False, seed=11, union=True)
    _compare_run(E=64, K=24, k=4, L=4, b=16, steps=12, shared=True, seed=12, union=True)


def test_union_waves_reject_bad_ids_and_unknown_flags():
    pl = moe.Planner(10, 4, 2, 1, flags=moe.WAVES_UNION)
    with pytest.raises(moe.MoeError):
        pl.decode(0, np.array([[0, 1], [2, 3], [4, 10]], dtype=np.int32))
    with pytest.raises(moe.MoeError):
        moe.Planner(10, 4, 2, 1, flags=0x100)


def test_lfu_policy_matches_oracle():
    _compare_run(E=16, K=8, k=2, L=1, b=1, steps=80, shared=False, seed=21, lfu=True)
    _compare_run(E=128, K=92, k=8, L=4, b=1, steps=40, shared=False, seed=22, lfu=True)
    _compare_run(E=128, K=92, k=8, L=2, b=4, steps=30, shared=False, seed=23, lfu=True)
    _compare_run(E=128, K=92, k=8, L=2, b=32, steps=10, shared=False, seed=24, lfu=True)
    _compare_run(E=128, K=92, k=8, L=2, b=32, steps=10, shared=False, seed=25, lfu=True, union=True)
    _compare_run(E=64, K=40, k=4, L=6, b=2, steps=20, shared=True, seed=26, lfu=True)


ADAPT = dict(period=3, delta=2, pairs=2, floor=10)


@pytest.mark.parametrize("b,union", [(1, False), (4, False), (12, False), (12, True)])
def test_adaptive_capacity_matches_oracle(b, union):
    """Adaptive per-layer capacity: layers routing among 12 .. 60 experts trade slots; slots,
    records, held and target counts and recency orders bit-exact, waves sized by capacity."""
    L = 5
    layer_E = [12 + 12 * l for l in range(L)]
    _compare_run(E=64, K=20, k=4, L=L, b=b, steps=40, shared=False, seed=40 + b + union, union=union,
                 adaptive=ADAPT, layer_E=layer_E)
    sim = lru.CacheSim(64, 20, 4, L, adaptive=ADAPT)
    rng = np.random.default_rng(40 + b + union)
    prev = [None] * L
    for step in range(40):
        for layer in range(L):
            prev[layer] = _sticky_ids(rng, b, 4, layer_E[layer], prev[layer], 0.7)
            sim.decode(layer, prev[layer], step)
    assert sim.adaptive.rebalances > 5 and sim.adaptive.target != [20] * L


def test_adaptive_capacity_rejects_shared_and_lfu():
    for fl in (moe.POOL_SHARED, moe.POLICY_LFU):
        with pytest.raises(RuntimeError):
            moe.Planner(16, 8, 2, 2, flags=moe.ADAPTIVE_CAPACITY | fl)
    pl = moe.Planner(16, 8, 2, 2)
    with pytest.raises(RuntimeError):
        pl.set_adaptive()
    pl = moe.Planner(16, 8, 2, 2, flags=moe.ADAPTIVE_CAPACITY)
    for bad in (dict(period=0), dict(delta=-1), dict(pairs=-1), dict(floor=1), dict(floor=9)):
        with pytest.raises(RuntimeError):
            pl.set_adaptive(**bad)
