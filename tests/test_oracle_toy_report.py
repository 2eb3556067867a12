"""Statistical pin of the oracle's LRU pool (the explainer page's toy table) and the
bus / preflight arithmetic pins (CPU)."""
import json
import os

import numpy as np
import pytest

from oracle import report, toy

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


@pytest.mark.slow
def test_toy_lru_table_within_one_point():
    tab = _load("toy_lru_table.json")
    E, k, n = tab["n_experts"], tab["top_k"], tab["n_tokens"]
    traces = {}
    worst = 0.0
    for stick, slots, lru_hit, lru_up, _lfu_hit, _lfu_up in tab["rows"]:
        rates, ups = [], []
        for seed in range(5):
            key = (stick, seed)
            if key not in traces:
                traces[key] = toy.sticky_trace(E, k, n, stick, seed)
            hits, misses = toy.replay_per_pick(traces[key], slots)
            rates.append(100.0 * hits / (hits + misses))
            ups.append(misses / n)
        mean = float(np.mean(rates))
        worst = max(worst, abs(mean - lru_hit))
        assert abs(mean - lru_hit) <= 1.0, (stick, slots, mean, lru_hit)
        assert abs(float(np.mean(ups)) - lru_up) <= 0.1, (stick, slots, np.mean(ups), lru_up)
    assert worst <= 1.0


def test_toy_router_shape():
    tr = toy.sticky_trace(512, 10, 50, 0.7, 0)
    assert all(len(p) == 10 and p == sorted(set(p)) and 0 <= p[0] and p[-1] < 512 for p in tr)


def test_napkin_matches_printed_output():
    g = _load("napkin.json")
    i, pr = g["inputs"], g["printed"]
    n = report.napkin(i["layers"], i["experts"], i["routed_per_token"], i["hidden"], i["inter"])
    assert round(n["params_per_expert"] / 1e6, 2) == pr["params_per_expert_M"]
    assert round(n["expert_mib"], 2) == pr["expert_mib"]
    assert n["n_experts_total"] == pr["n_experts_total"]
    assert round(n["all_experts_gib"], 1) == pr["all_experts_gib"]
    assert n["touched_per_token"] == pr["touched_per_token"]
    assert round(n["touched_mib"]) == pr["touched_mib"]
    for link in ("pcie4", "pcie5"):
        ms, tok = report.pcie_ms_per_token(n["touched_bytes"], pr[link]["gbs"])
        assert round(ms, 1) == pr[link]["ms"] and round(tok) == pr[link]["tok_s"]
    for line in pr["cache_lines"]:
        c = report.cache_line(n, line["cache_gib"], line["hit_rate"], 31.5)
        assert round(100 * c["fraction"], 1) == line["fraction_pct"]
        assert round(c["miss_mib"]) == line["miss_mib"]
        assert round(c["ms"], 1) == line["ms_pcie4"]
    # the 2,764,800-byte block of the NVMe page is this expert's size
    assert n["expert_bytes"] == 2764800


def test_preflight_matches_printed_output():
    g = _load("preflight.json")
    for c in g["cases"]:
        r = report.preflight(c["layers"], c["experts"], c["top_k"], c["expert_mb"], c["K"],
                             c["link_gbps"], c["tok_s"], g["kv_bytes_per_token"])
        p = c["printed"]
        assert round(r["slot_mb"]) == p["slot_mb"]
        assert round(r["kv_tokens"]) == p["kv_tokens"]
        assert r["batch_cap"] == p["batch_cap"]
        assert round(100 * r["random_miss"]) == p["random_miss_pct"]
        assert round(100 * r["max_miss"]) == p["max_miss_pct"]
        assert r["reuse_implied"] == {"reuse implied": True, "inconclusive": False}[p["verdict"]]


def test_toy_lfu_heap_replay_equals_pool():
    from oracle import lru
    for stick in (0.0, 0.4, 0.7):
        for slots in (7, 25, 60):
            tr = toy.sticky_trace(200, 10, 300, stick, 3)
            assert toy.replay_per_pick_lfu(tr, slots) == toy.replay_per_pick(tr, slots, pool_cls=lru.LFUPool)


def test_toy_lfu_table_popularity_cells():
    # The page prints LFU columns but not its LFU.  With counts that survive eviction (no
    # ageing) the replay lands within about a point where routing has little locality
    # (stickiness 0, and 0.4 up to 51 slots); at stickiness 0.4 with 102 or more slots and
    # at 0.7 it runs 1.2-5 points below the printed LFU, which must age its counts there;
    # those cells stay unpinned.
    tab = _load("toy_lru_table.json")
    E, k, n = tab["n_experts"], tab["top_k"], tab["n_tokens"]
    for stick, slots, _lh, _lu, lfu_hit, lfu_up in tab["rows"]:
        if not (stick == 0.0 or (stick == 0.4 and slots <= 51)):
            continue
        rates, ups = [], []
        for seed in range(5):
            h, m = toy.replay_per_pick_lfu(toy.sticky_trace(E, k, n, stick, seed), slots)
            rates.append(100.0 * h / (h + m))
            ups.append(m / n)
        assert abs(float(np.mean(rates)) - lfu_hit) <= 1.1, (stick, slots, np.mean(rates), lfu_hit)
        assert abs(float(np.mean(ups)) - lfu_up) <= 0.1, (stick, slots, np.mean(ups), lfu_up)
