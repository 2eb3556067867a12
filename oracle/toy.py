"""The explainer page's toy: a sticky fake router replayed pick by pick through an LRU.

Explainer page, section "How MoE expert offloading works with an LRU expert
cache": a fake router over 512 experts with 10 picks per token; with
probability "stickiness" a pick repeats one of the previous token's
experts (chosen uniformly), otherwise it draws expert
min(E - 1, floor(u^1.8 * E)) for a uniform u (so low ids are popular); a
token's picks are distinct and sorted.  The page replays 4000 tokens
through an LRU of 5/10/20/40 % of the experts, one pick at a time (a hit
refreshes the expert, a miss evicts the least recently used when full), and
prints hit rates and uploads per token.  Here the per-pick replay runs on
this oracle's own slot pool (a one-key plan per pick), so the printed table
is a statistical pin of the pool.  (Oracle: test infrastructure only.)
"""
import heapq

import numpy as np

from .lru import LinkedListPool


def _token_picks(rng, n_experts, k, prev, stickiness):
    """One token of the toy router: draws are made until k distinct experts are held.  A
    draw repeats a uniformly chosen expert of the previous token with probability
    `stickiness` (only when there is a previous token), else it is the power-law expert
    floor(E * u^1.8) of a uniform u, capped at E - 1.  Returned in ascending order."""
    held = np.zeros(n_experts, dtype=bool)
    n_held = 0
    while n_held < k:
        from_prev = len(prev) > 0 and rng.random() < stickiness
        e = prev[rng.integers(len(prev))] if from_prev else min(n_experts - 1, int(n_experts * rng.random() ** 1.8))
        if not held[e]:
            held[e] = True
            n_held += 1
    return np.flatnonzero(held).tolist()


def sticky_trace(n_experts, k, n_tokens, stickiness, seed):
    """n_tokens tokens of the toy router, each token's picks conditioned on the previous
    token's (PCG64 stream of `seed`)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    trace = []
    for _ in range(n_tokens):
        trace.append(_token_picks(rng, n_experts, k, trace[-1] if trace else [], stickiness))
    return trace


def replay_per_pick(trace, n_slots, pool_cls=LinkedListPool):
    """(hits, misses) of a per-pick LRU replay on the oracle's pool."""
    pool = pool_cls(n_slots)
    hits = misses = 0
    for picks in trace:
        for e in picks:
            res = pool.plan([e])
            if res.hits:
                hits += 1
            else:
                misses += 1
    return hits, misses


def replay_per_pick_lfu(trace, n_slots):
    """(hits, misses) of a per-pick replay under the LFU pool's rules (oracle.lru.LFUPool:
    counts survive eviction; a miss takes the lowest empty slot, else evicts the resident key
    of least (count, last use, slot)), kept in a heap so that 4000-token traces replay in
    well under a second.  Tests check it against LFUPool pick by pick on shorter traces."""
    count, where, heap = {}, {}, []
    free = list(range(n_slots))          # ascending: heapq pops the lowest empty slot
    last = [-1] * n_slots
    hits = misses = 0
    t = 0
    for picks in trace:
        for e in picks:
            count[e] = count.get(e, 0) + 1
            if e in where:
                hits += 1
                s = where[e]
            else:
                misses += 1
                if free:
                    s = heapq.heappop(free)
                else:
                    while True:             # skip entries made stale by a later use
                        c, lu, s, k = heapq.heappop(heap)
                        if where.get(k) == s and count[k] == c and last[s] == lu:
                            break
                    del where[k]
                where[e] = s
            last[s] = t
            heapq.heappush(heap, (count[e], t, s, e))
            t += 1
    return hits, misses
