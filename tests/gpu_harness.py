"""Test-side set-up of a cache on the GPU from seeded synthetic inputs, plus the
oracle replays the GPU tests compare against.  (Test infrastructure.)"""
import functools

import numpy as np
import torch

import expert_offload_lru_amd as moe
import synth
from oracle import ffn, formats, lru, route


def tol_ok(y, ref, rel=2e-3):
    """max |y - ref| <= rel * max |ref| (the stated output tolerance)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(y - ref))
    return err <= rel * scale, err, scale


class Model:
    """A cache plus its synthetic host store, router weights and shared experts."""

    def __init__(self, E, K, k, H, I, quant, L, flags=0, n_distinct=None, seed=11, shared_expert=False,
                 prefetch=False, adaptive=None):
        f = flags | (moe.SHARED_EXPERT if shared_expert else 0) | (moe.PREFETCH if prefetch else 0)
        f |= moe.ADAPTIVE_CAPACITY if adaptive else 0
        self.adaptive = adaptive
        self.E, self.K, self.k, self.H, self.I, self.quant, self.L = E, K, k, H, I, quant, L
        self.shared_pool = bool(flags & moe.POOL_SHARED)
        self.wave_rule = "union" if flags & moe.WAVES_UNION else "count"
        self.policy = "lfu" if flags & moe.POLICY_LFU else "lru"
        self.cache = moe.Cache(E, K, k, H, I, quant, L, f)
        if adaptive:
            self.cache.set_adaptive(**adaptive)
        self.S = S = self.cache.S
        self.M = n_distinct or L * E
        self.store = moe.HostBuffer(self.M * S)
        arr = self.store.numpy(shape=(self.M, S))
        keys = [(0, m) for m in range(self.M)] if n_distinct else [(l, e) for l in range(L) for e in range(E)]
        synth.fill_blocks(arr, seed, quant, H, I, keys)
        self.blocks = arr
        self.block_of = np.empty((L, E), dtype=np.int64)
        for l in range(L):
            for e in range(E):
                self.block_of[l, e] = synth.alias_index(l, e, E, self.M) if n_distinct else l * E + e
        for l in range(L):
            if n_distinct:
                self.cache.set_expert_ptrs(l, [self.store.ptr + int(self.block_of[l, e]) * S for e in range(E)])
            else:
                self.cache.set_layer(l, self.store.ptr + l * E * S)
        self.router_np = synth.router_weights(seed + 1, L, E, H)
        self.router = torch.from_numpy(self.router_np).cuda()
        self.shared_np = None
        self.shared = None
        if shared_expert:
            self.shared_np = synth.shared_expert_blocks(seed, L, quant, H, I)
            self.shared = torch.from_numpy(self.shared_np).cuda()
        self.records = []
        self.cache.set_trace(self.records.append)

    # -- GPU side ---------------------------------------------------------------------------
    def forward(self, layer, x, residual=False, prefetch=True):
        """x: cuda float32 [b, H] -> out cuda float32 [b, H]."""
        out = torch.empty_like(x)
        nxt = self.router[layer + 1] if (prefetch and layer + 1 < self.L) else None
        self.cache.forward(layer, x, x.shape[0], self.router[layer], out,
                           shared_w=self.shared[layer] if self.shared is not None else None,
                           next_router_w=nxt, residual=residual)
        return out

    # -- oracle side ------------------------------------------------------------------------
    @functools.lru_cache(maxsize=256)
    def _decoded(self, block):
        return formats.decode_expert(self.quant, self.blocks[block], self.H, self.I)

    def experts(self, layer, e):
        return self._decoded(int(self.block_of[layer, e]))

    def shared_weights(self, layer):
        if self.shared_np is None:
            return None
        return formats.decode_expert(self.quant, self.shared_np[layer], self.H, self.I)

    def oracle_sim(self):
        return lru.CacheSim(self.E, self.K, self.k, self.L, shared_pool=self.shared_pool, block_bytes=self.S,
                            wave_rule=self.wave_rule, policy=self.policy, adaptive=self.adaptive)

    def oracle_route(self, layer, x):
        return route.route(np.asarray(x, dtype=np.float64), self.router_np[layer], self.k)

    def oracle_y(self, layer, x, ids, gate):
        return ffn.moe_layer_given_routing(np.asarray(x, dtype=np.float64), np.asarray(ids), np.asarray(gate),
                                           self.experts, layer=layer, shared=self.shared_weights(layer))

    def close(self):
        self.cache.close()
        self.store.free()


def check_routing(model, layer, x_np, gpu_ids, gpu_gate):
    """Compare GPU routing with the oracle's; returns the oracle's (ids, gate) continued with the GPU's
    order where a near tie allowed it, and the count of near-tie deviations."""
    ids, gate, z, p = model.oracle_route(layer, x_np)
    gpu_ids = np.asarray(gpu_ids).reshape(ids.shape)
    dev = 0
    if not np.array_equal(ids, gpu_ids):
        amass = route.abs_mass(x_np, model.router_np[layer])
        assert route.ids_match_with_ties(ids, gpu_ids, z, amass), (layer, ids, gpu_ids)
        dev = int(np.sum(np.any(ids != gpu_ids, axis=1)))
        ids = gpu_ids
        gate = np.take_along_axis(p, ids, axis=1)
    gg = np.asarray(gpu_gate, dtype=np.float64).reshape(gate.shape)
    assert np.allclose(gg, gate, rtol=1e-5, atol=1e-7), (layer, gg, gate)
    return ids, gate, dev


def compare_records(oracle_recs, gpu_recs, where=""):
    assert len(oracle_recs) == len(gpu_recs), where
    for ro, rg in zip(oracle_recs, gpu_recs):
        assert (ro["t0"], ro["t1"]) == (rg["t0"], rg["t1"]), where
        assert ro["hits"] == rg["hits"], (where, ro["hits"], rg["hits"])
        assert ro["fills"] == [tuple(f) for f in rg["fills"]], (where, ro["fills"], rg["fills"])
        assert ro["evictions"] == [tuple(e) for e in rg["evictions"]], (where, ro["evictions"], rg["evictions"])


def check_stack_step(model, sim, step, cap, out, recs, check_y=lambda s, l: True):
    """Teacher-forced check of one moe_stack_forward call against the oracle.

    cap: float32 [L, b, H], the inputs the call wrote to layer_inputs; out: float32 [b, H];
    recs: the call's plan records.  Per layer: routing against the oracle's on that layer's
    input (near ties continued with the GPU's order), plan records and slots against the
    oracle's LRU `sim`, and where check_y(step, layer) the layer output (next layer's input
    minus this one's) within the stated tolerance.  Returns (near-tie deviations, worst
    max|err|/max|ref|, outputs checked)."""
    L = model.L
    by_layer = [[] for _ in range(L)]
    for r in recs:
        by_layer[r["layer"]].append(r)
    near, worst, n_y = 0, 0.0, 0
    for layer in range(L):
        rl = by_layer[layer]
        assert rl, (step, layer, "no plan record")
        x_np = np.asarray(cap[layer])
        gids = np.concatenate([np.array(r["ids"]) for r in rl])
        ggate = np.concatenate([np.array(r["gate"]) for r in rl])
        ids, gate, dev = check_routing(model, layer, x_np, gids, ggate)
        near += dev
        slots, orecs = sim.decode(layer, ids, step)
        compare_records(orecs, rl, where=(step, layer))
        gslots = np.concatenate([np.array(r["slots"]) for r in rl]).reshape(ids.shape)
        assert np.array_equal(gslots, slots), (step, layer)
        if check_y(step, layer):
            nxt = np.asarray(cap[layer + 1] if layer + 1 < L else out, dtype=np.float64)
            y_gpu = nxt - x_np.astype(np.float64)
            y_ref = model.oracle_y(layer, x_np, ids, gate)
            ok, err, scale = tol_ok(y_gpu, y_ref)
            worst = max(worst, err / scale)
            n_y += 1
            assert ok, (step, layer, err, scale)
    return near, worst, n_y
