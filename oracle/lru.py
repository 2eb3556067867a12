"""LRU expert-slot pool simulation, integer exact.  (Oracle: test infrastructure only.)

What the pages fix (explainer page, section "Inside llama.cpp PR #29887:
slot maps, banks, and only the misses cross PCIe"; its "The rules in the
code"; the T4 page, "What the MoE Cache Actually Caches"; the SGLang page,
"What happens with more than one request?"):

* a pool of K slots, each empty or holding one key; key = expert id for a
  per-layer pool, layer * E + expert for a pool shared by all layers;
* recency is a list of the slots, least recently used at the front;
* one plan serves one batch of routed ids: (1) the distinct keys, (2) every
  resident one is a hit and its slot moves to the most-recent end, (3) the
  distinct keys are sorted, (4) each non-resident key in that order takes
  the least recently used slot (evicting its key, if any), and that slot
  moves to the most-recent end; a plan with more distinct keys than slots
  is an error;
* stats: hits += hits of the plan, misses += fills, bytes += fills * block
  size, in the bucket for plans of at most 8 tokens (ids <= 8 * top_k) or
  the bucket for larger ones;
* a step is one wave when tokens * top_k <= K, otherwise several waves, each
  with its own plan and page-in.

Readings fixed here where the pages are silent:

* the distinct keys are listed in first-occurrence order over the ids taken
  token by token, pick by pick (rank order) before the sort;
* the initial recency list is slot 0 (front), 1, ..., K-1, all empty, so the
  lowest-numbered empty slot is taken first;
* waves are runs of floor(K / top_k) consecutive tokens in batch order; the
  optional union rule (a reader's comment under the SGLang page) instead
  closes a wave at the first token whose experts would make the wave's union
  exceed K;
* a hit is counted once per distinct key per plan;
* the optional LFU pool (LFUPool) keeps a use count per key that survives
  eviction and takes empty slots first, then the resident key of least
  (count, plan of last use, slot) that the plan does not name;
* the optional adaptive per-layer capacity (AdaptiveLRU) moves slots between
  per-layer LRU pools by window hit rate; its schedule is a reading, stated
  in its docstring;
* the optional two-tier store (RamTier) puts an LRU of pinned RAM blocks
  between a file of expert blocks and the uploads; its readings are in its
  docstring.

Two implementations that share nothing but the interface: ``LinkedListPool``
(doubly linked recency list) and ``TimestampPool`` (last-use stamps, victim =
argmin).
"""
import numpy as np


class PlanError(Exception):
    pass


class PlanResult:
    __slots__ = ("uniq", "hits", "fills", "evictions", "slot_of")

    def __init__(self):
        self.uniq = []        # distinct keys, first-occurrence order
        self.hits = []        # keys found resident, in uniq order
        self.fills = []       # (key, slot) in ascending key order
        self.evictions = []   # (evicted key, slot)
        self.slot_of = {}     # key -> slot after the plan

    def __repr__(self):
        return f"PlanResult(hits={self.hits}, fills={self.fills}, evictions={self.evictions})"


def distinct_first_occurrence(keys):
    seen, out = set(), []
    for k in keys:
        k = int(k)
        if k not in seen:
            seen.add(k)
            out.append(k)
    return out


class LinkedListPool:
    """K slots with a doubly linked recency list (front = least recently used)."""

    def __init__(self, n_slots):
        if n_slots <= 0:
            raise PlanError("pool needs at least one slot")
        self.n = n_slots
        self.prev = [s - 1 for s in range(n_slots)]
        self.next = [s + 1 if s + 1 < n_slots else -1 for s in range(n_slots)]
        self.front = 0
        self.back = n_slots - 1
        self.key_of = [-1] * n_slots
        self.where = {}

    def _to_back(self, s):
        if s == self.back:
            return
        p, n = self.prev[s], self.next[s]
        if p >= 0:
            self.next[p] = n
        else:
            self.front = n
        self.prev[n] = p
        self.prev[s] = self.back
        self.next[s] = -1
        self.next[self.back] = s
        self.back = s

    def resident(self, key):
        return key in self.where

    def order(self):
        """Slots from least to most recently used."""
        out, s = [], self.front
        while s >= 0:
            out.append(s)
            s = self.next[s]
        return out

    def plan(self, keys):
        res = PlanResult()
        res.uniq = distinct_first_occurrence(keys)
        if len(res.uniq) > self.n:
            raise PlanError(f"{len(res.uniq)} distinct experts for {self.n} slots")
        for k in res.uniq:
            s = self.where.get(k)
            if s is not None:
                self._to_back(s)
                res.hits.append(k)
        for k in sorted(res.uniq):
            if k in self.where:
                continue
            s = self.front
            old = self.key_of[s]
            if old >= 0:
                del self.where[old]
                res.evictions.append((old, s))
            self.key_of[s] = k
            self.where[k] = s
            self._to_back(s)
            res.fills.append((k, s))
        res.slot_of = {k: self.where[k] for k in res.uniq}
        return res


class TimestampPool:
    """K slots with last-use stamps; the victim is the slot with the oldest stamp."""

    def __init__(self, n_slots):
        if n_slots <= 0:
            raise PlanError("pool needs at least one slot")
        self.n = n_slots
        self.stamp = np.arange(n_slots, dtype=np.int64) - n_slots   # empty slots: older than any use
        self.clock = 0
        self.key_of = np.full(n_slots, -1, dtype=np.int64)

    def _use(self, s):
        self.stamp[s] = self.clock
        self.clock += 1

    def _slot(self, key):
        hit = np.nonzero(self.key_of == key)[0]
        return int(hit[0]) if hit.size else None

    def resident(self, key):
        return self._slot(key) is not None

    def order(self):
        return [int(s) for s in np.argsort(self.stamp, kind="stable")]

    def plan(self, keys):
        res = PlanResult()
        res.uniq = distinct_first_occurrence(keys)
        if len(res.uniq) > self.n:
            raise PlanError(f"{len(res.uniq)} distinct experts for {self.n} slots")
        for k in res.uniq:
            s = self._slot(k)
            if s is not None:
                self._use(s)
                res.hits.append(k)
        for k in sorted(res.uniq):
            if self._slot(k) is not None:
                continue
            s = int(np.argmin(self.stamp))
            old = int(self.key_of[s])
            if old >= 0:
                res.evictions.append((old, s))
            self.key_of[s] = k
            self._use(s)
            res.fills.append((k, s))
        res.slot_of = {k: self._slot(k) for k in res.uniq}
        return res


class LFUPool:
    """K slots evicting the least frequently used key (the 95 GiB page, "Decode": least
    frequently used eviction within each layer's pool; the explainer page's toy compares
    an LFU with the LRU).  The pages give no tie or ageing rule; the reading here:

    * every key has a use count that survives eviction, +1 per plan that names it;
    * a plan's fills take the empty slots first, lowest slot first, then the resident
      slots whose keys the plan does not name, by (count, plan of last use, slot);
    * hits and fills, the order of fills (ascending key) and errors are as in the LRU pool.

    The explainer's toy table prints LFU hit rates; this reading reproduces them where the
    toy routing has little locality, not at stickiness 0.7 (parity unpinned there).
    """

    def __init__(self, n_slots):
        if n_slots <= 0:
            raise PlanError("pool needs at least one slot")
        self.n = n_slots
        self.key_of = [-1] * n_slots
        self.last_use = [-1] * n_slots
        self.where = {}
        self.count = {}
        self.clock = 0

    def resident(self, key):
        return key in self.where

    def plan(self, keys):
        res = PlanResult()
        res.uniq = distinct_first_occurrence(keys)
        if len(res.uniq) > self.n:
            raise PlanError(f"{len(res.uniq)} distinct experts for {self.n} slots")
        named = set(res.uniq)
        for k in res.uniq:
            self.count[k] = self.count.get(k, 0) + 1
            if k in self.where:
                res.hits.append(k)
        empty = [s for s in range(self.n) if self.key_of[s] < 0]
        taken = sorted((s for s in range(self.n) if self.key_of[s] >= 0 and self.key_of[s] not in named),
                       key=lambda s: (self.count[self.key_of[s]], self.last_use[s], s))
        victims = empty + taken
        for i, k in enumerate(sorted(k for k in res.uniq if k not in self.where)):
            s = victims[i]
            old = self.key_of[s]
            if old >= 0:
                del self.where[old]
                res.evictions.append((old, s))
            self.key_of[s] = k
            self.where[k] = s
            res.fills.append((k, s))
        for k in res.uniq:
            self.last_use[self.where[k]] = self.clock
        self.clock += 1
        res.slot_of = {k: self.where[k] for k in res.uniq}
        return res


class AdaptiveLRU:
    """Per-layer LRU pools that trade capacity during decode (95 GiB page, "Decode": one
    pool per layer, because layers route differently; the layers share one total, and as
    decoding goes on capacity moves from layers whose hit rate is high to layers whose hit
    rate is low).  The page gives the idea, not the schedule; the readings here:

    * the total is L * K0 slots with global numbers, layer l starting with slots
      l*K0 .. l*K0+K0-1 (recency list in that order, all empty);
    * every `period` steps (a step begins with a decode call of layer 0) the layers with
      picks in the window since the last rebalance are ranked by pick hit rate (an exact
      ratio; ties by layer number); the i-th highest gives `delta` slots of target
      capacity to the i-th lowest, for i < `pairs`, while the giver's rate is strictly
      higher, the giver stays at or above `floor` and the taker at or below E;
    * capacity follows the targets lazily, inside a layer's next plan: a layer below its
      target first takes free slots, lowest first, placed in ascending order at the
      least-recently-used end; after the hits are refreshed, a layer above its target
      frees its least recently used slots (evicting their experts) but keeps as many
      slots as the plan's distinct experts; then the misses are filled as in LRU;
    * waves are sized by the layer's capacity min(slots held, target).
    """

    def __init__(self, n_experts, n_layers, slots_per_layer, period, delta, pairs, floor):
        if floor < 1 or period < 1 or delta < 0 or pairs < 0:
            raise ValueError("bad adaptive parameters")
        self.E, self.L, self.K0 = n_experts, n_layers, slots_per_layer
        self.period, self.delta, self.pairs, self.floor = period, delta, pairs, floor
        self.lists = [list(range(l * slots_per_layer, (l + 1) * slots_per_layer)) for l in range(n_layers)]
        self.key_of = [-1] * (n_layers * slots_per_layer)
        self.where = [dict() for _ in range(n_layers)]
        self.target = [slots_per_layer] * n_layers
        self.free = []
        self.window = [[0, 0] for _ in range(n_layers)]   # picks, pick hits
        self.steps = 0
        self.rebalances = 0

    def capacity(self, layer):
        return min(len(self.lists[layer]), self.target[layer])

    def resident(self, layer, key):
        return key in self.where[layer]

    def note(self, layer, picks, pick_hits):
        self.window[layer][0] += picks
        self.window[layer][1] += pick_hits

    def begin_step(self):
        if self.steps > 0 and self.steps % self.period == 0:
            self._rebalance()
        self.steps += 1

    def _rebalance(self):
        from fractions import Fraction
        rate = {l: Fraction(h, p) for l, (p, h) in enumerate(self.window) if p > 0}
        high = sorted(rate, key=lambda l: (-rate[l], l))
        low = sorted(rate, key=lambda l: (rate[l], l))
        for i in range(min(self.pairs, len(rate) // 2)):
            d, r = high[i], low[i]
            if rate[d] <= rate[r]:
                break
            if self.target[d] - self.delta < self.floor or self.target[r] + self.delta > self.E:
                continue
            self.target[d] -= self.delta
            self.target[r] += self.delta
        self.window = [[0, 0] for _ in range(self.L)]
        self.rebalances += 1

    def plan(self, layer, keys):
        order, where = self.lists[layer], self.where[layer]
        want = self.target[layer] - len(order)
        if want > 0 and self.free:
            taken = self.free[:want]
            del self.free[:want]
            order[:0] = taken
        res = PlanResult()
        res.uniq = distinct_first_occurrence(keys)
        if len(res.uniq) > len(order):
            raise PlanError(f"{len(res.uniq)} distinct experts for {len(order)} slots")
        for key in res.uniq:
            if key in where:
                order.remove(where[key])
                order.append(where[key])
                res.hits.append(key)
        extra = min(len(order) - self.target[layer], len(order) - len(res.uniq))
        for _ in range(max(extra, 0)):
            s = order.pop(0)
            old = self.key_of[s]
            if old >= 0:
                del where[old]
                self.key_of[s] = -1
                res.evictions.append((old, s))
            self.free.append(s)
        self.free.sort()
        for key in sorted(res.uniq):
            if key in where:
                continue
            s = order.pop(0)
            old = self.key_of[s]
            if old >= 0:
                del where[old]
                res.evictions.append((old, s))
            self.key_of[s] = key
            where[key] = s
            order.append(s)
            res.fills.append((key, s))
        res.slot_of = {key: where[key] for key in res.uniq}
        return res


def waves(n_tokens, top_k, n_slots):
    """Token ranges [(t0, t1)] of the waves of one step."""
    if n_tokens * top_k <= n_slots:
        return [(0, n_tokens)]
    w = n_slots // top_k
    if w == 0:
        raise PlanError(f"{n_slots} slots cannot hold the {top_k} experts of one token")
    return [(t, min(t + w, n_tokens)) for t in range(0, n_tokens, w)]


def waves_union(token_keys, n_slots):
    """Token ranges [(t0, t1)] of the waves of one step under the union rule: a wave takes
    the tokens in order while the union of their keys fits in the pool, and the next wave
    starts at the first token that would overflow it.  (SGLang page, "Comments": K // top_k
    tokens is a sizing guarantee, not the largest wave; tokens routed to overlapping experts
    need fewer slots than the sum of their top-k counts.)"""
    out = []
    t0, cur = 0, set()
    for t, ks in enumerate(token_keys):
        ks = set(int(k) for k in ks)
        if len(ks) > n_slots:
            raise PlanError(f"{n_slots} slots cannot hold the {len(ks)} experts of one token")
        if len(cur | ks) > n_slots:
            out.append((t0, t))
            t0, cur = t, ks
        else:
            cur |= ks
    if len(token_keys):
        out.append((t0, len(token_keys)))
    return out


class RamTier:
    """LRU of host RAM blocks between the file of expert blocks and the uploads.

    NVMe page, "Workflow": the experts are repacked into contiguous blocks read
    with pread, and an LRU cache of pinned RAM blocks (filled by reader threads)
    feeds the copies to the GPU.  Readings fixed here where the page is silent:

    * R blocks, keys layer * E + expert; "least recently used" is recency of use
      by the model: every expert a plan names makes its block, if present, the
      most recently used (a touch), whether or not it is uploaded;
    * an access (an upload from host memory) of a present key is a hit and a
      touch; an absent key is read into the least recently used block,
      evicting that block's key if it holds one;
    * order within a decode wave: the plan's hits (first-occurrence order) are
      touched, then its fills are accessed in the plan's fill order (ascending
      expert), a fill served from the staging bank being touched instead; a
      prefill call touches its resident experts, then accesses its uploads,
      both ascending;
    * a speculative copy reads a block only if it is present and changes no
      recency (a guess never causes a file read).
    """

    def __init__(self, n_blocks):
        if n_blocks < 1:
            raise ValueError("the RAM tier needs at least one block")
        self.R = n_blocks
        self.lru = []              # keys, least recently used first
        self.hits = self.misses = self.evictions = 0

    def present(self, key):
        return key in self.lru

    def touch(self, key):
        """A use that needs no read: a present key becomes the most recently used."""
        if key in self.lru:
            self.lru.remove(key)
            self.lru.append(key)

    def access(self, key):
        """Returns True for a hit."""
        if key in self.lru:
            self.lru.remove(key)
            self.lru.append(key)
            self.hits += 1
            return True
        if len(self.lru) == self.R:
            self.lru.pop(0)
            self.evictions += 1
        self.lru.append(key)
        self.misses += 1
        return False


class Stats:
    """Counters per bucket: 'small' (plans of <= 8 tokens), 'large', 'prefill'."""

    def __init__(self):
        self.b = {name: dict(hits=0, misses=0, picks=0, pick_hits=0, bytes_h2d=0, bytes_d2d=0,
                             evictions=0, plans=0, union_sum=0, union_max=0)
                  for name in ("small", "large", "prefill")}
        self.waves = 0
        self.steps = 0

    def add_plan(self, n_ids, top_k, res, picks, pick_hits, block_bytes):
        name = "small" if n_ids <= 8 * top_k else "large"
        d = self.b[name]
        d["hits"] += len(res.hits)
        d["misses"] += len(res.fills)
        d["bytes_h2d"] += len(res.fills) * block_bytes
        d["evictions"] += len(res.evictions)
        d["plans"] += 1
        d["picks"] += picks
        d["pick_hits"] += pick_hits
        d["union_sum"] += len(res.uniq)
        d["union_max"] = max(d["union_max"], len(res.uniq))


class CacheSim:
    """Replays routed ids through the pools of a cache (per-layer or shared)."""

    def __init__(self, n_experts, n_slots, top_k, n_layers, shared_pool=False, block_bytes=0,
                 pool_cls=LinkedListPool, wave_rule="count", policy="lru", adaptive=None, ram_blocks=None):
        self.E, self.K, self.k, self.L = n_experts, n_slots, top_k, n_layers
        # two-tier store: the uploads go through an LRU of RAM blocks fed from a file
        self.ram = RamTier(ram_blocks) if ram_blocks is not None else None
        self.shared = shared_pool
        if wave_rule not in ("count", "union"):
            raise ValueError(wave_rule)
        self.wave_rule = wave_rule
        self.block_bytes = block_bytes
        if top_k > n_slots:
            raise PlanError("cache too small: fewer slots than top_k")
        if policy not in ("lru", "lfu"):
            raise ValueError(policy)
        if policy == "lfu":
            pool_cls = LFUPool
        self.adaptive = None
        if adaptive is not None:
            # adaptive = dict(period, delta, pairs, floor): per-layer LRU pools trading capacity
            if shared_pool or policy != "lru":
                raise ValueError("adaptive capacity is defined for per-layer LRU pools")
            self.adaptive = AdaptiveLRU(n_experts, n_layers, n_slots, **adaptive)
            self.pools = None
        elif shared_pool:
            self.pools = [pool_cls(n_slots)]
        else:
            self.pools = [pool_cls(n_slots) for _ in range(n_layers)]
        self.stats = Stats()
        self.trace = []

    def pool(self, layer):
        return self.pools[0] if self.shared else self.pools[layer]

    def key(self, layer, expert):
        return layer * self.E + int(expert) if self.shared else int(expert)

    def expert_of(self, key):
        return key % self.E if self.shared else key

    def decode(self, layer, ids, step=None):
        """Plan one decode call of `layer`; ids [b, k].  Returns slots [b, k] and the wave records."""
        ids = np.asarray(ids)
        b = ids.shape[0]
        slots = np.full(ids.shape, -1, dtype=np.int64)
        ad = self.adaptive
        recs = []
        if ad is not None and layer == 0:
            ad.begin_step()
        cap = ad.capacity(layer) if ad is not None else self.K
        if self.wave_rule == "union":
            ranges = waves_union([[self.key(layer, e) for e in row] for row in ids], cap)
        else:
            ranges = waves(b, self.k, cap)
        for wi, (t0, t1) in enumerate(ranges):
            keys = [self.key(layer, e) for e in ids[t0:t1].reshape(-1)]
            if ad is not None:
                before = {k: ad.resident(layer, k) for k in set(keys)}
                res = ad.plan(layer, keys)
                ad.note(layer, len(keys), sum(1 for k in keys if before[k]))
            else:
                pool = self.pool(layer)
                before = {k: pool.resident(k) for k in set(keys)}
                res = pool.plan(keys)
            for t in range(t0, t1):
                for j in range(self.k):
                    slots[t, j] = res.slot_of[self.key(layer, ids[t, j])]
            pick_hits = sum(1 for k in keys if before[k])
            if self.ram is not None:
                for k in res.hits:
                    self.ram.touch(layer * self.E + self.expert_of(k))
                for k, _s in res.fills:
                    self.ram.access(layer * self.E + self.expert_of(k))
            self.stats.add_plan(len(keys), self.k, res, len(keys), pick_hits, self.block_bytes)
            self.stats.waves += 1
            rec = dict(step=step, layer=layer, wave=wi, t0=t0, t1=t1,
                       hits=[self.expert_of(k) for k in res.hits],
                       fills=[(self.expert_of(k), s) for k, s in res.fills],
                       evictions=[(k, s) for k, s in res.evictions])
            recs.append(rec)
            self.trace.append(rec)
        return slots, recs

    def prefill(self, layer, ids, batch=32):
        """Prefill plan: touched experts ascending, in batches; the pools are not changed.

        Returns [(batch of experts, resident flags)] and updates the prefill bucket
        (hits = experts served from a slot, misses = experts uploaded).
        """
        touched = sorted(set(int(e) for e in np.asarray(ids).reshape(-1)))
        if self.adaptive is not None:
            resident = lambda key: self.adaptive.resident(layer, key)
        else:
            resident = self.pool(layer).resident
        out = []
        d = self.stats.b["prefill"]
        for i in range(0, len(touched), batch):
            chunk = touched[i:i + batch]
            res = [resident(self.key(layer, e)) for e in chunk]
            out.append((chunk, res))
            n_res = sum(res)
            d["hits"] += n_res
            d["misses"] += len(chunk) - n_res
            d["bytes_d2d"] += n_res * self.block_bytes
            d["bytes_h2d"] += (len(chunk) - n_res) * self.block_bytes
        d["plans"] += 1
        d["union_sum"] += len(touched)
        d["union_max"] = max(d["union_max"], len(touched))
        if self.ram is not None:
            flags = [resident(self.key(layer, e)) for e in touched]
            for e, r in zip(touched, flags):
                if r:
                    self.ram.touch(layer * self.E + e)
            for e, r in zip(touched, flags):
                if not r:
                    self.ram.access(layer * self.E + e)
        return out


def coalesce(fills):
    """Runs of fills whose expert and slot both advance by one: [(expert0, slot0, n)].

    Fills are taken in the order the plan produced them (ascending expert).
    """
    runs = []
    for e, s in fills:
        if runs and e == runs[-1][0] + runs[-1][2] and s == runs[-1][1] + runs[-1][2]:
            e0, s0, n = runs[-1]
            runs[-1] = (e0, s0, n + 1)
        else:
            runs.append((e, s, 1))
    return runs
