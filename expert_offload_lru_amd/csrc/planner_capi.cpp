// C ABI of the host slot table alone (include/moe_planner.h).
#include <algorithm>
#include <new>
#include <string>

#include "errors.hpp"
#include "moe_planner.h"
#include "planner.hpp"

using moe::set_error;

struct moe_planner {
    moe::Planner pl;
    moe::WavePlan last;
    bool has_last = false;
    moe_planner(int E, int K, int k, int L, bool shared, size_t s, bool union_waves, bool lfu, bool adaptive)
        : pl(E, K, k, L, shared, s, union_waves, lfu, adaptive) {}
};

namespace {

void fill_bucket(const moe::BucketStats &b, moe_bucket_stats &o) {
    o.plans = b.plans;
    o.hits = b.hits;
    o.misses = b.misses;
    o.picks = b.picks;
    o.pick_hits = b.pick_hits;
    o.evictions = b.evictions;
    o.bytes_h2d = b.bytes_h2d;
    o.bytes_d2d = b.bytes_d2d;
    o.union_sum = b.union_sum;
    o.union_max = b.union_max;
}

}  // namespace

namespace moe {
// shared with the GPU library: record of one plan for a trace callback
void emit_trace(const WavePlan &p, int top_k, const int32_t *ids, const float *gate, moe_trace_fn fn, void *user) {
    if (!fn) return;
    std::vector<int32_t> fe(p.fills.size()), fs(p.fills.size()), es(p.evictions.size());
    std::vector<int64_t> ek(p.evictions.size());
    for (size_t i = 0; i < p.fills.size(); ++i) {
        fe[i] = p.fills[i].expert;
        fs[i] = p.fills[i].slot;
    }
    for (size_t i = 0; i < p.evictions.size(); ++i) {
        ek[i] = p.evictions[i].key;
        es[i] = p.evictions[i].slot;
    }
    moe_plan_record r;
    r.layer = p.layer;
    r.wave = p.wave;
    r.t0 = p.t0;
    r.t1 = p.t1;
    r.top_k = top_k;
    r.ids = ids + (size_t)p.t0 * top_k;
    r.gate = gate ? gate + (size_t)p.t0 * top_k : nullptr;
    r.slots = p.slots.data();
    r.n_hits = (int32_t)p.hits.size();
    r.hits = p.hits.data();
    r.n_fills = (int32_t)p.fills.size();
    r.fill_expert = fe.data();
    r.fill_slot = fs.data();
    r.n_evictions = (int32_t)p.evictions.size();
    r.evict_key = ek.data();
    r.evict_slot = es.data();
    fn(&r, user);
}

void planner_stats(const Planner &pl, moe_stats &o) {
    fill_bucket(pl.small, o.small);
    fill_bucket(pl.large, o.large);
    fill_bucket(pl.prefill, o.prefill);
    o.waves = pl.waves_total;
}
}  // namespace moe

extern "C" {

int moe_planner_create(int E, int K, int top_k, int n_layers, unsigned flags, size_t block_bytes,
                       moe_planner **out) {
    if (!out) return set_error(MOE_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (E <= 0 || K <= 0 || top_k <= 0 || n_layers <= 0 || top_k > E)
        return set_error(MOE_ERR_INVALID, "bad planner sizes");
    if (K < top_k) return set_error(MOE_ERR_CACHE_TOO_SMALL, "K < top_k: a token's picks cannot all be resident");
    if (flags & ~(MOE_POOL_SHARED | MOE_SHARED_EXPERT | MOE_PREFETCH | MOE_WAVES_UNION | MOE_POLICY_LFU |
                  MOE_ADAPTIVE_CAPACITY))
        return set_error(MOE_ERR_INVALID, "unknown flags");
    if ((flags & MOE_ADAPTIVE_CAPACITY) && (flags & (MOE_POOL_SHARED | MOE_POLICY_LFU)))
        return set_error(MOE_ERR_UNSUPPORTED, "adaptive capacity is defined for per-layer LRU pools");
    moe_planner *p = new (std::nothrow)
        moe_planner(E, K, top_k, n_layers, (flags & MOE_POOL_SHARED) != 0, block_bytes, (flags & MOE_WAVES_UNION) != 0,
                    (flags & MOE_POLICY_LFU) != 0, (flags & MOE_ADAPTIVE_CAPACITY) != 0);
    if (!p) return set_error(MOE_ERR_OOM, "planner allocation failed");
    *out = p;
    return MOE_OK;
}

void moe_planner_destroy(moe_planner *p) { delete p; }

int moe_planner_decode(moe_planner *p, int layer, const int32_t *ids, int n_tokens, int32_t *slots,
                       moe_trace_fn fn, void *user, int *n_waves_out) {
    if (!p || !ids || !slots || n_tokens < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (layer < 0 || layer >= p->pl.n_layers()) return set_error(MOE_ERR_INVALID, "layer out of range");
    std::vector<std::pair<int, int>> w;
    if (layer == 0) p->pl.begin_step();
    const int wrc = p->pl.waves(layer, n_tokens, ids, w);
    if (wrc == moe::PLAN_INVALID) return set_error(MOE_ERR_INVALID, "expert id out of range");
    if (wrc != moe::PLAN_OK) return set_error(MOE_ERR_CACHE_TOO_SMALL, "a token's experts do not fit in the slots");
    const int k = p->pl.top_k();
    for (size_t i = 0; i < w.size(); ++i) {
        int rc = p->pl.plan(layer, ids, w[i].first, w[i].second, (int)i, p->last);
        if (rc == moe::PLAN_INVALID) return set_error(MOE_ERR_INVALID, "expert id out of range");
        if (rc == moe::PLAN_TOO_SMALL) return set_error(MOE_ERR_CACHE_TOO_SMALL, "more distinct experts than slots");
        p->has_last = true;
        const int n_ids = (w[i].second - w[i].first) * k;
        p->pl.account(p->last, n_ids, p->last.pick_hits);
        std::copy(p->last.slots.begin(), p->last.slots.end(), slots + (size_t)w[i].first * k);
        moe::emit_trace(p->last, k, ids, nullptr, fn, user);
    }
    if (n_waves_out) *n_waves_out = (int)w.size();
    return MOE_OK;
}

int moe_planner_prefill(moe_planner *p, int layer, const int32_t *ids, int n_ids, int32_t *experts, int32_t *slots,
                        int *n_out) {
    if (!p || !ids || !experts || !slots || !n_out || n_ids < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
    std::vector<int32_t> e, s;
    if (p->pl.prefill_lookup(layer, ids, n_ids, e, s) != moe::PLAN_OK)
        return set_error(MOE_ERR_INVALID, "bad layer or expert id");
    int res = 0;
    for (size_t i = 0; i < e.size(); ++i) {
        experts[i] = e[i];
        slots[i] = s[i];
        res += s[i] >= 0;
    }
    p->pl.account_prefill(res, (int)e.size() - res, (int)e.size());
    *n_out = (int)e.size();
    return MOE_OK;
}

int moe_planner_order(const moe_planner *p, int layer, int32_t *order) {
    if (!p || !order || layer < 0 || layer >= p->pl.n_layers()) return set_error(MOE_ERR_INVALID, "bad arguments");
    std::vector<int> o = p->pl.pool(layer).order();
    std::copy(o.begin(), o.end(), order);
    return MOE_OK;
}

int moe_planner_last_runs(const moe_planner *p, int32_t *runs, int max_runs, int *n_out) {
    if (!p || !runs || !n_out) return set_error(MOE_ERR_INVALID, "bad arguments");
    int n = 0;
    if (p->has_last)
        for (const moe::Run &r : p->last.runs) {
            if (n >= max_runs) break;
            runs[3 * n] = r.expert;
            runs[3 * n + 1] = r.slot;
            runs[3 * n + 2] = r.n;
            ++n;
        }
    *n_out = n;
    return MOE_OK;
}

int moe_planner_rollback_last(moe_planner *p) {
    if (!p || !p->has_last) return set_error(MOE_ERR_INVALID, "no plan to roll back");
    p->pl.rollback(p->last);
    p->has_last = false;
    return MOE_OK;
}

int moe_planner_set_adaptive(moe_planner *p, int period, int delta, int pairs, int floor) {
    if (!p) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (!p->pl.adaptive()) return set_error(MOE_ERR_UNSUPPORTED, "the planner was created without adaptive capacity");
    if (p->pl.set_adaptive(period, delta, pairs, floor) != moe::PLAN_OK)
        return set_error(MOE_ERR_INVALID, "bad adaptive parameters");
    return MOE_OK;
}

int moe_planner_capacity(const moe_planner *p, int layer, int *held, int *target) {
    if (!p || !held || !target || layer < 0 || layer >= p->pl.n_layers())
        return set_error(MOE_ERR_INVALID, "bad arguments");
    *held = p->pl.held(layer);
    *target = p->pl.target(layer);
    return MOE_OK;
}

int moe_planner_stats(const moe_planner *p, moe_stats *out) {
    if (!p || !out) return set_error(MOE_ERR_INVALID, "bad arguments");
    *out = moe_stats();
    moe::planner_stats(p->pl, *out);
    return MOE_OK;
}

}  // extern "C"
