// Host-side slot table of the expert cache (see planner.hpp for the method
// and the pages it follows).
#include "planner.hpp"

#include <algorithm>

namespace moe {

// ----------------------------------------------------------------------------- SlotPool

SlotPool::SlotPool(int n_slots)
    : n_(n_slots), link_next_(n_slots + 1), link_prev_(n_slots + 1), key_(n_slots, -1) {
    // circular list sentinel(n) -> 0 -> 1 -> ... -> n-1 -> sentinel
    for (int i = 0; i <= n_; ++i) {
        link_next_[i] = (i == n_) ? 0 : i + 1;
        link_prev_[i] = (i == 0) ? n_ : i - 1;
    }
    if (n_ == 0) {
        link_next_[0] = link_prev_[0] = 0;
    } else {
        link_next_[n_ - 1] = n_;
        link_prev_[n_] = n_ - 1;
    }
}

void SlotPool::unlink(int s) {
    link_next_[link_prev_[s]] = link_next_[s];
    link_prev_[link_next_[s]] = link_prev_[s];
}

void SlotPool::insert_before(int s, int pos) {
    int p = link_prev_[pos];
    link_next_[p] = s;
    link_prev_[s] = p;
    link_next_[s] = pos;
    link_prev_[pos] = s;
}

void SlotPool::refresh(int s) {
    if (link_prev_[n_] == s) return;     // already most recent
    unlink(s);
    insert_before(s, n_);                // just before the sentinel = most recent end
}

void SlotPool::demote(int s) {
    unlink(s);
    insert_before(s, link_next_[n_]);    // right after the sentinel = least recent end
}

std::vector<int> SlotPool::order() const {
    std::vector<int> out;
    for (int s = link_next_[n_]; s != n_; s = link_next_[s]) out.push_back(s);
    return out;
}

// ----------------------------------------------------------------------------- Planner

Planner::Planner(int n_experts, int n_slots, int top_k, int n_layers, bool shared_pool, size_t block_bytes,
                 bool union_waves, bool lfu)
    : E_(n_experts), K_(n_slots), k_(top_k), L_(n_layers), shared_(shared_pool), block_bytes_(block_bytes),
      slot_map_((size_t)n_layers * n_experts, -1), seen_(n_experts, 0), wave_mark_(n_experts, 0) {
    union_waves_ = union_waves;
    lfu_ = lfu;
    if (lfu_) {
        counts_.assign((size_t)n_layers * n_experts, 0);
        last_use_.assign(shared_pool ? 1 : n_layers, std::vector<int64_t>(n_slots, -1));
        clock_.assign(shared_pool ? 1 : n_layers, 0);
    }
    int n_pools = shared_ ? 1 : L_;
    pools_.reserve(n_pools);
    for (int i = 0; i < n_pools; ++i) pools_.emplace_back(K_);
}

int Planner::waves(int n_tokens, const int32_t *ids, std::vector<std::pair<int, int>> &out) {
    out.clear();
    if (n_tokens <= 0) return PLAN_OK;
    if ((long long)n_tokens * k_ <= K_) {
        out.emplace_back(0, n_tokens);
        return PLAN_OK;
    }
    if (!union_waves_) {
        int per = K_ / k_;
        if (per <= 0) return PLAN_TOO_SMALL;
        for (int t = 0; t < n_tokens; t += per) out.emplace_back(t, std::min(t + per, n_tokens));
        return PLAN_OK;
    }
    // union rule: wave_mark_ marks the experts of the open wave (cleared again before returning)
    for (int i = 0; i < n_tokens * k_; ++i)
        if (ids[i] < 0 || ids[i] >= E_) return PLAN_INVALID;
    std::vector<int32_t> &in_wave = wave_experts_;
    in_wave.clear();
    int t0 = 0, rc = PLAN_OK;
    for (int t = 0; t < n_tokens && rc == PLAN_OK; ++t) {
        int fresh = 0;
        for (int j = 0; j < k_; ++j) {
            const int32_t e = ids[(size_t)t * k_ + j];
            bool dup = false;
            for (int q = 0; q < j; ++q) dup |= ids[(size_t)t * k_ + q] == e;
            fresh += !wave_mark_[e] && !dup;
        }
        if ((int)in_wave.size() + fresh > K_) {
            if (t == t0) {
                rc = PLAN_TOO_SMALL;
                break;
            }
            out.emplace_back(t0, t);
            for (int32_t e : in_wave) wave_mark_[e] = 0;
            in_wave.clear();
            t0 = t;
            --t;   // the token opens the next wave
            continue;
        }
        for (int j = 0; j < k_; ++j) {
            const int32_t e = ids[(size_t)t * k_ + j];
            if (!wave_mark_[e]) {
                wave_mark_[e] = 1;
                in_wave.push_back(e);
            }
        }
    }
    for (int32_t e : in_wave) wave_mark_[e] = 0;
    if (rc != PLAN_OK) {
        out.clear();
        return rc;
    }
    out.emplace_back(t0, n_tokens);
    return PLAN_OK;
}

void Planner::coalesce(const std::vector<Fill> &fills, std::vector<Run> &runs) {
    runs.clear();
    for (const Fill &f : fills) {
        if (!runs.empty()) {
            Run &r = runs.back();
            if (f.expert == r.expert + r.n && f.slot == r.slot + r.n) {
                ++r.n;
                continue;
            }
        }
        runs.push_back({f.expert, f.slot, 1});
    }
}

int Planner::plan(int layer, const int32_t *ids, int t0, int t1, int wave, WavePlan &out) {
    if (layer < 0 || layer >= L_ || t1 < t0) return PLAN_INVALID;
    out.layer = layer;
    out.wave = wave;
    out.t0 = t0;
    out.t1 = t1;
    out.uniq.clear();
    out.hits.clear();
    out.fills.clear();
    out.evictions.clear();
    out.runs.clear();
    const int n_ids = (t1 - t0) * k_;
    const int32_t *w = ids + (size_t)t0 * k_;
    out.slots.assign(n_ids, -1);

    // distinct experts in first-occurrence order (validated before any change)
    if (++seen_stamp_ == 0) {
        std::fill(seen_.begin(), seen_.end(), 0);
        seen_stamp_ = 1;
    }
    for (int i = 0; i < n_ids; ++i) {
        int32_t e = w[i];
        if (e < 0 || e >= E_) return PLAN_INVALID;
        if (seen_[e] != seen_stamp_) {
            seen_[e] = seen_stamp_;
            out.uniq.push_back(e);
        }
    }
    if ((int)out.uniq.size() > K_) return PLAN_TOO_SMALL;

    SlotPool &pool = this->pool(layer);
    int32_t *smap = &slot_map_[(size_t)layer * E_];
    out.pick_hits = 0;
    for (int i = 0; i < n_ids; ++i) out.pick_hits += smap[w[i]] >= 0;

    if (lfu_) {
        plan_lfu(layer, out, smap);
        for (int i = 0; i < n_ids; ++i) out.slots[i] = smap[w[i]];
        coalesce(out.fills, out.runs);
        return PLAN_OK;
    }
    // 1. every resident expert becomes most recently used, so nothing this
    //    wave needs can be the victim below
    for (int32_t e : out.uniq) {
        int s = smap[e];
        if (s >= 0) {
            pool.refresh(s);
            out.hits.push_back(e);
        }
    }
    // 2. missing experts, ascending, take the least recently used slots
    std::vector<int32_t> missing;
    missing.reserve(out.uniq.size() - out.hits.size());
    for (int32_t e : out.uniq)
        if (smap[e] < 0) missing.push_back(e);
    std::sort(missing.begin(), missing.end());
    for (int32_t e : missing) {
        int s = pool.victim();
        int64_t old = pool.key(s);
        if (old >= 0) {
            int ol = shared_ ? (int)(old / E_) : layer;
            int oe = shared_ ? (int)(old % E_) : (int)old;
            slot_map_[(size_t)ol * E_ + oe] = -1;
            out.evictions.push_back({old, s});
        }
        pool.set_key(s, shared_ ? (int64_t)layer * E_ + e : (int64_t)e);
        smap[e] = s;
        pool.refresh(s);
        out.fills.push_back({e, s});
    }
    for (int i = 0; i < n_ids; ++i) out.slots[i] = smap[w[i]];
    coalesce(out.fills, out.runs);
    return PLAN_OK;
}

// Fills of a plan under the least-frequently-used policy (95 GiB page, "Decode"): every
// expert the plan names counts one more use; the missing ones, ascending, take the empty
// slots first (lowest first), then the resident slots the plan does not name, least
// (use count, plan of last use, slot) first.
void Planner::plan_lfu(int layer, WavePlan &out, int32_t *smap) {
    SlotPool &pool = this->pool(layer);
    const int pi = shared_ ? 0 : layer;
    std::vector<int64_t> &last = last_use_[pi];
    for (int32_t e : out.uniq) {
        counts_[(size_t)layer * E_ + e] += 1;
        if (smap[e] >= 0) out.hits.push_back(e);
    }
    std::vector<int32_t> missing;
    for (int32_t e : out.uniq)
        if (smap[e] < 0) missing.push_back(e);
    std::sort(missing.begin(), missing.end());
    std::vector<int> &vict = victims_;
    vict.clear();
    for (int s = 0; s < K_; ++s)
        if (pool.key(s) < 0) vict.push_back(s);
    const size_t n_empty = vict.size();
    auto count_of = [&](int s) {   // key layer*E+e (shared pool) or e (this layer's pool)
        const int64_t key = pool.key(s);
        return counts_[shared_ ? (size_t)key : (size_t)layer * E_ + (size_t)key];
    };
    if (missing.size() > n_empty) {
        for (int s = 0; s < K_; ++s) {
            const int64_t key = pool.key(s);
            if (key < 0) continue;
            const int kl = shared_ ? (int)(key / E_) : layer;
            const int ke = shared_ ? (int)(key % E_) : (int)key;
            if (kl == layer && seen_[ke] == seen_stamp_) continue;   // named by this plan
            vict.push_back(s);
        }
        const size_t need = missing.size() - n_empty;   // <= candidates: the plan fits in K
        std::partial_sort(vict.begin() + n_empty, vict.begin() + n_empty + need, vict.end(), [&](int a, int b) {
            const uint64_t ca = count_of(a), cb = count_of(b);
            if (ca != cb) return ca < cb;
            if (last[a] != last[b]) return last[a] < last[b];
            return a < b;
        });
    }
    for (size_t i = 0; i < missing.size(); ++i) {
        const int32_t e = missing[i];
        const int s = vict[i];
        const int64_t old = pool.key(s);
        if (old >= 0) {
            const int ol = shared_ ? (int)(old / E_) : layer;
            const int oe = shared_ ? (int)(old % E_) : (int)old;
            slot_map_[(size_t)ol * E_ + oe] = -1;
            out.evictions.push_back({old, s});
        }
        pool.set_key(s, shared_ ? (int64_t)layer * E_ + e : (int64_t)e);
        smap[e] = s;
        out.fills.push_back({e, s});
    }
    for (int32_t e : out.uniq) last[smap[e]] = clock_[pi];
    clock_[pi] += 1;
}

void Planner::rollback(const WavePlan &p) {
    SlotPool &pool = this->pool(p.layer);
    for (const Fill &f : p.fills) {
        slot_map_[(size_t)p.layer * E_ + f.expert] = -1;
        pool.set_key(f.slot, -1);
        pool.demote(f.slot);
    }
}

int Planner::prefill_lookup(int layer, const int32_t *ids, int n_ids, std::vector<int32_t> &experts,
                            std::vector<int32_t> &slot_or_minus1) const {
    if (layer < 0 || layer >= L_) return PLAN_INVALID;
    std::vector<uint8_t> touched(E_, 0);
    for (int i = 0; i < n_ids; ++i) {
        if (ids[i] < 0 || ids[i] >= E_) return PLAN_INVALID;
        touched[ids[i]] = 1;
    }
    experts.clear();
    slot_or_minus1.clear();
    for (int e = 0; e < E_; ++e)
        if (touched[e]) {
            experts.push_back(e);
            slot_or_minus1.push_back(slot_map_[(size_t)layer * E_ + e]);
        }
    return PLAN_OK;
}

void Planner::account(const WavePlan &p, int n_ids, int pick_hits) {
    BucketStats &b = (n_ids <= 8 * k_) ? small : large;
    b.plans += 1;
    b.hits += p.hits.size();
    b.misses += p.fills.size();
    b.evictions += p.evictions.size();
    b.bytes_h2d += (uint64_t)p.fills.size() * block_bytes_;
    b.picks += n_ids;
    b.pick_hits += pick_hits;
    b.union_sum += p.uniq.size();
    b.union_max = std::max<uint64_t>(b.union_max, p.uniq.size());
    waves_total += 1;
}

void Planner::account_prefill(int n_resident, int n_uploaded, int n_touched) {
    prefill.plans += 1;
    prefill.hits += n_resident;
    prefill.misses += n_uploaded;
    prefill.bytes_d2d += (uint64_t)n_resident * block_bytes_;
    prefill.bytes_h2d += (uint64_t)n_uploaded * block_bytes_;
    prefill.union_sum += n_touched;
    prefill.union_max = std::max<uint64_t>(prefill.union_max, n_touched);
}

void Planner::reset_stats() {
    small = BucketStats();
    large = BucketStats();
    prefill = BucketStats();
    waves_total = 0;
}

}  // namespace moe
