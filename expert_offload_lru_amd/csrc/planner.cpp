// Host-side slot table of the expert cache (see planner.hpp for the method
// and the pages it follows).
#include "planner.hpp"

#include <algorithm>

namespace moe {

// ----------------------------------------------------------------------------- SlotPool

SlotPool::SlotPool(int n_space, int lo, int hi)
    : n_(n_space), link_next_(n_space + 1, -1), link_prev_(n_space + 1, -1), key_(n_space, -1) {
    // circular list sentinel -> lo -> lo+1 -> ... -> hi-1 -> sentinel
    link_next_[n_] = link_prev_[n_] = n_;
    for (int s = lo; s < hi; ++s) insert_before(s, n_);
    count_ = hi - lo;
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

void SlotPool::remove(int s) {
    unlink(s);
    link_next_[s] = link_prev_[s] = -1;
    --count_;
}

void SlotPool::insert_lru(int s) {
    insert_before(s, link_next_[n_]);
    ++count_;
}

std::vector<int> SlotPool::order() const {
    std::vector<int> out;
    for (int s = link_next_[n_]; s != n_; s = link_next_[s]) out.push_back(s);
    return out;
}

// ----------------------------------------------------------------------------- Planner

Planner::Planner(int n_experts, int n_slots, int top_k, int n_layers, bool shared_pool, size_t block_bytes,
                 bool union_waves, bool lfu, bool adaptive)
    : E_(n_experts), K_(n_slots), k_(top_k), L_(n_layers), shared_(shared_pool), block_bytes_(block_bytes),
      slot_map_((size_t)n_layers * n_experts, -1), seen_(n_experts, 0), wave_mark_(n_experts, 0) {
    union_waves_ = union_waves;
    lfu_ = lfu;
    adaptive_ = adaptive && !shared_pool && !lfu;
    if (adaptive_) {
        targets_.assign(n_layers, n_slots);
        win_picks_.assign(n_layers, 0);
        win_hits_.assign(n_layers, 0);
        floor_ = std::max(top_k, n_slots / 2);
        pools_.reserve(n_layers);
        for (int l = 0; l < n_layers; ++l) pools_.emplace_back(n_layers * n_slots, l * n_slots, (l + 1) * n_slots);
        return;
    }
    if (lfu_) {
        counts_.assign((size_t)n_layers * n_experts, 0);
        last_use_.assign(shared_pool ? 1 : n_layers, std::vector<int64_t>(n_slots, -1));
        clock_.assign(shared_pool ? 1 : n_layers, 0);
    }
    int n_pools = shared_ ? 1 : L_;
    pools_.reserve(n_pools);
    for (int i = 0; i < n_pools; ++i) pools_.emplace_back(K_);
}

int Planner::set_adaptive(int period, int delta, int pairs, int floor) {
    if (!adaptive_ || period < 1 || delta < 0 || pairs < 0 || floor < k_ || floor > K_) return PLAN_INVALID;
    period_ = period;
    delta_ = delta;
    pairs_ = pairs;
    floor_ = floor;
    return PLAN_OK;
}

int Planner::capacity(int layer) const {
    if (!adaptive_) return K_;
    return std::min(pools_[layer].size(), targets_[layer]);
}

void Planner::begin_step() {
    if (!adaptive_) return;
    if (steps_ > 0 && steps_ % (uint64_t)period_ == 0) {
        // rate(a) > rate(b), compared exactly as hits_a * picks_b > hits_b * picks_a
        auto higher = [&](int a, int b) {
            return (unsigned __int128)win_hits_[a] * win_picks_[b] > (unsigned __int128)win_hits_[b] * win_picks_[a];
        };
        std::vector<int> high, low;
        for (int l = 0; l < L_; ++l)
            if (win_picks_[l] > 0) high.push_back(l);
        low = high;
        std::sort(high.begin(), high.end(), [&](int a, int b) { return higher(a, b) || (!higher(b, a) && a < b); });
        std::sort(low.begin(), low.end(), [&](int a, int b) { return higher(b, a) || (!higher(a, b) && a < b); });
        const int n = std::min<int>(pairs_, (int)high.size() / 2);
        for (int i = 0; i < n; ++i) {
            const int d = high[i], r = low[i];
            if (!higher(d, r)) break;
            if (targets_[d] - delta_ < floor_ || targets_[r] + delta_ > E_) continue;
            targets_[d] -= delta_;
            targets_[r] += delta_;
        }
        std::fill(win_picks_.begin(), win_picks_.end(), 0);
        std::fill(win_hits_.begin(), win_hits_.end(), 0);
        rebalances_ += 1;
    }
    steps_ += 1;
}

int Planner::waves(int layer, int n_tokens, const int32_t *ids, std::vector<std::pair<int, int>> &out) {
    out.clear();
    if (layer < 0 || layer >= L_) return PLAN_INVALID;
    if (n_tokens <= 0) return PLAN_OK;
    const int cap = capacity(layer);
    if ((long long)n_tokens * k_ <= cap) {
        out.emplace_back(0, n_tokens);
        return PLAN_OK;
    }
    if (!union_waves_) {
        int per = cap / k_;
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
        if ((int)in_wave.size() + fresh > cap) {
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
    if (adaptive_) {
        // slots this plan can hold: what the layer has, plus what it may take from the free list
        const int grow = std::min<int>(std::max(targets_[layer] - pools_[layer].size(), 0), (int)free_.size());
        if ((int)out.uniq.size() > pools_[layer].size() + grow) return PLAN_TOO_SMALL;
    } else if ((int)out.uniq.size() > K_) {
        return PLAN_TOO_SMALL;
    }

    SlotPool &pool = this->pool(layer);
    int32_t *smap = &slot_map_[(size_t)layer * E_];
    out.pick_hits = 0;
    for (int i = 0; i < n_ids; ++i) out.pick_hits += smap[w[i]] >= 0;

    if (adaptive_) {
        plan_adaptive(layer, out, smap);
        win_picks_[layer] += n_ids;
        win_hits_[layer] += out.pick_hits;
        for (int i = 0; i < n_ids; ++i) out.slots[i] = smap[w[i]];
        coalesce(out.fills, out.runs);
        return PLAN_OK;
    }

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

// A plan of a layer with adaptive capacity: the layer first takes free slots up to its
// target (the lowest ones, placed in ascending order at the least-recently-used end),
// refreshes its hits, then releases its least recently used slots down to its target
// (evicting their experts) while it keeps at least the plan's distinct experts, and fills
// the misses, ascending, from the least recently used slots.
void Planner::plan_adaptive(int layer, WavePlan &out, int32_t *smap) {
    SlotPool &pool = pools_[layer];
    const int want = targets_[layer] - pool.size();
    if (want > 0 && !free_.empty()) {
        const int n = std::min<int>(want, (int)free_.size());
        for (int i = n - 1; i >= 0; --i) pool.insert_lru(free_[i]);
        free_.erase(free_.begin(), free_.begin() + n);
    }
    for (int32_t e : out.uniq) {
        const int s = smap[e];
        if (s >= 0) {
            pool.refresh(s);
            out.hits.push_back(e);
        }
    }
    for (int extra = std::min(pool.size() - targets_[layer], pool.size() - (int)out.uniq.size()); extra > 0;
         --extra) {
        const int s = pool.victim();
        const int64_t old = pool.key(s);
        if (old >= 0) {
            smap[old] = -1;
            pool.set_key(s, -1);
            out.evictions.push_back({old, s});
        }
        pool.remove(s);
        free_.insert(std::lower_bound(free_.begin(), free_.end(), s), s);
    }
    std::vector<int32_t> missing;
    for (int32_t e : out.uniq)
        if (smap[e] < 0) missing.push_back(e);
    std::sort(missing.begin(), missing.end());
    for (int32_t e : missing) {
        const int s = pool.victim();
        const int64_t old = pool.key(s);
        if (old >= 0) {
            smap[old] = -1;
            out.evictions.push_back({old, s});
        }
        pool.set_key(s, (int64_t)e);
        smap[e] = s;
        pool.refresh(s);
        out.fills.push_back({e, s});
    }
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
                            std::vector<int32_t> &slot_or_minus1, std::vector<int32_t> *count) const {
    if (layer < 0 || layer >= L_) return PLAN_INVALID;
    std::vector<int32_t> own;
    std::vector<int32_t> &touched = count ? *count : own;
    // four partial counts, so that an expert repeated in nearby ids does not chain the
    // increments through memory
    std::vector<int32_t> part(4 * (size_t)E_, 0);
    int i = 0;
    for (; i + 4 <= n_ids; i += 4) {
        const unsigned a = (unsigned)ids[i], b = (unsigned)ids[i + 1], c = (unsigned)ids[i + 2], d = (unsigned)ids[i + 3];
        if (a >= (unsigned)E_ || b >= (unsigned)E_ || c >= (unsigned)E_ || d >= (unsigned)E_) return PLAN_INVALID;
        part[a] += 1;
        part[E_ + b] += 1;
        part[2 * (size_t)E_ + c] += 1;
        part[3 * (size_t)E_ + d] += 1;
    }
    for (; i < n_ids; ++i) {
        if ((unsigned)ids[i] >= (unsigned)E_) return PLAN_INVALID;
        part[ids[i]] += 1;
    }
    touched.assign(E_, 0);
    for (int e = 0; e < E_; ++e) touched[e] = part[e] + part[E_ + e] + part[2 * (size_t)E_ + e] + part[3 * (size_t)E_ + e];
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
