// Host-side slot table of the expert cache: LRU slot pools, the per-call
// plan, wave split, upload coalescing and statistics.  Pure C++17, no HIP:
// the same code runs inside the GPU library and in a CPU-only test library.
//
// Method (explainer page "MoE expert offload and the LRU expert cache ...",
// section "Inside llama.cpp PR #29887: slot maps, banks, and only the misses
// cross PCIe", and its "The rules in the code"; SGLang page, sections "What
// does Paged Experts actually do?" and "What happens with more than one
// request?"; T4 page, "What the MoE Cache Actually Caches"):
//   * a pool of K slots, per layer or shared by all layers (key = layer*E+e);
//   * a plan over one batch of routed ids refreshes every resident expert
//     first, then hands the least recently used slots to the missing experts
//     in ascending expert order, so that consecutive experts tend to land in
//     consecutive slots and their uploads merge (optionally the least
//     frequently used slots instead: 95 GiB page, "Decode");
//   * a decode step whose tokens*top_k exceed K runs in waves of K/top_k
//     tokens, one plan and one page-in each.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

namespace moe {

struct Fill {
    int32_t expert;
    int32_t slot;
};

struct Eviction {
    int64_t key;
    int32_t slot;
};

struct Run {            // fills merged into one copy: n experts from `expert`, into slots from `slot`
    int32_t expert;
    int32_t slot;
    int32_t n;
};

// Counters of one bucket of plans.
struct BucketStats {
    uint64_t plans = 0, hits = 0, misses = 0, picks = 0, pick_hits = 0, evictions = 0;
    uint64_t bytes_h2d = 0, bytes_d2d = 0, union_sum = 0, union_max = 0;
};

// Slots on a circular doubly linked recency list closed by a sentinel node
// (index n_space): sentinel.next is the least recently used slot, sentinel.prev
// the most recently used.  A pool holds the slots [lo, hi) of a numbering of
// n_space slots, initially in the order lo, lo+1, ..., hi-1, all empty; with
// adaptive capacity slots later leave (remove) and join (insert_lru) it.
class SlotPool {
public:
    explicit SlotPool(int n_slots) : SlotPool(n_slots, 0, n_slots) {}
    SlotPool(int n_space, int lo, int hi);
    int size() const { return count_; }               // slots held
    int victim() const { return link_next_[n_]; }   // least recently used slot
    void refresh(int s);                              // make s the most recently used
    void demote(int s);                               // make s the least recently used
    void remove(int s);                               // s leaves the pool
    void insert_lru(int s);                           // s joins as the least recently used
    int64_t key(int s) const { return key_[s]; }
    void set_key(int s, int64_t k) { key_[s] = k; }
    std::vector<int> order() const;                   // least -> most recently used

private:
    void unlink(int s);
    void insert_before(int s, int pos);
    int n_;
    int count_ = 0;
    std::vector<int> link_next_, link_prev_;
    std::vector<int64_t> key_;
};

// Result of planning one wave.
struct WavePlan {
    int layer = 0, wave = 0, t0 = 0, t1 = 0;
    std::vector<int32_t> uniq;          // distinct experts, first-occurrence order
    std::vector<int32_t> hits;          // resident experts, in `uniq` order
    std::vector<Fill> fills;            // ascending expert
    std::vector<Eviction> evictions;
    std::vector<int32_t> slots;         // [(t1-t0)*top_k] slot of every pick
    std::vector<Run> runs;              // coalesced fills
    int pick_hits = 0;                  // picks whose expert was resident before the plan
};

enum PlanStatus { PLAN_OK = 0, PLAN_INVALID = -1, PLAN_TOO_SMALL = -2 };

class Planner {
public:
    // adaptive: per-layer pools numbered globally (layer l starts with l*K .. l*K+K-1) whose
    // capacity follows per-layer targets (set_adaptive); not with a shared pool or LFU.
    Planner(int n_experts, int n_slots, int top_k, int n_layers, bool shared_pool, size_t block_bytes,
            bool union_waves = false, bool lfu = false, bool adaptive = false);

    int n_experts() const { return E_; }
    int n_slots() const { return K_; }
    int top_k() const { return k_; }
    int n_layers() const { return L_; }
    bool shared_pool() const { return shared_; }

    bool union_waves() const { return union_waves_; }
    bool lfu() const { return lfu_; }
    bool adaptive() const { return adaptive_; }

    // Adaptive per-layer capacity (95 GiB page, "Decode": capacity moves from layers with
    // high hit rates to layers with low ones, at the same total).  Every `period` steps the
    // layers with picks since the last rebalance are ranked by pick hit rate (exact ratios,
    // ties by layer); the i-th highest gives `delta` slots of target to the i-th lowest, for
    // i < pairs, while its rate is strictly higher, it stays >= floor and the taker <= E.
    // A layer follows its target in its next plan.  Returns PLAN_INVALID for bad values.
    int set_adaptive(int period, int delta, int pairs, int floor);
    // A decode step begins (a call of layer 0): rebalance when one is due.
    void begin_step();
    // Slots a wave of `layer` may use: K, or with adaptive capacity min(held, target).
    int capacity(int layer) const;
    int held(int layer) const { return pool(layer).size(); }
    int target(int layer) const { return adaptive_ ? targets_[layer] : K_; }
    uint64_t rebalances() const { return rebalances_; }

    // Token ranges of the waves of a decode call of `layer` with n_tokens tokens and routed
    // ids (token-major, top_k per token), C = capacity(layer).  Count rule: runs of C / top_k
    // tokens.  Union rule: a wave takes tokens in order while the union of their experts fits
    // in C slots (SGLang page, "Comments": C / top_k tokens is a sizing guarantee, not the
    // largest wave).
    int waves(int layer, int n_tokens, const int32_t *ids, std::vector<std::pair<int, int>> &out);

    // Plan tokens [t0, t1) of ids (token-major, top_k per token) for `layer`.
    // On error the pools are unchanged.
    int plan(int layer, const int32_t *ids, int t0, int t1, int wave, WavePlan &out);
    void plan_lfu(int layer, WavePlan &out, int32_t *smap);
    void plan_adaptive(int layer, WavePlan &out, int32_t *smap);

    // Undo the fills of a plan whose uploads could not be submitted: the
    // filled slots become empty and least recently used.
    void rollback(const WavePlan &p);

    // Prefill: touched experts in ascending order, with residency; pools untouched.
    // With count, also the number of ids of each expert (count[e], e < E).
    int prefill_lookup(int layer, const int32_t *ids, int n_ids, std::vector<int32_t> &experts,
                       std::vector<int32_t> &slot_or_minus1, std::vector<int32_t> *count = nullptr) const;

    int slot_of(int layer, int expert) const { return slot_map_[(size_t)layer * E_ + expert]; }
    SlotPool &pool(int layer) { return pools_[shared_ ? 0 : layer]; }
    const SlotPool &pool(int layer) const { return pools_[shared_ ? 0 : layer]; }

    // Statistics.
    BucketStats small, large, prefill;
    uint64_t waves_total = 0;
    void account(const WavePlan &p, int n_ids, int pick_hits);
    void account_prefill(int n_resident, int n_uploaded, int n_touched);
    void reset_stats();

    static void coalesce(const std::vector<Fill> &fills, std::vector<Run> &runs);

private:
    int E_, K_, k_, L_;
    bool union_waves_ = false;
    bool shared_;
    size_t block_bytes_;
    std::vector<SlotPool> pools_;
    std::vector<int32_t> slot_map_;     // [L*E] slot of (layer, expert), -1 if not cached
    std::vector<int32_t> seen_;         // scratch: per-expert stamp for dedup
    int32_t seen_stamp_ = 0;
    std::vector<uint8_t> wave_mark_;    // scratch of the union wave rule: experts of the open wave
    std::vector<int32_t> wave_experts_;
    // least-frequently-used policy: a use count per (layer, expert) that survives eviction,
    // and per pool the plan number of each slot's last use
    bool lfu_ = false;
    std::vector<uint64_t> counts_;
    std::vector<std::vector<int64_t>> last_use_;
    std::vector<int64_t> clock_;
    std::vector<int> victims_;
    // adaptive per-layer capacity
    bool adaptive_ = false;
    int period_ = 8, delta_ = 2, pairs_ = 4, floor_ = 0;
    std::vector<int> targets_;
    std::vector<int> free_;             // released slots, ascending
    std::vector<uint64_t> win_picks_, win_hits_;
    uint64_t steps_ = 0, rebalances_ = 0;
};

}  // namespace moe
