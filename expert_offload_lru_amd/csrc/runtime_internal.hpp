// Internal interface of the host runtime, shared by its source files: the cache
// object behind the C ABI (include/moe_offload.h) and the functions one part of the
// runtime calls in another (decode, uploads, two-tier store, captured steps, prefill).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <chrono>
#include <cerrno>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include <fcntl.h>
#include <unistd.h>

#include "errors.hpp"
#include "kernels.hpp"
#include "moe_offload.h"
#include "moe_planner.h"
#include "planner.hpp"

namespace moe {
void emit_trace(const WavePlan &p, int top_k, const int32_t *ids, const float *gate, moe_trace_fn fn, void *user);
void planner_stats(const Planner &pl, moe_stats &o);
// dst[0 .. bytes) = src[0 .. bytes) by a kernel on the stream's compute queue (prefill.hip):
// src is the device address of mapped host memory (read over the link), dst device memory,
// both 16-byte aligned, bytes a multiple of 4.  For small host-to-device copies that a
// kernel waits for: no hand-over between the copy engine and the compute queue.
hipError_t launch_copy_from_host(const void *src, void *dst, size_t bytes, hipStream_t stream);
}  // namespace moe

using moe::set_error;

constexpr int kReaderRing = 256;
constexpr int kFillRing = 8;
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 1024;
constexpr size_t kTimedMax = 4096; // timed launches held before their events are read
constexpr int kStageSlots = 64;   // prefetch staging bank: 2 banks of 32 experts
constexpr int kNearSlots = 16;    // the last 16 take the uploads for the next layers (near stream)
constexpr int kNearDepth = 2;     // speculation depths that take the near stream
constexpr int kPrefetchBacklog = 4; // default: speculative uploads only while fewer experts than this wait on the link
constexpr int kStackSpec = 3;       // default layers the stack driver speculates ahead (at most kMaxSpec)
constexpr int kStagedRing = 8;      // ev_staged slots: more than 1 + kMaxSpec layers
constexpr size_t kTwoStreamRuns = 8; // demand-upload runs of one wave that go over two streams

inline size_t expert_bytes_of(int quant, int hidden, int inter) {
    if (hidden <= 0 || inter <= 0) return 0;
    const size_t n = (size_t)hidden * inter;
    switch (quant) {
        case MOE_Q_F32: return 12 * n;
        case MOE_Q_INT4_G32_F16:
            if (hidden % 32 || inter % 32) return 0;
            return 3 * (n / 2 + n / 16);
        case MOE_Q_E2M1_E4M3_G16:
            if (hidden % 16 || inter % 16) return 0;
            return 3 * (n / 2 + n / 16);
        default: return 0;
    }
}

inline int hip_fail(hipError_t e, const char *what) {
    return set_error(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

inline double now_us() {
    return std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

// Adds the wall time of its scope to a host-time counter.
struct HostClock {
    double &acc;
    double t0;
    explicit HostClock(double &a) : acc(a), t0(now_us()) {}
    ~HostClock() { acc += now_us() - t0; }
};

struct TimedLaunch {
    int cls;
    hipEvent_t a, b;
    double bytes, flops;
};

struct UnitBuild {
    int32_t src;           // pool slot, -1 shared expert, <= -2 staging slot (-2 - src)
    int32_t copy_to;       // pool slot the block is copied into, or -1
    int32_t expert;        // -1 for the shared expert
    int32_t p0, np;        // its pairs: Units::pairs[p0 .. p0 + np)
};

// The units of one wave with their pairs, rebuilt per wave in reused storage.
struct Units {
    std::vector<UnitBuild> u;
    std::vector<uint16_t> pairs;
};

// Two-tier store (NVMe page, "Workflow": experts repacked into contiguous blocks read with
// pread, an LRU cache of pinned RAM blocks filled by reader threads, copies to the GPU from
// there).  The file holds block (layer, e) at byte offset (layer * E + e) * S.  A block is
// read into the least recently used RAM block, once every copy that read that block has
// completed: per block and per upload stream, the event recorded after the stream's last
// copy from it (a fence slot only ever holds events recorded on its own stream, and such an
// event is re-recorded only later on that stream, so waiting on it is never too early).
enum TierStream { kTierCopy = 0, kTierNear = 1, kTierSpec = 2, kTierStreams = 3 };

struct FileTier {
    int fd = -1;                      // buffered reads: direct I/O cannot target the GPU driver's pinned pages
    int R = 0, n_readers = 1;
    uint8_t *ram = nullptr;           // R pinned blocks
    moe::SlotPool lru{1};             // RAM blocks by recency, key = layer * E + e
    std::vector<int32_t> block_of;    // [L*E] RAM block of (layer, expert), -1 if absent
    std::vector<std::array<hipEvent_t, kTierStreams>> fence;   // per block and upload stream
    uint64_t hits = 0, misses = 0, evictions = 0, bytes_read = 0;
};

struct moe_cache {
    int E = 0, K = 0, k = 0, H = 0, I = 0, quant = 0, L = 0;
    unsigned flags = 0;
    size_t S = 0;
    int device = 0;
    moe::Planner pl;

    uint8_t *bank = nullptr;          // n_pools * K blocks
    int n_pools = 0;
    uint8_t *staging = nullptr;       // kStageSlots blocks (prefetch)
    std::vector<std::vector<const uint8_t *>> host_blocks;   // [L][E]
    std::vector<char> layer_ready;

    // routing buffers
    double *d_z = nullptr;
    double *d_zx = nullptr;           // one-launch router exchange array (every entry the sentinel
                                      // between launches)
    unsigned router_wait_us = moe::kRouterWaitUs;
    // fused decode kernel: its completion counters and flags (moe::kSyncBytes), the epoch of
    // the last fused launch
    unsigned *d_fused_sync = nullptr;
    unsigned long long fused_epoch = 0;
    // host-mapped flag that a kernel's bounded wait sets when it gives up (a fused down
    // workgroup waiting for gate/up, a router selection waiting for logits)
    int *h_wait_timeout = nullptr;
    int *h_wait_timeout_dev = nullptr;
    bool fuse_decode = false;
    // device copy of the slot table (slot of key layer*E+e, or -1), which the down kernel of a
    // wave updates, and its host shadow: what the device copy holds once the enqueued updates
    // have run.  One-token calls launch the resident picks' gate/up from it before planning.
    int32_t *d_map = nullptr;
    std::vector<int32_t> map_shadow;
    // A stale entry is harmless: where the device copy names a slot that no longer holds the
    // expert, the plan calls it a miss and the fill launch overwrites what the early launch
    // wrote; where it says -1 for a resident expert, the shadow says so too and the host
    // launches that hit itself.
    bool prelaunch = true;        // moe_cache_set_prelaunch
    // a plan changed slots that no down launch passed to the device copy (more changes than
    // one launch carries, several launch lists, the fused kernel, early launches off): the
    // next one-token call copies the whole table first
    bool map_dirty = false;
    bool map_carried = false;     // the last down + combine launch passed its plan's changes
    std::vector<int32_t> map_keys, map_vals;   // reused by the slot table's catch-up
    Units units_gu;               // the units a wave's own gate/up launches compute
    int32_t *d_ids = nullptr;
    float *d_gate = nullptr;
    // host-mapped routing results, two sets: a call's router may be launched (by the stack
    // driver, ahead) while the previous call still reads its speculative ids from the other
    struct RouteSet {
        int32_t *ids = nullptr, *spec = nullptr, *ids_dev = nullptr, *spec_dev = nullptr;
        float *gate = nullptr, *gate_dev = nullptr;
        int layer = -1, n_tok = 0, n_spec = 0;   // the call whose router last wrote the set
    };
    RouteSet rs[2];
    int rcur = 0;                     // the set of the call being processed
    int32_t *h_ids_base = nullptr, *h_spec_base = nullptr;
    float *h_gate_base = nullptr;
    int32_t *h_ids = nullptr;         // the current call's set (pinned, device-mapped)
    float *h_gate = nullptr;
    int32_t *h_spec = nullptr;
    int32_t *h_ids_dev = nullptr;
    float *h_gate_dev = nullptr;
    int32_t *h_spec_dev = nullptr;
    // a call whose router (and early gate/up) the stack driver launched ahead
    struct Ahead {
        bool on = false;
        int layer = -1, n_tok = 0, n_spec = 0, set = 0;
        const float *x = nullptr;
        hipStream_t stream = nullptr;
        bool pre = false;
        hipEvent_t pre_a = nullptr, pre_b = nullptr;
        // the early down + combine (one token), which wrote `out` if every pick was covered
        bool pre_down = false;
        hipEvent_t pre_da = nullptr, pre_db = nullptr;
        float *out = nullptr;
        unsigned fflags = 0;
    } ahead;
    int max_route_tokens = 0;
    int last_tokens = 0;

    // expert activations
    float *d_h = nullptr;             // [max_pairs x I]
    float *d_y = nullptr;             // [max_pairs x H]
    int max_pairs = 0;
    void *d_xq = nullptr;             // fp16 activation copy of x [32 x H]
    float *d_stack[2] = {nullptr, nullptr};   // stack driver ping-pong [32 x H]
    hipStream_t last_stream = nullptr;
    bool have_last_stream = false;
    uint64_t completed_seq = 0;       // reader events known complete

    hipStream_t copy_stream = nullptr;   // demand uploads (and the prefill arena)
    hipStream_t copy_stream2 = nullptr;  // every other run of a large wave's demand uploads
    hipEvent_t ev_copy2 = nullptr;       // joins copy_stream2 back into copy_stream
    hipStream_t spec_stream = nullptr;   // speculative uploads: a demand upload never queues behind them
    hipEvent_t ev_route = nullptr;
    std::vector<hipEvent_t> reader_ring;
    uint64_t reader_seq = 0;
    std::vector<int64_t> slot_reader;     // per global slot: reader sequence number, -1 never read
    std::vector<hipEvent_t> fill_ring;
    int fill_next = 0;

    // prefetch staging: which (layer, expert) each staging slot holds
    std::vector<int64_t> stage_key;       // -1 empty
    std::vector<char> stage_used;
    std::vector<uint64_t> stage_busy;     // call number of the last call that reads the slot
    int stage_next = 0;
    hipEvent_t ev_staged[kStagedRing] = {};   // after the uploads for layer l, at l % kStagedRing
    hipEvent_t ev_near[kStagedRing] = {};     // the same on the near stream
    // backlog of each upload stream: events recorded after upload batches, with the bytes
    // issued on that stream up to them (a stream completes its copies in order)
    struct CopyMark {
        hipEvent_t ev;
        uint64_t bytes;
    };
    struct CopyQueue {
        std::deque<CopyMark> marks;
        uint64_t issued = 0, done = 0;
    };
    CopyQueue demand_q, spec_q, near_q;
    std::vector<std::pair<size_t, size_t>> runs;   // scratch: (first fill, count) of each upload run
    std::vector<const uint8_t *> fill_src;         // scratch: host block of each fill of a wave
    int staged_for[kStagedRing] = {-1, -1, -1, -1, -1, -1, -1, -1};
    int near_for[kStagedRing] = {-1, -1, -1, -1, -1, -1, -1, -1};
    int near_next = kStageSlots - kNearSlots;
    uint64_t call_no = 0;

    moe_trace_fn trace_fn = nullptr;
    void *trace_user = nullptr;

    // fence checks (environment at creation): MOE_DEBUG_POISON fills every block an upload is
    // about to overwrite with all-one bytes (NaN scales) on the upload's stream first;
    // MOE_DEBUG_DELAY_US puts a delay kernel of that many microseconds ahead of every upload.
    // A reader that is not ordered after the upload then reads NaN, or the old expert, late.
    // moe_debug_fail_upload makes an upload submission fail as if the copy call had failed.
    // MOE_DEBUG_ROUTER_WAIT_US sets how long the one-launch router's selections wait for
    // the logits (0: every selection gives up at once), for checks of the timeout path.
    bool debug_poison = false;
    unsigned debug_delay_us = 0;
    int64_t debug_fail_upload = -1;       // submissions until the forced failure, -1 none

    FileTier *tier = nullptr;         // moe_cache_set_file_store: the host store is a file + RAM LRU

    uint64_t forwards = 0, pf_issued = 0, pf_used = 0, pf_wasted = 0, h2d_copied = 0, d2d_copied = 0;
    uint64_t pf_candidates = 0, pf_deferred = 0;
    int pf_backlog = kPrefetchBacklog, pf_ahead = kStackSpec;
    double plan_us = 0, wait_us = 0, call_us = 0, upload_us = 0, launch_us = 0, prefetch_us = 0, event_us = 0;

    unsigned time_mask = 0;
    int time_stride = 1;
    uint64_t time_count[8] = {};          // launches seen per timing class
    std::vector<TimedLaunch> timed;
    std::vector<hipEvent_t> event_pool;
    moe_timing timing{};

    // captured decode steps (moe_cache_set_graph): one-token stack calls while every expert
    // of every layer holds a slot, replayed as one graph per set of routing results; a
    // step's plans, counters and trace records are applied when the next call comes in
    bool graph_on = false;
    bool all_resident = false;        // valid while resident_checked == plan_changes
    uint64_t plan_changes = 0;        // plans that filled or evicted, and rollbacks
    uint64_t resident_checked = ~0ull;
    hipStream_t cap_stream = nullptr; // capture only: nothing runs on it
    float *d_gx = nullptr;            // [H] the step's input, copied in ahead of each replay
    int32_t *d_gids = nullptr;        // [L x top_k] the step's routing results on the device,
    float *d_ggate = nullptr;         // copied to the host arrays once, at the end of the step
    struct StepGraph {
        hipGraphExec_t exec = nullptr;
        hipEvent_t done = nullptr;
        int32_t *ids = nullptr;                       // [L x top_k] routing results (pinned)
        float *gate = nullptr;
        float *out = nullptr;                         // what the graph was captured for
        float *layer_inputs = nullptr;
        std::vector<const float *> routers;
        std::vector<const void *> shared;
    } sg[2];
    int sg_next = 0, sg_pending = -1;
    int *h_graph_bad = nullptr, *h_graph_bad_dev = nullptr;   // raised by a step that found a pick absent
    uint64_t graph_steps = 0;

    moe::WavePlan wp;
    std::vector<std::pair<int, int>> wave_ranges;
    Units units;                          // per-wave unit lists (reused storage)
    std::vector<int32_t> unit_of;         // expert -> unit index while a wave's units are built, else -1
    std::vector<moe::UnitList> lists;
    std::vector<moe::UnitList> lists_down;   // the fused launch's down list

    // prefill workspace (allocated on the first prefill call, grown as needed)
    int pf_cap = 0;                   // tokens
    _Float16 *pf_x16 = nullptr;       // [cap x H]
    _Float16 *pf_h16 = nullptr;       // [cap*(k+1) x I]
    float *pf_y = nullptr;            // [cap*(k+1) x H]
    // a call's plan: pairs, then items, then the dispatch tables of its GEMM launches, each
    // part 16-byte aligned, laid out alike in pinned host memory and on the device, so one
    // copy moves it
    uint8_t *pf_plan = nullptr;       // device
    uint8_t *pf_host = nullptr;       // pinned staging (mapped, coherent)
    const uint8_t *pf_host_dev = nullptr;   // its device address
    size_t pf_items_cap = 0;
    size_t pf_sched_cap = 0;
    uint8_t *arena = nullptr;         // 2 x 32 blocks
    hipEvent_t arena_read[2] = {nullptr, nullptr};
    hipEvent_t arena_ready[2] = {nullptr, nullptr};

    moe_cache(int E_, int K_, int k_, int L_, bool shared, size_t S_, bool union_waves, bool lfu, bool adaptive)
        : pl(E_, K_, k_, L_, shared, S_, union_waves, lfu, adaptive) {}

    // slot numbers are per layer (layer l's pool at l*K), or global (shared pool, and
    // per-layer pools with adaptive capacity)
    bool global_slots() const { return pl.shared_pool() || pl.adaptive(); }
    size_t global_slot(int layer, int slot) const { return (global_slots() ? 0 : (size_t)layer * K) + slot; }
    uint8_t *slot_ptr(int layer, int slot) const { return bank + global_slot(layer, slot) * S; }
    const uint8_t *pool_base(int layer) const { return global_slots() ? bank : bank + (size_t)layer * K * S; }
};

// Functions one part of the runtime calls in another (namespace rt keeps them out of the
// library's global names).
namespace rt {
hipEvent_t take_event(moe_cache *c);
void resolve_timing(moe_cache *c);
void pack_units(const Units &units, size_t begin, size_t end, std::vector<moe::UnitList> &lists);
size_t matrix_bytes(int quant, size_t rows, size_t cols);
void discard_ahead(moe_cache *c);
int ensure_route_capacity(moe_cache *c, int n_tok);
void drop_graphs(moe_cache *c);
int graph_sync(moe_cache *c);
int flush_graph(moe_cache *c);
int graph_step(moe_cache *c, const float *x, const float *const *router_ws, const void *const *shared_ws, float *out, float *layer_inputs, hipStream_t stream, bool *done);
void tier_touch(moe_cache *c, int layer, const int32_t *experts, int n);
int tier_fetch(moe_cache *c, int layer, const int32_t *experts, int n, const uint8_t **out, const char *touch_only = nullptr);
void tier_fence(moe_cache *c, const uint8_t *const *src, int n, hipEvent_t ev, TierStream which);
int pre_upload(moe_cache *c, uint8_t *dst, size_t n, hipStream_t st);
int upload_fills(moe_cache *c, int layer, const moe::WavePlan &p, hipEvent_t *fill_ev, std::vector<int> &staged);
void prefetch_next(moe_cache *c, int layer, int n_tok, int n_spec);
void pre_args(const moe_cache *c, int layer, const void *shared_w, const void *vec, moe::GemvArgs &a, moe::PreArgs &pa);
int prefill_forward(moe_cache *c, int layer, const float *x, int n_tok, const float *router_w, const void *shared_w, float *out, unsigned fflags, hipStream_t stream);
}  // namespace rt
using namespace rt;

// Events for one timed launch: the dispatch records them itself (kernel start and
// end as the command processor sees them), so the durations match a kernel trace.
struct TimeScope {
    moe_cache *c;
    int cls;
    hipEvent_t a = nullptr, b = nullptr;
    double bytes, flops;
    TimeScope(moe_cache *c_, int cls_, double bytes_, double flops_) : c(c_), cls(cls_), bytes(bytes_), flops(flops_) {
        if ((c->time_mask & (1u << cls)) && c->time_count[cls]++ % (uint64_t)c->time_stride == 0) {
            if (c->timed.size() >= kTimedMax) resolve_timing(c);
            a = take_event(c);
            b = a ? take_event(c) : nullptr;
            if (a && !b) {
                c->event_pool.push_back(a);
                a = nullptr;
            }
        }
    }
    ~TimeScope() {
        if (a) c->timed.push_back({cls, a, b, bytes, flops});
    }
};
