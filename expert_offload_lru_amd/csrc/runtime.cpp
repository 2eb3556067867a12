// Host runtime of the offloaded MoE layer: the cache object behind the C ABI
// (include/moe_offload.h).  Decode calls follow the pages' sequence
// (explainer page, "Inside llama.cpp PR #29887": the router's ids reach the
// host, the slot table plans, only the missing experts are uploaded, the
// expert kernels read the cache; SGLang page, "What happens with more than
// one request?": waves when tokens*top_k exceed K):
//
//   stream:   router ──► [host: wait ids, plan wave, enqueue copies] ──►
//             gate/up(hit units) ─► wait(fill) ─► gate/up(filled units) ─►
//             down(all units) ─► record reader event ─► ... ─► combine
//   copy stream: wait(last reader of each victim slot) ─► H2D / D2D runs ─►
//                record fill event
//   speculation stream: H2D of predicted misses of later layers into a staging
//                bank ─► record staged event per layer
//
// Overlap (95 GiB page, "Decode": hits and the shared expert compute while
// misses transfer) comes from launching the hit units before the compute
// stream waits on the fill event.  A slot is overwritten only after the
// kernels that last read it (per-slot reader sequence numbers on a ring of
// events), so waves, a shared pool and prefetch staging stay race-free.
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
}  // namespace moe

using moe::set_error;

namespace {

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

size_t expert_bytes_of(int quant, int hidden, int inter) {
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

int hip_fail(hipError_t e, const char *what) {
    return set_error(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

double now_us() {
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

}  // namespace

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
    unsigned *d_tickets = nullptr;    // one-launch router counters (zero between launches)
    // fused decode kernel: its completion counters and flags (moe::kSyncBytes), the epoch of
    // the last fused launch, and a host-mapped flag a down workgroup sets if it gave up waiting
    unsigned *d_fused_sync = nullptr;
    unsigned long long fused_epoch = 0;
    int *h_fused_timeout = nullptr;
    int *h_fused_timeout_dev = nullptr;
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
    Units units_gu;               // the units a wave's own gate/up launches compute
    int32_t *d_ids = nullptr;
    float *d_gate = nullptr;
    // host-mapped routing results, two sets: a call's router may be launched (by the stack
    // driver, ahead) while the previous call still reads its speculative ids from the other
    struct RouteSet {
        int32_t *ids = nullptr, *spec = nullptr, *ids_dev = nullptr, *spec_dev = nullptr;
        float *gate = nullptr, *gate_dev = nullptr;
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
    int32_t *pf_pairs = nullptr;      // device [cap*(k+1)]
    moe::PrefillItem *pf_items = nullptr;   // device
    int32_t *pf_sched = nullptr;      // device dispatch tables of the prefill GEMM launches
    size_t pf_sched_cap = 0;
    uint8_t *pf_host = nullptr;       // pinned staging of pairs + items
    size_t pf_items_cap = 0;
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

namespace {

// ----------------------------------------------------------------------------- timing

hipEvent_t take_event(moe_cache *c) {
    if (!c->event_pool.empty()) {
        hipEvent_t e = c->event_pool.back();
        c->event_pool.pop_back();
        return e;
    }
    // timing only: no system-scope fence when the event is recorded, so the stop stamp is not
    // delayed by a cache writeback (and the following launch is not slowed by it)
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

void resolve_timing(moe_cache *c) {
    if (c->timed.empty()) return;
    hipEventSynchronize(c->timed.back().b);
    for (TimedLaunch &t : c->timed) {
        float ms = 0.f;
        hipEventElapsedTime(&ms, t.a, t.b);
        moe_kernel_timing *k = nullptr;
        switch (t.cls) {
            case 0: k = &c->timing.router; break;
            case 1: k = &c->timing.gate_up; break;
            case 2: k = &c->timing.down; break;
            case 3: k = &c->timing.combine; break;
            case 5: k = &c->timing.expert_fused; break;
            case 6: k = &c->timing.gate_up_early; break;
            default: k = &c->timing.prefill_gemm; break;
        }
        k->launches += 1;
        k->ms += ms;
        k->bytes += t.bytes;
        k->flops += t.flops;
        c->event_pool.push_back(t.a);
        c->event_pool.push_back(t.b);
    }
    c->timed.clear();
}

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

// ----------------------------------------------------------------------------- unit lists

// Pack units into launch lists of at most kMaxUnits units and kMaxPairs pairs.
void pack_units(const Units &units, size_t begin, size_t end, std::vector<moe::UnitList> &lists) {
    lists.clear();
    int np = 0;
    for (size_t i = begin; i < end; ++i) {
        const UnitBuild &u = units.u[i];
        if (lists.empty() || lists.back().n_units == moe::kMaxUnits || np + u.np > moe::kMaxPairs) {
            lists.emplace_back();
            lists.back().n_units = 0;
            lists.back().pbeg[0] = 0;
            lists.back().pad_ = 0;
            np = 0;
        }
        moe::UnitList &cur = lists.back();
        cur.src[cur.n_units] = u.src;
        cur.copy_to[cur.n_units] = u.copy_to;
        for (int j = 0; j < u.np; ++j) cur.pair[np + j] = units.pairs[u.p0 + j];
        np += u.np;
        cur.n_units += 1;
        cur.pbeg[cur.n_units] = (uint16_t)np;
    }
}

size_t matrix_bytes(int quant, size_t rows, size_t cols) {
    const size_t n = rows * cols;
    if (quant == MOE_Q_F32) return 4 * n;
    return n / 2 + n / 16;
}

int check_shapes(int quant, int hidden, int inter) {
    for (int n_mats = 1; n_mats <= 2; ++n_mats) {
        const int cols = n_mats == 2 ? hidden : inter;
        if (!moe::gemv_shape(quant, cols, n_mats).ok) return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

// The current call reads its routing from set st.
void use_route_set(moe_cache *c, int st) {
    c->rcur = st;
    const moe_cache::RouteSet &r = c->rs[st];
    c->h_ids = r.ids;
    c->h_gate = r.gate;
    c->h_spec = r.spec;
    c->h_ids_dev = r.ids_dev;
    c->h_gate_dev = r.gate_dev;
    c->h_spec_dev = r.spec_dev;
}

// Forget a call launched ahead that is not the one now made (only after an error): its
// router may still be queued, so the stream drains before its buffers are reused.
void discard_ahead(moe_cache *c) {
    if (!c->ahead.on) return;
    hipStreamSynchronize(c->ahead.stream);
    if (c->ahead.pre_a) c->event_pool.push_back(c->ahead.pre_a);
    if (c->ahead.pre_b) c->event_pool.push_back(c->ahead.pre_b);
    c->ahead = moe_cache::Ahead();
}

// Captured steps name the routing buffers: they go when those are reallocated (after the
// step in flight, if any, has finished).
void drop_graphs(moe_cache *c) {
    for (moe_cache::StepGraph &g : c->sg) {
        if (g.done) hipEventSynchronize(g.done);
        if (g.exec) hipGraphExecDestroy(g.exec);
        g.exec = nullptr;
        g.out = nullptr;
        g.routers.clear();
        g.shared.clear();
    }
}

int ensure_route_capacity(moe_cache *c, int n_tok) {
    if (n_tok <= c->max_route_tokens) return MOE_OK;
    discard_ahead(c);
    drop_graphs(c);
    const int cap = std::max(n_tok, 32);
    hipError_t e;
    if (c->d_z) hipFree(c->d_z);
    if (c->d_ids) hipFree(c->d_ids);
    if (c->d_gate) hipFree(c->d_gate);
    if (c->h_ids_base) hipHostFree(c->h_ids_base);
    if (c->h_gate_base) hipHostFree(c->h_gate_base);
    if (c->h_spec_base) hipHostFree(c->h_spec_base);
    c->d_z = nullptr;
    c->d_ids = nullptr;
    c->d_gate = nullptr;
    c->h_ids_base = c->h_spec_base = nullptr;
    c->h_gate_base = nullptr;
    c->rs[0] = c->rs[1] = moe_cache::RouteSet();
    c->h_ids = nullptr;
    c->h_gate = nullptr;
    c->h_spec = nullptr;
    c->max_route_tokens = 0;
    const size_t nk = (size_t)cap * c->k;
    if ((e = hipMalloc(&c->d_z, (1 + moe::kMaxSpec) * (size_t)cap * c->E * sizeof(double))) != hipSuccess ||
        (e = hipMalloc(&c->d_ids, nk * sizeof(int32_t))) != hipSuccess ||
        (e = hipMalloc(&c->d_gate, nk * sizeof(float))) != hipSuccess)
        return set_error(MOE_ERR_OOM, std::string("routing buffers: ") + hipGetErrorString(e));
    const unsigned hf = hipHostMallocMapped | hipHostMallocCoherent;
    if ((e = hipHostMalloc((void **)&c->h_ids_base, 2 * nk * sizeof(int32_t), hf)) != hipSuccess ||
        (e = hipHostMalloc((void **)&c->h_gate_base, 2 * nk * sizeof(float), hf)) != hipSuccess ||
        (e = hipHostMalloc((void **)&c->h_spec_base, 2 * moe::kMaxSpec * nk * sizeof(int32_t), hf)) != hipSuccess)
        return set_error(MOE_ERR_OOM, std::string("pinned routing buffers: ") + hipGetErrorString(e));
    int32_t *ids_dev = nullptr, *spec_dev = nullptr;
    float *gate_dev = nullptr;
    if ((e = hipHostGetDevicePointer((void **)&ids_dev, c->h_ids_base, 0)) != hipSuccess ||
        (e = hipHostGetDevicePointer((void **)&gate_dev, c->h_gate_base, 0)) != hipSuccess ||
        (e = hipHostGetDevicePointer((void **)&spec_dev, c->h_spec_base, 0)) != hipSuccess)
        return hip_fail(e, "hipHostGetDevicePointer");
    for (int st = 0; st < 2; ++st) {
        moe_cache::RouteSet &r = c->rs[st];
        r.ids = c->h_ids_base + st * nk;
        r.gate = c->h_gate_base + st * nk;
        r.spec = c->h_spec_base + st * moe::kMaxSpec * nk;
        r.ids_dev = ids_dev + st * nk;
        r.gate_dev = gate_dev + st * nk;
        r.spec_dev = spec_dev + st * moe::kMaxSpec * nk;
    }
    use_route_set(c, c->rcur);
    c->max_route_tokens = cap;
    return MOE_OK;
}

// ----------------------------------------------------------------------------- uploads

// Uploads of one wave's fills from host memory on the copy stream.  A fill
// whose expert sits in the prefetch staging bank is not copied here: the
// expert GEMV reads it from staging and writes it into its slot (staged[i] =
// staging slot, else -1).  Returns MOE_OK or an error (the caller rolls the
// plan back).
// An event recorded on the copy stream after the uploads issued so far.  Events
// are reused from rings: a re-recorded event completes no earlier than its
// older record, so the backlog below only ever errs on the high side.
void note_copy_mark(moe_cache::CopyQueue &q, hipEvent_t ev) {
    q.marks.push_back({ev, q.issued});
    if (q.marks.size() > 64) {
        q.done = q.marks.front().bytes;
        q.marks.pop_front();
    }
}

uint64_t queue_backlog(moe_cache::CopyQueue &q) {
    while (!q.marks.empty() && hipEventQuery(q.marks.front().ev) == hipSuccess) {
        q.done = q.marks.front().bytes;
        q.marks.pop_front();
    }
    return q.issued - q.done;
}

// Bytes issued on the upload streams that have not completed yet (they share the link).
uint64_t copy_backlog(moe_cache *c) {
    return queue_backlog(c->demand_q) + queue_backlog(c->spec_q) + queue_backlog(c->near_q);
}

// ----------------------------------------------------------------------------- two-tier store

// Read blocks (RAM block, key) from the file, spread over the reader threads.  On failure
// the blocks that may hold partial data are emptied.
int tier_read(moe_cache *c, const std::vector<std::pair<int, int64_t>> &reads) {
    FileTier &t = *c->tier;
    if (reads.empty()) return MOE_OK;
    std::vector<int> err(reads.size(), 0);
    auto read_some = [&](size_t first, size_t stride) {
        for (size_t i = first; i < reads.size(); i += stride) {
            uint8_t *dst = t.ram + (size_t)reads[i].first * c->S;
            const off_t off = (off_t)reads[i].second * (off_t)c->S;
            size_t done = 0;
            while (done < c->S) {
                const ssize_t r = pread(t.fd, dst + done, c->S - done, off + (off_t)done);
                if (r < 0 && errno == EINTR) continue;
                if (r <= 0) {
                    err[i] = r < 0 ? errno : -1;
                    break;
                }
                done += (size_t)r;
            }
        }
    };
    const size_t n_thr = std::min<size_t>((size_t)t.n_readers, reads.size());
    if (n_thr <= 1) {
        read_some(0, 1);
    } else {
        std::vector<std::thread> thr;
        for (size_t i = 1; i < n_thr; ++i) thr.emplace_back(read_some, i, n_thr);
        read_some(0, n_thr);
        for (std::thread &th : thr) th.join();
    }
    int bad = 0;
    for (size_t i = 0; i < reads.size(); ++i) {
        if (!err[i]) {
            t.bytes_read += c->S;
            continue;
        }
        bad = err[i];
        const int b = reads[i].first;
        t.block_of[reads[i].second] = -1;
        t.lru.set_key(b, -1);
        t.lru.demote(b);
    }
    if (bad) return set_error(MOE_ERR_IO, std::string("reading the expert file: ") + (bad > 0 ? strerror(bad) : "short file"));
    return MOE_OK;
}

// Uses that need no read (hits in the slots, fills served from staging): a present block
// becomes the most recently used.
void tier_touch(moe_cache *c, int layer, const int32_t *experts, int n) {
    if (!c->tier) return;
    FileTier &t = *c->tier;
    for (int i = 0; i < n; ++i) {
        const int b = t.block_of[(size_t)layer * c->E + experts[i]];
        if (b >= 0) t.lru.refresh(b);
    }
}

// Pinned RAM addresses of the blocks of (layer, experts[0..n)), used in that order: a
// present block becomes the most recently used; an absent one is read into the least
// recently used block (evicting its key, after the copies that read it completed).  Where
// touch_only[i], the use needs no read: out[i] = nullptr, and only a present block is
// refreshed.  A block used by this call is never taken again for a later key of the call
// (the tier is sized for a wave's or a prefill batch's uploads; should a call need more,
// it fails instead of overwriting a block it is about to copy from).
int tier_fetch(moe_cache *c, int layer, const int32_t *experts, int n, const uint8_t **out,
               const char *touch_only = nullptr) {
    FileTier &t = *c->tier;
    std::vector<std::pair<int, int64_t>> reads;
    std::vector<int> used;                  // blocks this call already handed out
    // on an error before the reads, the keys queued for reading are absent again
    auto drop_queued = [&]() {
        for (const auto &rd : reads) {
            t.block_of[rd.second] = -1;
            t.lru.set_key(rd.first, -1);
            t.lru.demote(rd.first);
        }
    };
    for (int i = 0; i < n; ++i) {
        const int64_t key = (int64_t)layer * c->E + experts[i];
        int b = t.block_of[key];
        if (touch_only && touch_only[i]) {
            if (b >= 0) t.lru.refresh(b);
            out[i] = nullptr;
            continue;
        }
        if (b >= 0) {
            t.hits += 1;
        } else {
            b = t.lru.victim();
            if (std::find(used.begin(), used.end(), b) != used.end()) {
                drop_queued();
                return set_error(MOE_ERR_INVALID, "the RAM tier holds fewer blocks than one call's uploads");
            }
            for (hipEvent_t &f : t.fence[b]) {
                if (!f) continue;
                HostClock hc(c->event_us);
                const hipError_t e = hipEventSynchronize(f);
                if (e != hipSuccess) {
                    drop_queued();
                    return hip_fail(e, "hipEventSynchronize(RAM block)");
                }
                f = nullptr;
            }
            const int64_t old = t.lru.key(b);
            if (old >= 0) {
                t.block_of[old] = -1;
                t.evictions += 1;
            }
            t.lru.set_key(b, key);
            t.block_of[key] = b;
            t.misses += 1;
            reads.push_back({b, key});
        }
        t.lru.refresh(b);
        used.push_back(b);
        out[i] = t.ram + (size_t)b * c->S;
    }
    return tier_read(c, reads);
}

// The copies just issued on upload stream `which` from RAM blocks complete by event ev,
// recorded on that stream after them.
void tier_fence(moe_cache *c, const uint8_t *const *src, int n, hipEvent_t ev, TierStream which) {
    if (!c->tier || !ev) return;
    FileTier &t = *c->tier;
    for (int i = 0; i < n; ++i) {
        if (!src[i] || src[i] < t.ram || src[i] >= t.ram + (size_t)t.R * c->S) continue;
        t.fence[(size_t)(src[i] - t.ram) / c->S][which] = ev;
    }
}

// Before an upload of n blocks into dst on stream st: the fence checks' delay and poison,
// and the forced failure of moe_debug_fail_upload (then nothing is enqueued).
int pre_upload(moe_cache *c, uint8_t *dst, size_t n, hipStream_t st) {
    if (c->debug_fail_upload >= 0 && c->debug_fail_upload-- == 0)
        return set_error(MOE_ERR_HIP, "upload submission failed (forced by moe_debug_fail_upload)");
    hipError_t e;
    if (c->debug_delay_us && (e = moe::launch_delay_us(c->debug_delay_us, st)) != hipSuccess)
        return hip_fail(e, "delay kernel");
    if (c->debug_poison && (e = moe::launch_fill_u32(reinterpret_cast<unsigned *>(dst), 0xFFFFFFFFu, n * c->S / 4,
                                                     st)) != hipSuccess)
        return hip_fail(e, "poison fill");
    return MOE_OK;
}

int upload_fills(moe_cache *c, int layer, const moe::WavePlan &p, hipEvent_t *fill_ev, std::vector<int> &staged) {
    HostClock hc(c->upload_us);
    *fill_ev = nullptr;
    staged.assign(p.fills.size(), -1);
    // the RAM tier's recency follows every use: the plan's hits first
    tier_touch(c, layer, p.hits.data(), (int)p.hits.size());
    if (p.fills.empty()) return MOE_OK;
    hipError_t e;
    if (c->staging) {
        for (size_t i = 0; i < p.fills.size(); ++i) {
            const int64_t key = (int64_t)layer * c->E + p.fills[i].expert;
            for (int s = 0; s < kStageSlots; ++s)
                if (c->stage_key[s] == key) {
                    staged[i] = s;
                    c->stage_used[s] = 1;
                    c->stage_busy[s] = c->call_no;
                    c->pf_used += 1;
                    c->d2d_copied += c->S;
                    break;
                }
        }
    }
    bool any_h2d = false;
    for (size_t i = 0; i < p.fills.size(); ++i) any_h2d |= staged[i] < 0;
    if (!any_h2d) {
        for (const moe::Fill &f : p.fills) tier_touch(c, layer, &f.expert, 1);
        return MOE_OK;
    }
    // the copy stream must not overwrite a slot before its last readers ran
    int64_t wait_seq = -1;
    for (size_t i = 0; i < p.fills.size(); ++i)
        if (staged[i] < 0) wait_seq = std::max(wait_seq, c->slot_reader[c->global_slot(layer, p.fills[i].slot)]);
    // the host block of every fill to copy (with a file store: its RAM block, read from the
    // file where absent, the fills taken in the plan's order)
    std::vector<const uint8_t *> &hb = c->fill_src;
    hb.assign(p.fills.size(), nullptr);
    if (c->tier) {
        // in fill order; a fill served from staging is a use without a read
        std::vector<int32_t> ex(p.fills.size());
        std::vector<char> touch(p.fills.size());
        for (size_t i = 0; i < p.fills.size(); ++i) {
            ex[i] = p.fills[i].expert;
            touch[i] = staged[i] >= 0;
        }
        const int rc = tier_fetch(c, layer, ex.data(), (int)ex.size(), hb.data(), touch.data());
        if (rc) return rc;
    } else {
        for (size_t i = 0; i < p.fills.size(); ++i) hb[i] = c->host_blocks[layer][p.fills[i].expert];
    }
    // runs of consecutive experts into consecutive slots whose host blocks are contiguous
    std::vector<std::pair<size_t, size_t>> &runs = c->runs;
    runs.clear();
    for (size_t i = 0; i < p.fills.size();) {
        if (staged[i] >= 0) {
            ++i;
            continue;
        }
        size_t n = 1;
        while (i + n < p.fills.size() && staged[i + n] < 0 && p.fills[i + n].expert == p.fills[i].expert + (int)n &&
               p.fills[i + n].slot == p.fills[i].slot + (int)n && hb[i + n] == hb[i] + n * c->S)
            ++n;
        runs.push_back({i, n});
        i += n;
    }
    // a wave of many runs spreads them over two streams: two copies in flight move about
    // 10 % more over the link than one (measured at 16 experts; no gain at 4)
    const bool two = runs.size() >= kTwoStreamRuns;
    if (wait_seq >= 0 && (uint64_t)wait_seq >= c->completed_seq) {
        for (hipStream_t cs : {c->copy_stream, two ? c->copy_stream2 : nullptr})
            if (cs && (e = hipStreamWaitEvent(cs, c->reader_ring[wait_seq % kReaderRing], 0)) != hipSuccess)
                return hip_fail(e, "hipStreamWaitEvent(reader)");
    }
    for (size_t r = 0; r < runs.size(); ++r) {
        const size_t i = runs[r].first, n = runs[r].second;
        hipStream_t cs = (two && (r & 1)) ? c->copy_stream2 : c->copy_stream;
        if (int rc = pre_upload(c, c->slot_ptr(layer, p.fills[i].slot), n, cs)) return rc;
        e = hipMemcpyAsync(c->slot_ptr(layer, p.fills[i].slot), hb[i], n * c->S, hipMemcpyHostToDevice, cs);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(H2D)");
        c->h2d_copied += n * c->S;
        c->demand_q.issued += n * c->S;
    }
    if (two && ((e = hipEventRecord(c->ev_copy2, c->copy_stream2)) != hipSuccess ||
                (e = hipStreamWaitEvent(c->copy_stream, c->ev_copy2, 0)) != hipSuccess))
        return hip_fail(e, "second upload stream");
    hipEvent_t ev = c->fill_ring[c->fill_next];
    c->fill_next = (c->fill_next + 1) % kFillRing;
    if ((e = hipEventRecord(ev, c->copy_stream)) != hipSuccess) return hip_fail(e, "hipEventRecord(fill)");
    note_copy_mark(c->demand_q, ev);
    // copies on copy_stream2 are joined into copy_stream before ev (ev_copy2)
    tier_fence(c, hb.data(), (int)hb.size(), ev, kTierCopy);
    *fill_ev = ev;
    return MOE_OK;
}

// Speculative uploads of the picks of layers l+1 .. l+n_spec computed on this
// layer's input, into the staging bank (NVMe page, "Workflow": the next layer's
// router on the current layer's input starts copies one layer early; prefetch in
// the idle gap).  They go on streams of their own, so a demand upload of a later call
// never waits behind them; the streams share the link.  Uploads for the next layers
// (d <= kNearDepth) take the second demand stream and the last kNearSlots staging slots,
// the others the speculation stream and the rest of the bank: an upload needed a layer or
// two from now does not queue behind guesses for layers further ahead.  After the uploads for a
// layer, ev_staged (or ev_near) [layer % kStagedRing] is recorded; each stream is in
// order and keeps to its own slots, so that event covers every upload issued on it
// for that layer.
void prefetch_next(moe_cache *c, int layer, int n_tok, int n_spec) {
    HostClock hc(c->prefetch_us);
    // a staged block outlives the next call's uploads; and speculation yields the link to
    // demand uploads: it only tops the two queues up to pf_backlog experts
    const int queued = (int)(copy_backlog(c) / c->S);
    int budget = std::min(kStageSlots / 2, c->pf_backlog - queued);
    for (int d = 1; d <= n_spec && budget > 0; ++d) {
        const int nl = layer + d;
        if (nl >= c->L || !c->layer_ready[nl]) break;
        const int32_t *spec = c->h_spec + (size_t)(d - 1) * n_tok * c->k;
        std::vector<int32_t> want;
        for (int i = 0; i < n_tok * c->k; ++i) {
            const int32_t e = spec[i];
            if (e < 0 || e >= c->E) continue;
            if (std::find(want.begin(), want.end(), e) != want.end()) continue;
            if (c->pl.slot_of(nl, e) >= 0) continue;            // already resident
            const int64_t key = (int64_t)nl * c->E + e;
            if (c->tier && c->tier->block_of[key] < 0) continue;   // a guess never reads the file
            bool staged = false;
            for (int s = 0; s < kStageSlots; ++s)
                if (c->stage_key[s] == key) staged = true;
            if (!staged) want.push_back(e);
        }
        c->pf_candidates += want.size();
        if ((int)want.size() > budget) {
            c->pf_deferred += want.size() - std::max(budget, 0);
            want.resize(std::max(budget, 0));
        }
        const bool near = d <= kNearDepth;
        const int lo = near ? kStageSlots - kNearSlots : 0, n_part = near ? kNearSlots : kStageSlots - kNearSlots;
        int &next = near ? c->near_next : c->stage_next;
        // near uploads share copy_stream2 (the second demand stream, used by waves of many runs):
        // a stream fewer, so a cache's streams and the compute stream fit in four hardware queues
        hipStream_t st = near ? c->copy_stream2 : c->spec_stream;
        moe_cache::CopyQueue &q = near ? c->near_q : c->spec_q;
        bool issued = false;
        std::vector<const uint8_t *> srcs;
        for (int32_t e : want) {
            int s = next, tries = 0;
            while (c->stage_busy[s] == c->call_no && tries < n_part) {   // read by this call's kernels
                s = lo + (s - lo + 1) % n_part;
                ++tries;
            }
            if (tries == n_part) break;
            next = lo + (s - lo + 1) % n_part;
            if (c->stage_key[s] >= 0 && !c->stage_used[s]) c->pf_wasted += 1;
            // a staging slot is written only here, always by the same stream, and read only by
            // kernels of the call that claims it (busy marking above); the stream keeps its
            // uploads in order
            const uint8_t *src = c->tier ? c->tier->ram + (size_t)c->tier->block_of[(size_t)nl * c->E + e] * c->S
                                         : c->host_blocks[nl][e];
            srcs.push_back(src);
            if (pre_upload(c, c->staging + (size_t)s * c->S, 1, st) != MOE_OK ||
                hipMemcpyAsync(c->staging + (size_t)s * c->S, src, c->S, hipMemcpyHostToDevice, st) != hipSuccess) {
                c->stage_key[s] = -1;
                continue;
            }
            c->stage_key[s] = (int64_t)nl * c->E + e;
            c->stage_used[s] = 0;
            c->pf_issued += 1;
            c->h2d_copied += c->S;
            q.issued += c->S;
            --budget;
            issued = true;
        }
        hipEvent_t ev = near ? c->ev_near[nl % kStagedRing] : c->ev_staged[nl % kStagedRing];
        if (issued && hipEventRecord(ev, st) == hipSuccess) {
            (near ? c->near_for : c->staged_for)[nl % kStagedRing] = nl;
            note_copy_mark(q, ev);
            tier_fence(c, srcs.data(), (int)srcs.size(), ev, near ? kTierNear : kTierSpec);
        } else if (!srcs.empty() && c->tier) {
            // no event covers these copies: the blocks wait for the stream itself
            hipStreamSynchronize(st);
        }
    }
}

// ----------------------------------------------------------------------------- routing readback

// The host learns a decode call's routing from host-mapped memory that the
// selection kernel writes (ids, gates and speculative ids).  Before the launch
// every entry the host will read holds a sentinel no result can take (id -1,
// gate -1.0f: gates are softmax probabilities); the results are complete once
// none is left.  Watching the memory is a shorter round trip than an event's
// completion signal.  While sentinels remain the stream is queried now and
// then, so a failed stream, or one that drained without writing, is reported
// instead of waited on.
constexpr uint32_t kGateSentinel = 0xBF800000u;   // -1.0f

void mark_routing(moe_cache *c, int st, int n_tok, int n_spec) {
    const int nk = n_tok * c->k;
    const moe_cache::RouteSet &r = c->rs[st];
    uint32_t *g = reinterpret_cast<uint32_t *>(r.gate);
    for (int i = 0; i < nk; ++i) {
        r.ids[i] = -1;
        g[i] = kGateSentinel;
    }
    for (int i = 0; i < n_spec * nk; ++i) r.spec[i] = -1;
}

bool routing_written(const moe_cache *c, int n_tok, int n_spec, int &from) {
    const int nk = n_tok * c->k;
    const volatile int32_t *ids = c->h_ids;
    const volatile uint32_t *g = reinterpret_cast<const volatile uint32_t *>(c->h_gate);
    const volatile int32_t *spec = c->h_spec;
    for (; from < nk * (2 + n_spec); ++from) {
        const int i = from;
        const bool ok = i < nk ? ids[i] != -1 : (i < 2 * nk ? g[i - nk] != kGateSentinel : spec[i - 2 * nk] != -1);
        if (!ok) return false;
    }
    return true;
}

int wait_routing(moe_cache *c, hipStream_t stream, int n_tok, int n_spec) {
    int from = 0;
    const double t0 = now_us();
    for (unsigned it = 1; !routing_written(c, n_tok, n_spec, from); ++it) {
        if ((it & 1023u) || now_us() - t0 < 100.0) continue;
        const hipError_t q = hipStreamQuery(stream);
        if (q == hipErrorNotReady) continue;
        if (q != hipSuccess) return hip_fail(q, "router (stream query)");
        if (!routing_written(c, n_tok, n_spec, from))
            return set_error(MOE_ERR_HIP, "the stream drained without the router writing its results");
        break;
    }
    std::atomic_thread_fence(std::memory_order_acquire);
    return MOE_OK;
}

// ----------------------------------------------------------------------------- decode

double gemv_bytes(const moe_cache *c, int n_units, int n_pairs, int n_mats, int n_copy) {
    const size_t cols = n_mats == 2 ? c->H : c->I;
    const size_t rows = n_mats == 2 ? c->I : c->H;
    const double w = (double)(n_units + n_copy) * n_mats * matrix_bytes(c->quant, rows, cols);
    const double act = c->quant == MOE_Q_F32 ? 4.0 : 2.0;
    // weights read (+ written for copy-through), activation vectors read, outputs written
    return w + (double)n_pairs * (cols * act + rows * (n_mats == 2 ? act : 4.0));
}

int launch_units(moe_cache *c, int layer, int n_mats, const Units &units, size_t b, size_t e,
                 const void *shared_w, const void *vec, int n_tok, hipStream_t stream) {
    if (b >= e) return MOE_OK;
    std::vector<moe::UnitList> &lists = c->lists;
    pack_units(units, b, e, lists);
    moe::GemvArgs a{};
    a.bank = c->pool_base(layer);
    a.staging = c->staging;
    a.shared_w = (const uint8_t *)shared_w;
    a.copy_bank = const_cast<uint8_t *>(c->pool_base(layer));
    a.block_bytes = c->S;
    const size_t mg = matrix_bytes(c->quant, c->I, c->H);
    a.mat_off0 = n_mats == 2 ? 0 : 2 * mg;
    a.mat_off1 = mg;
    a.rows = n_mats == 2 ? c->I : c->H;
    a.cols = n_mats == 2 ? c->H : c->I;
    a.vec = vec;
    a.vec_by_token = n_mats == 2;
    a.nk = n_tok * c->k;
    a.top_k = c->k;
    a.out = n_mats == 2 ? (void *)c->d_h : (void *)c->d_y;
    const moe::GemvShape sh = moe::gemv_shape(c->quant, a.cols, n_mats);
    a.tiles_per_unit = (a.rows + sh.rows_per_wg - 1) / sh.rows_per_wg;
    for (size_t i = 0; i < lists.size(); ++i) {
        const int np = lists[i].pbeg[lists[i].n_units];
        int n_copy = 0;
        for (int u = 0; u < lists[i].n_units; ++u) n_copy += lists[i].copy_to[u] >= 0;
        const double bytes = gemv_bytes(c, lists[i].n_units, np, n_mats, n_copy);
        const double flops = 2.0 * np * (double)a.rows * a.cols * n_mats;
        TimeScope ts(c, n_mats == 2 ? 1 : 2, bytes, flops);
        hipError_t err;
        {
            HostClock hc(c->launch_us);
            err = moe::launch_expert_gemv(c->quant, n_mats, a, lists[i], stream, ts.a, ts.b);
        }
        if (err != hipSuccess) return hip_fail(err, "expert GEMV launch");
    }
    return MOE_OK;
}

// Down projection and combine of one wave (tokens t0 .. t1-1).  A wave whose
// units and pairs fit one launch list takes the fused kernel; a larger one the
// unit-tiled down GEMV and then the combine of its tokens.
// Slot-table entries a plan changed, as (key layer*E+e, slot or -1); none (and false) if
// more than fit in one down launch's arguments: the device copy then keeps stale entries.
bool map_updates(const moe_cache *c, int layer, const moe::WavePlan &p, moe::CombineArgs &cb) {
    cb.n_upd = 0;
    const int n = (int)(p.evictions.size() + p.fills.size());
    if (n > moe::kMaxMapUpdates || !c->d_map) return false;
    for (const moe::Eviction &ev : p.evictions) {
        cb.upd_key[cb.n_upd] = c->pl.shared_pool() ? (int32_t)ev.key : (int32_t)((int64_t)layer * c->E + ev.key);
        cb.upd_val[cb.n_upd++] = -1;
    }
    for (const moe::Fill &f : p.fills) {
        cb.upd_key[cb.n_upd] = (int32_t)((int64_t)layer * c->E + f.expert);
        cb.upd_val[cb.n_upd++] = f.slot;
    }
    cb.map = c->d_map;
    return true;
}

int down_and_combine(moe_cache *c, int layer, const Units &units, const void *shared_w, int n_tok,
                     int t0, int t1, const float *x, float *out, bool residual, bool has_shared, hipStream_t stream,
                     const moe::WavePlan *plan = nullptr) {
    std::vector<moe::UnitList> &lists = c->lists;
    pack_units(units, 0, units.u.size(), lists);
    if (lists.size() == 1) {
        moe::GemvArgs a{};
        a.bank = c->pool_base(layer);
        a.staging = c->staging;
        a.shared_w = (const uint8_t *)shared_w;
        a.copy_bank = const_cast<uint8_t *>(c->pool_base(layer));
        a.block_bytes = c->S;
        a.mat_off0 = 2 * matrix_bytes(c->quant, c->I, c->H);
        a.rows = c->H;
        a.cols = c->I;
        a.vec = c->d_h;
        a.vec_by_token = 0;
        a.nk = n_tok * c->k;
        a.top_k = c->k;
        moe::CombineArgs cb{};
        cb.x = residual ? x : nullptr;
        cb.gate = c->d_gate;
        cb.out = out;
        cb.t0 = t0;
        cb.nt = t1 - t0;
        cb.has_shared = has_shared ? 1 : 0;
        // the plan's slot-table changes ride along (when they fit); the shadow follows once the
        // launch is in
        if (plan) map_updates(c, layer, *plan, cb);
        const moe::UnitList &ul = lists[0];
        const int np = ul.pbeg[ul.n_units];
        int n_copy = 0;
        for (int u = 0; u < ul.n_units; ++u) n_copy += ul.copy_to[u] >= 0;
        const double bytes = gemv_bytes(c, ul.n_units, np, 1, n_copy) + (double)(t1 - t0) * c->H * 4 * (residual ? 2 : 1);
        TimeScope ts(c, 2, bytes, 2.0 * np * (double)c->H * c->I);
        hipError_t err;
        {
            HostClock hc(c->launch_us);
            err = moe::launch_down_combine(c->quant, a, cb, ul, stream, ts.a, ts.b);
        }
        if (err != hipSuccess) return hip_fail(err, "down+combine launch");
        for (int i = 0; i < cb.n_upd; ++i) c->map_shadow[cb.upd_key[i]] = cb.upd_val[i];
        return MOE_OK;
    }
    int rc = launch_units(c, layer, 1, units, 0, units.u.size(), shared_w, c->d_h, n_tok, stream);
    if (rc) return rc;
    hipError_t err = moe::launch_combine(x, c->d_y, c->d_gate, out, n_tok, t0, t1 - t0, c->H, c->k, has_shared,
                                         residual ? 1 : 0, stream);
    if (err != hipSuccess) return hip_fail(err, "combine launch");
    return MOE_OK;
}

// Gate/up of units [b, e) and the down projection + combine of the whole wave in
// one launch (k_expert_fused), where the shape and the list sizes allow it:
// the down weights stream while the gate/up workgroups run.  *done = false,
// with nothing launched, where they do not (the caller launches the two kernels).
int fused_expert_launch(moe_cache *c, int layer, const Units &units, size_t b, size_t e, const void *shared_w,
                        const void *gu_vec, int n_tok, int t0, int t1, const float *x, float *out, bool residual,
                        bool has_shared, hipStream_t stream, bool *done) {
    *done = false;
    if (!c->fuse_decode || b >= e) return MOE_OK;
    pack_units(units, b, e, c->lists);
    pack_units(units, 0, units.u.size(), c->lists_down);
    if (c->lists.size() != 1 || c->lists_down.size() != 1) return MOE_OK;
    const moe::UnitList &ulg = c->lists[0], &uld = c->lists_down[0];

    moe::GemvArgs g{};
    g.bank = c->pool_base(layer);
    g.staging = c->staging;
    g.shared_w = (const uint8_t *)shared_w;
    g.copy_bank = const_cast<uint8_t *>(c->pool_base(layer));
    g.block_bytes = c->S;
    const size_t mg = matrix_bytes(c->quant, c->I, c->H);
    g.mat_off0 = 0;
    g.mat_off1 = mg;
    g.rows = c->I;
    g.cols = c->H;
    g.vec = gu_vec;
    g.vec_by_token = 1;
    g.nk = n_tok * c->k;
    g.top_k = c->k;
    g.out = c->d_h;
    const moe::GemvShape gs = moe::gemv_shape(c->quant, c->H, 2);
    g.tiles_per_unit = (c->I + gs.rows_per_wg - 1) / gs.rows_per_wg;

    moe::GemvArgs d = g;
    d.mat_off0 = 2 * mg;
    d.mat_off1 = 0;
    d.rows = c->H;
    d.cols = c->I;
    d.vec = c->d_h;
    d.vec_by_token = 0;
    d.out = c->d_y;
    d.tiles_per_unit = 0;

    moe::CombineArgs cb{};
    cb.x = residual ? x : nullptr;
    cb.gate = c->d_gate;
    cb.out = out;
    cb.t0 = t0;
    cb.nt = t1 - t0;
    cb.has_shared = has_shared ? 1 : 0;

    moe::FusedSync fs{};
    fs.sync = c->d_fused_sync;
    fs.n_gu = ulg.n_units * g.tiles_per_unit;
    fs.epoch = c->fused_epoch + 1;
    fs.timed_out = c->h_fused_timeout_dev;

    const int npg = ulg.pbeg[ulg.n_units], npd = uld.pbeg[uld.n_units];
    int copy_g = 0, copy_d = 0;
    for (int u = 0; u < ulg.n_units; ++u) copy_g += ulg.copy_to[u] >= 0;
    for (int u = 0; u < uld.n_units; ++u) copy_d += uld.copy_to[u] >= 0;
    const double bytes = gemv_bytes(c, ulg.n_units, npg, 2, copy_g) + gemv_bytes(c, uld.n_units, npd, 1, copy_d) +
                         (double)(t1 - t0) * c->H * 4 * (residual ? 2 : 1);
    const double flops = 2.0 * npg * (double)c->I * c->H * 2 + 2.0 * npd * (double)c->H * c->I;
    hipError_t err;
    {
        TimeScope ts(c, 5, bytes, flops);
        {
            HostClock hc(c->launch_us);
            err = moe::launch_expert_fused(c->quant, g, ulg, d, cb, uld, fs, stream, ts.a, ts.b);
        }
        if (err == hipErrorNotSupported) {
            // nothing was launched: hand the events back instead of recording an empty timing
            if (ts.a) c->event_pool.push_back(ts.a);
            if (ts.b) c->event_pool.push_back(ts.b);
            ts.a = ts.b = nullptr;
            return MOE_OK;
        }
    }
    if (err != hipSuccess) return hip_fail(err, "fused expert launch");
    c->fused_epoch = fs.epoch;
    *done = true;
    return MOE_OK;
}

// Gate/up of a one-token call's resident picks (and the shared expert), launched before the
// host plans, from the router's device ids and the device copy of the slot table.  Its
// timing record is completed by the caller once the plan tells which units it computed.
void pre_args(const moe_cache *c, int layer, const void *shared_w, const void *vec, moe::GemvArgs &a,
              moe::PreArgs &pa) {
    a = moe::GemvArgs{};
    a.bank = c->pool_base(layer);
    a.staging = c->staging;
    a.shared_w = (const uint8_t *)shared_w;
    a.copy_bank = const_cast<uint8_t *>(c->pool_base(layer));
    a.block_bytes = c->S;
    a.mat_off0 = 0;
    a.mat_off1 = matrix_bytes(c->quant, c->I, c->H);
    a.rows = c->I;
    a.cols = c->H;
    a.vec = vec;
    a.vec_by_token = 1;
    a.nk = c->k;
    a.top_k = c->k;
    a.out = c->d_h;
    a.tiles_per_unit = (c->I + moe::gemv_shape(c->quant, c->H, 2).rows_per_wg - 1) /
                       moe::gemv_shape(c->quant, c->H, 2).rows_per_wg;
    pa = moe::PreArgs{};
    pa.ids = c->d_ids;
    pa.map = c->d_map;
    pa.map_base = layer * c->E;
    pa.n_experts = c->E;
    pa.n_routed = c->k;
    pa.has_shared = shared_w ? 1 : 0;
}

int prelaunch_gate_up(moe_cache *c, int layer, const void *shared_w, const void *vec, hipStream_t stream,
                      hipEvent_t *ev_a, hipEvent_t *ev_b) {
    moe::GemvArgs a;
    moe::PreArgs pa;
    pre_args(c, layer, shared_w, vec, a, pa);
    TimeScope ts(c, 6, 0.0, 0.0);
    hipError_t err;
    {
        HostClock hc(c->launch_us);
        err = moe::launch_expert_gemv_pre(c->quant, a, pa, stream, ts.a, ts.b);
    }
    *ev_a = ts.a;
    *ev_b = ts.b;
    ts.a = ts.b = nullptr;    // recorded by the caller with the bytes it turns out to have read
    if (err != hipSuccess) {
        if (*ev_a) c->event_pool.push_back(*ev_a);
        if (*ev_b) c->event_pool.push_back(*ev_b);
        *ev_a = *ev_b = nullptr;
        return hip_fail(err, "expert GEMV launch (resident picks)");
    }
    return MOE_OK;
}

// Launch a decode call's router, writing its host results into routing set st, and for
// one token the early gate/up of its resident picks; c->ahead describes the call.
int issue_route(moe_cache *c, int layer, const float *x, int n_tok, const float *router_w, const void *shared_w,
                const float *const *spec_ws, int n_spec, hipStream_t stream, int st) {
    const bool f32 = c->quant == MOE_Q_F32;
    const moe_cache::RouteSet &r = c->rs[st];
    moe::RouterArgs ra{};
    ra.x = x;
    ra.xq = f32 ? nullptr : c->d_xq;
    ra.quant = c->quant;
    ra.w0 = router_w;
    for (int d = 0; d < n_spec; ++d) ra.wspec[d] = spec_ws[d];
    ra.n_spec = n_spec;
    ra.n_tok = n_tok;
    ra.E = c->E;
    ra.H = c->H;
    ra.top_k = c->k;
    ra.z = c->d_z;
    ra.ids = c->d_ids;
    ra.gate = c->d_gate;
    ra.ids_host = r.ids_dev;
    ra.gate_host = r.gate_dev;
    ra.spec_ids_host = n_spec > 0 ? r.spec_dev : nullptr;
    ra.tickets = c->d_tickets;
    mark_routing(c, st, n_tok, n_spec);
    hipError_t err;
    {
        const double bytes = (double)(1 + n_spec) * c->E * c->H * 4 + (double)n_tok * c->H * 4;
        TimeScope ts(c, 0, bytes, 2.0 * (1 + n_spec) * c->E * (double)c->H * n_tok);
        HostClock hc(c->launch_us);
        if ((err = moe::launch_router(ra, stream, ts.a, ts.b)) != hipSuccess) return hip_fail(err, "router launch");
    }
    moe_cache::Ahead a;
    a.on = true;
    a.layer = layer;
    a.n_tok = n_tok;
    a.n_spec = n_spec;
    a.set = st;
    a.x = x;
    a.stream = stream;
    // one token: the resident picks' gate/up go out at once, before the host trip; the plan
    // then launches only what that did not cover
    a.pre = n_tok == 1 && c->prelaunch && !c->fuse_decode;
    if (a.pre) {
        const int rc = prelaunch_gate_up(c, layer, shared_w, f32 ? (const void *)x : c->d_xq, stream, &a.pre_a,
                                         &a.pre_b);
        if (rc) return rc;
    }
    c->ahead = a;
    return MOE_OK;
}

// Speculation: the routers of the layers after `layer` (as many as given, up to kMaxSpec).
int spec_count(const moe_cache *c, int layer, const float *const *spec_ws, int n_spec_in) {
    int n = 0;
    if (c->staging)
        while (n < std::min(n_spec_in, moe::kMaxSpec) && spec_ws[n] && layer + n + 1 < c->L) ++n;
    return n;
}

// ----------------------------------------------------------------------------- captured steps
//
// When every expert of every layer holds a slot, a one-token decode step needs no host
// decision: every pick is a hit, so nothing is uploaded or evicted, and the units of each
// layer follow from the router's ids and the device copy of the slot table.  Such a step
// is captured once (per set of routing results and per input, output and weight pointers)
// as a graph of the layers' router, early gate/up and device-listed down + combine
// launches, and replayed: one submission for the whole stack, no host round trip between
// layers (SGLang page, "What happens with more than one request?": the single-wave step is
// the one a graph can hold; NVMe page, "Workflow": graphs for one-token layers cut the
// CPU-GPU synchronisation).  The host replays the step's plans from the routing results
// afterwards, which keeps the recency order, the counters and the trace records those of
// the uncaptured path.

// Every (layer, expert) holds a slot, and the device copy of the slot table is made exact.
// Checked again only after a plan changed residency.
int check_resident(moe_cache *c, hipStream_t stream) {
    if (c->resident_checked == c->plan_changes) return MOE_OK;
    c->all_resident = false;
    for (int l = 0; l < c->L; ++l)
        for (int e = 0; e < c->E; ++e)
            if (c->pl.slot_of(l, e) < 0) {
                c->resident_checked = c->plan_changes;
                return MOE_OK;
            }
    // the shadow is what the device copy holds once the enqueued updates ran; entries a
    // plan could not pass along (too many changes in one wave) are written here
    bool exact = true;
    for (int l = 0; l < c->L; ++l)
        for (int e = 0; e < c->E; ++e) {
            const size_t key = (size_t)l * c->E + e;
            if (c->map_shadow[key] != c->pl.slot_of(l, e)) {
                c->map_shadow[key] = c->pl.slot_of(l, e);
                exact = false;
            }
        }
    if (!exact) {
        hipError_t e = hipMemcpyAsync(c->d_map, c->map_shadow.data(), c->map_shadow.size() * sizeof(int32_t),
                                      hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e, "slot table copy");
    }
    c->all_resident = true;
    c->resident_checked = c->plan_changes;
    return MOE_OK;
}

// Apply the plans of the captured step in flight, once it has finished: per layer the
// one-wave plan of its routed ids (all hits), its counters and its trace record.
int flush_graph(moe_cache *c) {
    if (c->sg_pending < 0) return MOE_OK;
    moe_cache::StepGraph &g = c->sg[c->sg_pending];
    c->sg_pending = -1;
    {
        HostClock hc(c->wait_us);
        const hipError_t e = hipEventSynchronize(g.done);
        if (e != hipSuccess) return hip_fail(e, "captured step");
    }
    if (*(volatile int *)c->h_graph_bad)
        return set_error(MOE_ERR_HIP, "a captured decode step found a pick without a slot; its outputs are not valid");
    HostClock hp(c->plan_us);
    for (int l = 0; l < c->L; ++l) {
        const int32_t *ids = g.ids + (size_t)l * c->k;
        const float *gate = g.gate + (size_t)l * c->k;
        if (l == 0) c->pl.begin_step();
        if (c->pl.waves(l, 1, ids, c->wave_ranges) != moe::PLAN_OK || c->wave_ranges.size() != 1)
            return set_error(MOE_ERR_INVALID, "captured step: the routing does not plan as one wave");
        const int rc = c->pl.plan(l, ids, 0, 1, 0, c->wp);
        if (rc != moe::PLAN_OK) return set_error(MOE_ERR_INVALID, "captured step: router produced an expert id out of range");
        if (!c->wp.fills.empty()) {
            c->pl.rollback(c->wp);
            return set_error(MOE_ERR_INVALID, "captured step: a pick had no slot");
        }
        c->pl.account(c->wp, c->k, c->wp.pick_hits);
        tier_touch(c, l, c->wp.hits.data(), (int)c->wp.hits.size());
        moe::emit_trace(c->wp, c->k, ids, gate, c->trace_fn, c->trace_user);
    }
    // the last layer's routing is the cache's last routing
    memcpy(c->h_ids, g.ids + (size_t)(c->L - 1) * c->k, c->k * sizeof(int32_t));
    memcpy(c->h_gate, g.gate + (size_t)(c->L - 1) * c->k, c->k * sizeof(float));
    return MOE_OK;
}

// Before any other use of the cache: the captured step in flight is applied, and a step
// that found a pick without a slot keeps failing every forward call.
int graph_sync(moe_cache *c) {
    if (c->h_graph_bad && *(volatile int *)c->h_graph_bad)
        return set_error(MOE_ERR_HIP, "a captured decode step found a pick without a slot; outputs since then are "
                                      "not valid");
    return flush_graph(c);
}

// Capture the step for (out, layer_inputs, router_ws, shared_ws) into g: per layer a copy
// of its input into layer_inputs (when given), the router (its results into the layer's
// row of d_gids / d_ggate), the early gate/up of every pick and the down + combine with
// the residual, layer 0 reading d_gx, layer l writing the stack's ping-pong buffer (the
// last: out); then one copy of all layers' routing results into g's host arrays.
int capture_step(moe_cache *c, moe_cache::StepGraph &g, const float *const *router_ws, const void *const *shared_ws,
                 float *out, float *layer_inputs) {
    hipError_t e;
    if (g.exec) {
        hipGraphExecDestroy(g.exec);
        g.exec = nullptr;
    }
    if (!c->cap_stream && (e = hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking)) != hipSuccess)
        return hip_fail(e, "capture stream");
    const bool f32 = c->quant == MOE_Q_F32;
    const bool has_shared = (c->flags & MOE_SHARED_EXPERT) != 0;
    if ((e = hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal)) != hipSuccess)
        return hip_fail(e, "hipStreamBeginCapture");
    const float *in = c->d_gx;
    for (int l = 0; l < c->L && e == hipSuccess; ++l) {
        float *dst = (l == c->L - 1) ? out : c->d_stack[l & 1];
        const void *shared_w = has_shared ? shared_ws[l] : nullptr;
        if (layer_inputs &&
            (e = hipMemcpyAsync(layer_inputs + (size_t)l * c->H, in, (size_t)c->H * sizeof(float),
                                hipMemcpyDeviceToDevice, c->cap_stream)) != hipSuccess)
            break;
        moe::RouterArgs ra{};
        ra.x = in;
        ra.xq = f32 ? nullptr : c->d_xq;
        ra.quant = c->quant;
        ra.w0 = router_ws[l];
        ra.n_spec = 0;
        ra.n_tok = 1;
        ra.E = c->E;
        ra.H = c->H;
        ra.top_k = c->k;
        ra.z = c->d_z;
        int32_t *ids = c->d_gids + (size_t)l * c->k;
        float *gate = c->d_ggate + (size_t)l * c->k;
        ra.ids = ids;
        ra.gate = gate;
        ra.ids_host = nullptr;
        ra.gate_host = nullptr;
        ra.spec_ids_host = nullptr;
        ra.tickets = c->d_tickets;
        if ((e = moe::launch_router(ra, c->cap_stream)) != hipSuccess) break;
        moe::GemvArgs a;
        moe::PreArgs pa;
        pre_args(c, l, shared_w, f32 ? (const void *)in : c->d_xq, a, pa);
        pa.ids = ids;
        if ((e = moe::launch_expert_gemv_pre(c->quant, a, pa, c->cap_stream)) != hipSuccess) break;
        moe::GemvArgs d{};
        d.bank = c->pool_base(l);
        d.staging = c->staging;
        d.shared_w = (const uint8_t *)shared_w;
        d.copy_bank = const_cast<uint8_t *>(c->pool_base(l));
        d.block_bytes = c->S;
        d.mat_off0 = 2 * matrix_bytes(c->quant, c->I, c->H);
        d.rows = c->H;
        d.cols = c->I;
        d.vec = c->d_h;
        d.vec_by_token = 0;
        d.nk = c->k;
        d.top_k = c->k;
        moe::CombineArgs cb{};
        cb.x = in;
        cb.gate = gate;
        cb.out = dst;
        cb.t0 = 0;
        cb.nt = 1;
        cb.has_shared = has_shared ? 1 : 0;
        cb.map = c->d_map;
        cb.n_upd = 0;
        if ((e = moe::launch_down_combine_picks(c->quant, d, cb, pa, c->h_graph_bad_dev, c->cap_stream)) !=
            hipSuccess)
            break;
        in = dst;
    }
    const size_t nr = (size_t)c->L * c->k;
    if (e == hipSuccess)
        e = hipMemcpyAsync(g.ids, c->d_gids, nr * sizeof(int32_t), hipMemcpyDeviceToHost, c->cap_stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(g.gate, c->d_ggate, nr * sizeof(float), hipMemcpyDeviceToHost, c->cap_stream);
    hipGraph_t graph = nullptr;
    const hipError_t ee = hipStreamEndCapture(c->cap_stream, &graph);
    if (e == hipSuccess) e = ee;
    if (e == hipSuccess) e = hipGraphInstantiate(&g.exec, graph, nullptr, nullptr, 0);
    if (graph) hipGraphDestroy(graph);
    if (e != hipSuccess) {
        g.exec = nullptr;
        return hip_fail(e, "decode step capture");
    }
    g.out = out;
    g.layer_inputs = layer_inputs;
    g.routers.assign(router_ws, router_ws + c->L);
    g.shared.assign(c->L, nullptr);
    if (has_shared) g.shared.assign(shared_ws, shared_ws + c->L);
    return MOE_OK;
}

// One-token stack call as a captured step, where it qualifies (*done); else nothing is
// done and the caller takes the regular path.
int graph_step(moe_cache *c, const float *x, const float *const *router_ws, const void *const *shared_ws,
               float *out, float *layer_inputs, hipStream_t stream, bool *done) {
    *done = false;
    const bool has_shared = (c->flags & MOE_SHARED_EXPERT) != 0;
    if (c->h_graph_bad && *(volatile int *)c->h_graph_bad) return graph_sync(c);
    if (!c->graph_on || c->pl.adaptive() || c->k + (has_shared ? 1 : 0) > 16) return MOE_OK;
    for (int l = 0; l < c->L; ++l)
        if (!c->layer_ready[l]) return MOE_OK;
    HostClock hc(c->call_us);
    discard_ahead(c);
    hipError_t e;
    if (c->have_last_stream && c->last_stream != stream) {
        if ((e = hipStreamSynchronize(c->last_stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
        c->completed_seq = c->reader_seq;
    }
    int rc = check_resident(c, stream);
    if (rc || !c->all_resident) return rc;
    const unsigned hf = hipHostMallocMapped | hipHostMallocCoherent;
    if (!c->h_graph_bad_dev) {
        if (!c->h_graph_bad) {
            if ((e = hipHostMalloc((void **)&c->h_graph_bad, sizeof(int), hf)) != hipSuccess) {
                c->h_graph_bad = nullptr;
                return set_error(MOE_ERR_OOM, "pinned flag");
            }
            *c->h_graph_bad = 0;
        }
        if ((e = hipHostGetDevicePointer((void **)&c->h_graph_bad_dev, c->h_graph_bad, 0)) != hipSuccess) {
            c->h_graph_bad_dev = nullptr;
            return hip_fail(e, "hipHostGetDevicePointer");
        }
    }
    moe_cache::StepGraph &g = c->sg[c->sg_next];
    const size_t nr = (size_t)c->L * c->k;
    // each buffer on its own, so that a failed allocation is retried by the next call
    if (!g.ids && (e = hipHostMalloc((void **)&g.ids, nr * sizeof(int32_t), hipHostMallocDefault)) != hipSuccess) {
        g.ids = nullptr;
        return set_error(MOE_ERR_OOM, "pinned routing results");
    }
    if (!g.gate && (e = hipHostMalloc((void **)&g.gate, nr * sizeof(float), hipHostMallocDefault)) != hipSuccess) {
        g.gate = nullptr;
        return set_error(MOE_ERR_OOM, "pinned routing results");
    }
    if (!c->d_gids && (e = hipMalloc(&c->d_gids, nr * sizeof(int32_t))) != hipSuccess) {
        c->d_gids = nullptr;
        return set_error(MOE_ERR_OOM, "routing result buffers");
    }
    if (!c->d_ggate && (e = hipMalloc(&c->d_ggate, nr * sizeof(float))) != hipSuccess) {
        c->d_ggate = nullptr;
        return set_error(MOE_ERR_OOM, "routing result buffers");
    }
    if (!g.done && (e = hipEventCreateWithFlags(&g.done, hipEventDisableTiming)) != hipSuccess)
        return hip_fail(e, "event creation");
    if (!c->d_gx && (e = hipMalloc(&c->d_gx, (size_t)c->H * sizeof(float))) != hipSuccess)
        return set_error(MOE_ERR_OOM, "captured step input buffer");
    bool same = g.exec && g.out == out && g.layer_inputs == layer_inputs;
    for (int l = 0; same && l < c->L; ++l)
        same = g.routers[l] == router_ws[l] && g.shared[l] == (has_shared ? shared_ws[l] : nullptr);
    if (!same && (rc = capture_step(c, g, router_ws, shared_ws, out, layer_inputs)) != MOE_OK) return rc;
    {
        HostClock hl(c->launch_us);
        // the input is copied in ahead of the replay, so a new x needs no new graph
        if ((e = hipMemcpyAsync(c->d_gx, x, (size_t)c->H * sizeof(float), hipMemcpyDeviceToDevice, stream)) !=
            hipSuccess)
            return hip_fail(e, "hipMemcpyAsync(step input)");
        if ((e = hipGraphLaunch(g.exec, stream)) != hipSuccess) return hip_fail(e, "hipGraphLaunch");
        if ((e = hipEventRecord(g.done, stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    c->last_stream = stream;
    c->have_last_stream = true;
    c->call_no += c->L;
    c->forwards += c->L;
    c->last_tokens = 1;
    c->graph_steps += 1;
    // the previous captured step (the other set of results) is applied while this one runs
    rc = flush_graph(c);
    c->sg_pending = c->sg_next;
    c->sg_next ^= 1;
    *done = true;
    return rc;
}

// The stack driver's next call, whose router the current call launches once its own
// expert kernels are queued.
struct NextCall {
    const float *x;
    const float *router_w;
    const void *shared_w;
    const float *const *spec_ws;
    int n_spec_in;
};

int decode_forward(moe_cache *c, int layer, const float *x, int n_tok, const float *router_w, const void *shared_w,
                   const float *const *spec_ws, int n_spec_in, float *out, unsigned fflags, hipStream_t stream,
                   const NextCall *next = nullptr) {
    int rc = ensure_route_capacity(c, n_tok);
    if (rc) return rc;
    if (*(volatile int *)c->h_fused_timeout)
        return set_error(MOE_ERR_HIP, "a fused expert kernel stopped waiting for its gate/up workgroups; "
                                      "outputs since then are not valid");
    // speculation: the routers of the next n_spec layers (as many as given, up to kMaxSpec)
    const int n_spec = spec_count(c, layer, spec_ws, n_spec_in);
    const bool spec = n_spec > 0;
    hipError_t err;
    c->call_no += 1;
    if (c->have_last_stream && c->last_stream != stream) {
        // slot reuse is fenced by stream order; a change of stream drains the old one first
        if ((err = hipStreamSynchronize(c->last_stream)) != hipSuccess) return hip_fail(err, "hipStreamSynchronize");
        c->completed_seq = c->reader_seq;
    }
    const bool f32 = c->quant == MOE_Q_F32;

    // the router (and the early gate/up) of this call: launched ahead by the previous call of
    // the stack driver, or now
    if (c->ahead.on && !(c->ahead.layer == layer && c->ahead.n_tok == n_tok && c->ahead.x == x &&
                         c->ahead.stream == stream && c->ahead.n_spec == n_spec))
        discard_ahead(c);
    if (!c->ahead.on && (rc = issue_route(c, layer, x, n_tok, router_w, shared_w, spec_ws, n_spec, stream,
                                          1 - c->rcur)) != MOE_OK)
        return rc;
    use_route_set(c, c->ahead.set);
    const bool pre = c->ahead.pre;
    hipEvent_t pre_a = c->ahead.pre_a, pre_b = c->ahead.pre_b;
    c->ahead = moe_cache::Ahead();
    struct EventsBack {      // timing events of the early launch go back to the pool on an early return
        moe_cache *c;
        hipEvent_t &a, &b;
        ~EventsBack() {
            if (a) c->event_pool.push_back(a);
            if (b) c->event_pool.push_back(b);
        }
    } events_back{c, pre_a, pre_b};
    // the plan needs this layer's ids and gates only; the speculative ids are awaited where
    // they are read, after the first expert launch
    const double tw = now_us();
    if ((rc = wait_routing(c, stream, n_tok, 0)) != MOE_OK) return rc;
    c->wait_us += now_us() - tw;
    // the router kernel started, so every kernel enqueued before it on this stream has finished
    if (c->have_last_stream && c->last_stream == stream) c->completed_seq = c->reader_seq;
    c->last_stream = stream;
    c->have_last_stream = true;

    if (layer == 0) c->pl.begin_step();   // a decode step begins (adaptive capacity rebalances)
    const int wrc = c->pl.waves(layer, n_tok, c->h_ids, c->wave_ranges);
    if (wrc == moe::PLAN_INVALID) return set_error(MOE_ERR_INVALID, "router produced an expert id out of range");
    if (wrc != moe::PLAN_OK) return set_error(MOE_ERR_CACHE_TOO_SMALL, "a token's experts do not fit in the slots");
    const bool has_shared = (c->flags & MOE_SHARED_EXPERT) != 0;
    const int nk = n_tok * c->k;
    const bool multi_wave = c->wave_ranges.size() > 1;
    const void *gu_vec = f32 ? (const void *)x : c->d_xq;
    std::vector<int> staged;

    for (size_t w = 0; w < c->wave_ranges.size(); ++w) {
        const int t0 = c->wave_ranges[w].first, t1 = c->wave_ranges[w].second;
        const double tp = now_us();
        rc = c->pl.plan(layer, c->h_ids, t0, t1, (int)w, c->wp);
        c->plan_us += now_us() - tp;
        if (rc == moe::PLAN_INVALID) return set_error(MOE_ERR_INVALID, "router produced an expert id out of range");
        if (rc == moe::PLAN_TOO_SMALL) return set_error(MOE_ERR_CACHE_TOO_SMALL, "more distinct experts than slots");
        const moe::WavePlan &p = c->wp;
        if (!p.fills.empty() || !p.evictions.empty()) c->plan_changes += 1;

        hipEvent_t fill_ev = nullptr;
        rc = upload_fills(c, layer, p, &fill_ev, staged);
        if (rc) {
            c->pl.rollback(p);
            c->plan_changes += 1;
            return rc;
        }
        c->pl.account(p, (t1 - t0) * c->k, p.pick_hits);
        moe::emit_trace(p, c->k, c->h_ids, c->h_gate, c->trace_fn, c->trace_user);

        // units: shared expert, then hits (first-occurrence order), then fills (ascending);
        // pairs of a unit in (token, rank) order
        Units &units = c->units;
        units.u.clear();
        if (has_shared) units.u.push_back({-1, -1, -1, 0, t1 - t0});
        const size_t first_routed = units.u.size();
        for (int32_t ex : p.hits) {
            c->unit_of[ex] = (int32_t)units.u.size();
            units.u.push_back({c->pl.slot_of(layer, ex), -1, ex, 0, 0});
        }
        const size_t first_fill = units.u.size();
        bool any_staged = false;
        for (size_t i = 0; i < p.fills.size(); ++i) {
            c->unit_of[p.fills[i].expert] = (int32_t)units.u.size();
            if (staged[i] >= 0) {
                units.u.push_back({-2 - staged[i], p.fills[i].slot, p.fills[i].expert, 0, 0});
                any_staged = true;
            } else {
                units.u.push_back({p.fills[i].slot, -1, p.fills[i].expert, 0, 0});
            }
        }
        const int32_t *wid = c->h_ids + (size_t)t0 * c->k;
        const int wn = (t1 - t0) * c->k;
        for (int i = 0; i < wn; ++i) units.u[c->unit_of[wid[i]]].np += 1;
        int n_pairs = 0;
        for (UnitBuild &u : units.u) {
            u.p0 = n_pairs;
            n_pairs += u.np;
            u.np = 0;
        }
        units.pairs.resize(n_pairs);
        if (has_shared) {
            for (int t = t0; t < t1; ++t) units.pairs[units.u[0].np++] = (uint16_t)(nk + t);
        }
        for (int i = 0; i < wn; ++i) {
            UnitBuild &u = units.u[c->unit_of[wid[i]]];
            units.pairs[u.p0 + u.np++] = (uint16_t)(t0 * c->k + i);
        }
        for (size_t u = first_routed; u < units.u.size(); ++u) c->unit_of[units.u[u].expert] = -1;

        // hits (and the shared expert) start at once; fills after their data landed
        // (95 GiB page, "Decode": compute on hits while misses transfer).  Fills served
        // from the staging bank join the hits' launch when their copies have completed.
        // staged fills from either part of the bank wait on that stream's event for this layer
        bool far_pending = false, near_pending = false;
        if (any_staged) {
            bool far_used = false, near_used = false;
            for (size_t i = 0; i < p.fills.size(); ++i) {
                if (staged[i] < 0) continue;
                (staged[i] >= kStageSlots - kNearSlots ? near_used : far_used) = true;
            }
            HostClock hc(c->event_us);
            const int r = layer % kStagedRing;
            if (far_used && c->staged_for[r] == layer) far_pending = hipEventQuery(c->ev_staged[r]) != hipSuccess;
            if (near_used && c->near_for[r] == layer) near_pending = hipEventQuery(c->ev_near[r]) != hipSuccess;
        }
        const bool staged_pending = far_pending || near_pending;
        const bool wait_fills = fill_ev || staged_pending;
        // with the early launch, this wave's own gate/up launches take the units it did not cover:
        // the fills, and any hit the device copy of the slot table did not show at its slot
        const Units *gu = &units;
        size_t gu_fill = first_fill;
        if (pre) {
            Units &g = c->units_gu;
            g.u.clear();
            g.pairs.clear();
            gu_fill = 0;
            int n_cov = 0, np_cov = 0;
            for (size_t i = 0; i < units.u.size(); ++i) {
                const UnitBuild &ub = units.u[i];
                // units: the shared expert, the hits, then the fills
                const bool covered = ub.expert < 0 ||
                                     (i < first_fill && c->map_shadow[(size_t)layer * c->E + ub.expert] == ub.src);
                if (covered) {
                    n_cov += 1;
                    np_cov += ub.np;
                    continue;
                }
                if (i < first_fill) gu_fill += 1;
                UnitBuild nb = ub;
                nb.p0 = (int32_t)g.pairs.size();
                g.pairs.insert(g.pairs.end(), units.pairs.begin() + ub.p0, units.pairs.begin() + ub.p0 + ub.np);
                g.u.push_back(nb);
            }
            gu = &g;
            if (pre_a)
                c->timed.push_back({6, pre_a, pre_b, gemv_bytes(c, n_cov, np_cov, 2, 0),
                                    2.0 * np_cov * (double)c->I * c->H * 2});
            pre_a = pre_b = nullptr;
        }
        const size_t split = wait_fills ? gu_fill : gu->u.size();
        const bool residual = (fflags & MOE_FWD_RESIDUAL) != 0;
        bool fused = false;
        if (!wait_fills) {
            rc = fused_expert_launch(c, layer, units, 0, units.u.size(), shared_w, gu_vec, n_tok, t0, t1, x, out,
                                     residual, has_shared, stream, &fused);
            if (rc) return rc;
        }
        if (!fused) {
            rc = launch_units(c, layer, 2, *gu, 0, split, shared_w, gu_vec, n_tok, stream);
            if (rc) return rc;
        }
        if (wait_fills) {
            err = hipSuccess;
            {
                HostClock hc(c->event_us);
                if (far_pending) err = hipStreamWaitEvent(stream, c->ev_staged[layer % kStagedRing], 0);
                if (err == hipSuccess && near_pending)
                    err = hipStreamWaitEvent(stream, c->ev_near[layer % kStagedRing], 0);
                if (err == hipSuccess && fill_ev) err = hipStreamWaitEvent(stream, fill_ev, 0);
            }
            if (err != hipSuccess)
                return hip_fail(err, "hipStreamWaitEvent(fill)");
            rc = fused_expert_launch(c, layer, units, split, units.u.size(), shared_w, gu_vec, n_tok, t0, t1, x, out,
                                     residual, has_shared, stream, &fused);
            if (rc) return rc;
            if (!fused) {
                rc = launch_units(c, layer, 2, *gu, split, gu->u.size(), shared_w, gu_vec, n_tok, stream);
                if (rc) return rc;
            }
        }
        if (!fused) {
            rc = down_and_combine(c, layer, units, shared_w, n_tok, t0, t1, x, out, residual, has_shared, stream,
                                  c->prelaunch ? &p : nullptr);
            if (rc) return rc;
        }
        // the stack driver's next layer: its router (and early gate/up) go out now, queued behind
        // this layer's kernels, before the host's remaining bookkeeping for this call
        if (next && w + 1 == c->wave_ranges.size() && layer + 1 < c->L) {
            const int nn = spec_count(c, layer + 1, next->spec_ws, next->n_spec_in);
            if ((rc = issue_route(c, layer + 1, next->x, n_tok, next->router_w, next->shared_w, next->spec_ws, nn,
                                  stream, 1 - c->rcur)) != MOE_OK)
                return rc;
        }
        // speculative uploads once this wave's expert kernels are queued: they need not hold up
        // the layer, and a copy outlasts a layer, so they still start well ahead
        if (w == 0 && spec && n_spec > 0) {
            const double ts = now_us();
            if ((rc = wait_routing(c, stream, n_tok, n_spec)) != MOE_OK) return rc;
            c->wait_us += now_us() - ts;
            prefetch_next(c, layer, n_tok, n_spec);
        }

        // the slots of this wave were last read by the launches above; later waves of this
        // call must not overwrite them before these kernels ran
        const uint64_t seq = c->reader_seq++;
        if (multi_wave) {
            if ((err = hipEventRecord(c->reader_ring[seq % kReaderRing], stream)) != hipSuccess)
                return hip_fail(err, "hipEventRecord(reader)");
        }
        for (size_t u = first_routed; u < units.u.size(); ++u) {
            const int slot = units.u[u].copy_to >= 0 ? units.u[u].copy_to : units.u[u].src;
            c->slot_reader[c->global_slot(layer, slot)] = multi_wave ? (int64_t)seq : -1;
        }

    }
    return MOE_OK;
}


// ----------------------------------------------------------------------------- prefill

constexpr int kArenaBatch = 32;       // experts per batch (NVMe page, "Workflow")
constexpr int kSchedSlack = 64;       // dispatch-table entries allowed beyond 3 per (item, tile)

// Dispatch table of one prefill GEMM launch.  The hardware hands workgroup b to
// XCD b % 8, and each XCD starts its workgroups in index order.  Items go to the
// XCDs longest first, each to the least loaded (an item costs about 1 + its
// 32-row tiles per column tile), and every XCD runs its items longest first, the
// column tiles of an item together; unused entries are -1.  Returns the table
// length, or 0 when it would exceed cap (the launch then goes without a table).
int build_sched(const moe::PrefillItem *items, int n_items, int n_tiles, int32_t *out, size_t cap) {
    std::vector<int> order(n_items);
    for (int i = 0; i < n_items; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return items[x].rows > items[y].rows; });
    std::vector<int> lists[8];
    int64_t load[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i : order) {
        const int x = (int)(std::min_element(load, load + 8) - load);
        lists[x].push_back(i);
        load[x] += 1 + (items[i].rows + 31) / 32;
    }
    size_t len = 0;
    for (const auto &l : lists) len = std::max(len, l.size() * (size_t)n_tiles);
    const size_t n = 8 * len;
    if (n > cap || n > (size_t)3 * n_items * n_tiles + kSchedSlack) return 0;
    std::fill(out, out + n, -1);
    for (int x = 0; x < 8; ++x)
        for (size_t q = 0; q < lists[x].size(); ++q)
            for (int t = 0; t < n_tiles; ++t) out[8 * (q * n_tiles + t) + x] = lists[x][q] * n_tiles + t;
    return (int)n;
}

int ensure_prefill(moe_cache *c, int n_tok) {
    if (n_tok <= c->pf_cap) return MOE_OK;
    const int cap = std::max(n_tok, 64);
    const size_t rows = (size_t)cap * (c->k + 1);
    const size_t max_items = rows / moe::kPrefillRows + (size_t)c->E + 2;
    const size_t max_batches = (size_t)(c->E + kArenaBatch - 1) / kArenaBatch + 1;
    const size_t sched_cap = 3 * max_items * (moe::prefill_tiles(2, c->I) + moe::prefill_tiles(1, c->H)) +
                             2 * max_batches * kSchedSlack;
    hipError_t e;
    if (c->pf_x16) hipFree(c->pf_x16);
    if (c->pf_h16) hipFree(c->pf_h16);
    if (c->pf_y) hipFree(c->pf_y);
    if (c->pf_pairs) hipFree(c->pf_pairs);
    if (c->pf_items) hipFree(c->pf_items);
    if (c->pf_sched) hipFree(c->pf_sched);
    if (c->pf_host) hipHostFree(c->pf_host);
    c->pf_sched = nullptr;
    c->pf_x16 = nullptr;
    c->pf_h16 = nullptr;
    c->pf_y = nullptr;
    c->pf_pairs = nullptr;
    c->pf_items = nullptr;
    c->pf_host = nullptr;
    c->pf_cap = 0;
    const size_t host_bytes = rows * sizeof(int32_t) + max_items * sizeof(moe::PrefillItem) + sched_cap * sizeof(int32_t);
    if ((e = hipMalloc(&c->pf_x16, (size_t)cap * c->H * 2)) != hipSuccess ||
        (e = hipMalloc(&c->pf_h16, rows * c->I * 2)) != hipSuccess ||
        (e = hipMalloc(&c->pf_y, rows * c->H * sizeof(float))) != hipSuccess ||
        (e = hipMalloc(&c->pf_pairs, rows * sizeof(int32_t))) != hipSuccess ||
        (e = hipMalloc(&c->pf_items, max_items * sizeof(moe::PrefillItem))) != hipSuccess ||
        (e = hipMalloc(&c->pf_sched, sched_cap * sizeof(int32_t))) != hipSuccess ||
        (e = hipHostMalloc((void **)&c->pf_host, host_bytes, hipHostMallocDefault)) != hipSuccess)
        return set_error(MOE_ERR_OOM, std::string("prefill workspace: ") + hipGetErrorString(e));
    if (!c->arena) {
        if ((e = hipMalloc(&c->arena, (size_t)2 * kArenaBatch * c->S)) != hipSuccess) {
            c->arena = nullptr;
            return set_error(MOE_ERR_OOM, std::string("prefill arena: ") + hipGetErrorString(e));
        }
        for (int i = 0; i < 2; ++i)
            if ((e = hipEventCreateWithFlags(&c->arena_read[i], hipEventDisableTiming)) != hipSuccess ||
                (e = hipEventCreateWithFlags(&c->arena_ready[i], hipEventDisableTiming)) != hipSuccess)
                return hip_fail(e, "event creation");
    }
    c->pf_items_cap = max_items;
    c->pf_sched_cap = sched_cap;
    c->pf_cap = cap;
    return MOE_OK;
}

// A call of more than 32 tokens: route every token, group the (token, pick) pairs
// by expert, and run the touched experts in ascending order, 32 at a time.  A
// resident expert is read in place from its slot; the others are uploaded into a
// double-buffered arena.  The LRU state is read, never changed (explainer page,
// "The rules in the code"; T4 page, "What the MoE Cache Actually Caches").
int prefill_forward_impl(moe_cache *c, int layer, const float *x, int n_tok, const float *router_w,
                         const void *shared_w, float *out, unsigned fflags, hipStream_t stream);

int prefill_forward(moe_cache *c, int layer, const float *x, int n_tok, const float *router_w, const void *shared_w,
                    float *out, unsigned fflags, hipStream_t stream) {
    discard_ahead(c);
    return prefill_forward_impl(c, layer, x, n_tok, router_w, shared_w, out, fflags, stream);
}

int prefill_forward_impl(moe_cache *c, int layer, const float *x, int n_tok, const float *router_w, const void *shared_w,
                    float *out, unsigned fflags, hipStream_t stream) {
    if (c->H % 64 || c->I % 64)
        return set_error(MOE_ERR_UNSUPPORTED, "the prefill path needs hidden and inter to be multiples of 64");
    int rc = ensure_route_capacity(c, n_tok);
    if (rc) return rc;
    if ((rc = ensure_prefill(c, n_tok))) return rc;
    hipError_t err;
    c->call_no += 1;
    if (c->have_last_stream && c->last_stream != stream) {
        if ((err = hipStreamSynchronize(c->last_stream)) != hipSuccess) return hip_fail(err, "hipStreamSynchronize");
        c->completed_seq = c->reader_seq;
    }
    const int k = c->k;
    const int nk = n_tok * k;
    const bool has_shared = (c->flags & MOE_SHARED_EXPERT) != 0;

    moe::RouterArgs ra{};
    ra.x = x;
    ra.xq = c->pf_x16;
    ra.xq_natural = 0;   // int4: the grouped GEMM takes x in the dequantiser's pair order
    ra.quant = c->quant;
    ra.w0 = router_w;
    ra.n_tok = n_tok;
    ra.E = c->E;
    ra.H = c->H;
    ra.top_k = k;
    ra.z = c->d_z;
    ra.ids = c->d_ids;
    ra.gate = c->d_gate;
    ra.ids_host = c->h_ids_dev;
    ra.gate_host = c->h_gate_dev;
    {
        TimeScope ts(c, 0, (double)c->E * c->H * 4 + (double)n_tok * c->H * 6, 2.0 * c->E * (double)c->H * n_tok);
        HostClock hc(c->launch_us);
        if ((err = moe::launch_router(ra, stream, ts.a, ts.b)) != hipSuccess) return hip_fail(err, "router launch");
    }
    if ((err = hipEventRecord(c->ev_route, stream)) != hipSuccess) return hip_fail(err, "hipEventRecord(route)");
    const double tw = now_us();
    if ((err = hipEventSynchronize(c->ev_route)) != hipSuccess) return hip_fail(err, "hipEventSynchronize(route)");
    c->wait_us += now_us() - tw;
    if (c->have_last_stream && c->last_stream == stream) c->completed_seq = c->reader_seq;
    c->last_stream = stream;
    c->have_last_stream = true;

    // group pairs by expert (counting sort; pairs stay ascending within an expert)
    const double tp = now_us();
    std::vector<int32_t> experts, slots;
    if (c->pl.prefill_lookup(layer, c->h_ids, nk, experts, slots) != moe::PLAN_OK)
        return set_error(MOE_ERR_INVALID, "router produced an expert id out of range");
    std::vector<int32_t> count(c->E + 1, 0), start(c->E + 1, 0);
    for (int i = 0; i < nk; ++i) count[c->h_ids[i]] += 1;
    int32_t *pairs = reinterpret_cast<int32_t *>(c->pf_host);
    const size_t rows = (size_t)nk + (has_shared ? n_tok : 0);
    {
        int32_t acc = 0;
        for (int e = 0; e < c->E; ++e) {
            start[e] = acc;
            acc += count[e];
        }
        std::vector<int32_t> pos(start.begin(), start.end());
        for (int i = 0; i < nk; ++i) pairs[pos[c->h_ids[i]]++] = i;
        for (int t = 0; t < (has_shared ? n_tok : 0); ++t) pairs[nk + t] = nk + t;
    }
    moe::PrefillItem *items = reinterpret_cast<moe::PrefillItem *>(c->pf_host + rows * sizeof(int32_t));
    // Batches: first the shared expert and every resident expert (read in place from
    // their slots, so they start at once), then the others in batches of up to
    // kArenaBatch read through the two arena halves in turn.
    struct Batch {
        int item_begin, item_end;
        int upload_no;                               // ordinal among the batches with uploads, -1 none
        int sched_off[2] = {0, 0}, sched_n[2] = {0, 0};   // dispatch tables of the down / gate-up launch
        std::vector<std::pair<int, int>> uploads;   // (expert, arena slot)
    };
    std::vector<Batch> batches;
    size_t n_items = 0;
    int n_res = 0, n_up = 0;
    auto add_items = [&](uint64_t block, int32_t off, int32_t n) {
        for (int32_t r = 0; r < n; r += moe::kPrefillRows)
            items[n_items++] = {block, off + r, std::min(moe::kPrefillRows, n - r)};
    };
    std::vector<size_t> missing;
    {
        Batch bt;
        bt.item_begin = (int)n_items;
        bt.upload_no = -1;
        if (has_shared) add_items((uint64_t)(uintptr_t)shared_w, (int32_t)nk, n_tok);
        for (size_t j = 0; j < experts.size(); ++j) {
            if (slots[j] < 0) {
                missing.push_back(j);
                continue;
            }
            add_items((uint64_t)(uintptr_t)c->slot_ptr(layer, slots[j]), start[experts[j]], count[experts[j]]);
            ++n_res;
        }
        bt.item_end = (int)n_items;
        if (bt.item_end > bt.item_begin) batches.push_back(std::move(bt));
    }
    for (size_t b0 = 0; b0 < missing.size(); b0 += kArenaBatch) {
        Batch bt;
        bt.item_begin = (int)n_items;
        bt.upload_no = (int)(b0 / kArenaBatch);
        const int half = bt.upload_no & 1;
        for (size_t q = b0; q < std::min(missing.size(), b0 + kArenaBatch); ++q) {
            const int e = experts[missing[q]];
            const int as = half * kArenaBatch + (int)(q - b0);
            bt.uploads.push_back({e, as});
            add_items((uint64_t)(uintptr_t)(c->arena + (size_t)as * c->S), start[e], count[e]);
            ++n_up;
        }
        bt.item_end = (int)n_items;
        batches.push_back(std::move(bt));
    }
    c->pl.account_prefill(n_res, n_up, (int)experts.size());
    if (c->tier) {
        // the RAM tier: the resident experts are used (ascending), then the uploads are read
        for (size_t j = 0; j < experts.size(); ++j)
            if (slots[j] >= 0) tier_touch(c, layer, &experts[j], 1);
    }
    int32_t *sched = reinterpret_cast<int32_t *>(c->pf_host + rows * sizeof(int32_t) +
                                                 c->pf_items_cap * sizeof(moe::PrefillItem));
    size_t n_sched = 0;
    for (Batch &bt : batches)
        for (int nm = 1; nm <= 2; ++nm) {
            const int n = build_sched(items + bt.item_begin, bt.item_end - bt.item_begin,
                                      moe::prefill_tiles(nm, nm == 2 ? c->I : c->H), sched + n_sched,
                                      c->pf_sched_cap - n_sched);
            bt.sched_off[nm - 1] = (int)n_sched;
            bt.sched_n[nm - 1] = n;
            n_sched += n;
        }
    c->plan_us += now_us() - tp;

    // plan to the device, on the compute stream ahead of the GEMMs
    HostClock hc_launch(c->launch_us);   // from here on: copies and launches
    if ((err = hipMemcpyAsync(c->pf_pairs, pairs, rows * sizeof(int32_t), hipMemcpyHostToDevice, stream)) != hipSuccess ||
        (err = hipMemcpyAsync(c->pf_items, items, n_items * sizeof(moe::PrefillItem), hipMemcpyHostToDevice, stream)) !=
            hipSuccess ||
        (n_sched && (err = hipMemcpyAsync(c->pf_sched, sched, n_sched * sizeof(int32_t), hipMemcpyHostToDevice,
                                          stream)) != hipSuccess))
        return hip_fail(err, "hipMemcpyAsync(prefill plan)");

    const size_t mg = matrix_bytes(c->quant, c->I, c->H);
    std::vector<const uint8_t *> hb;
    for (size_t bi = 0; bi < batches.size(); ++bi) {
        const Batch &bt = batches[bi];
        const int half = bt.upload_no & 1;
        if (!bt.uploads.empty()) {
            // the batch's host blocks (with a file store: RAM blocks, read where absent, in
            // ascending expert order)
            hb.assign(bt.uploads.size(), nullptr);
            if (c->tier) {
                std::vector<int32_t> ex(bt.uploads.size());
                for (size_t j = 0; j < ex.size(); ++j) ex[j] = bt.uploads[j].first;
                if (int rc = tier_fetch(c, layer, ex.data(), (int)ex.size(), hb.data())) return rc;
            } else {
                for (size_t j = 0; j < hb.size(); ++j) hb[j] = c->host_blocks[layer][bt.uploads[j].first];
            }
            // the arena half is free once the GEMMs of the upload batch before the previous one ran
            if (bt.upload_no >= 2 && (err = hipStreamWaitEvent(c->copy_stream, c->arena_read[half], 0)) != hipSuccess)
                return hip_fail(err, "hipStreamWaitEvent(arena)");
            size_t i = 0;
            while (i < bt.uploads.size()) {
                size_t n = 1;
                while (i + n < bt.uploads.size() && bt.uploads[i + n].first == bt.uploads[i].first + (int)n &&
                       bt.uploads[i + n].second == bt.uploads[i].second + (int)n && hb[i + n] == hb[i] + n * c->S)
                    ++n;
                if (int rc = pre_upload(c, c->arena + (size_t)bt.uploads[i].second * c->S, n, c->copy_stream))
                    return rc;
                err = hipMemcpyAsync(c->arena + (size_t)bt.uploads[i].second * c->S, hb[i], n * c->S,
                                     hipMemcpyHostToDevice, c->copy_stream);
                if (err != hipSuccess) return hip_fail(err, "hipMemcpyAsync(arena)");
                c->h2d_copied += n * c->S;
                i += n;
            }
            if ((err = hipEventRecord(c->arena_ready[half], c->copy_stream)) != hipSuccess ||
                (err = hipStreamWaitEvent(stream, c->arena_ready[half], 0)) != hipSuccess)
                return hip_fail(err, "arena events");
            tier_fence(c, hb.data(), (int)hb.size(), c->arena_ready[half], kTierCopy);
        }
        for (int nm = 2; nm >= 1; --nm) {
            moe::PrefillGemmArgs g{};
            g.items = c->pf_items + bt.item_begin;
            g.n_items = bt.item_end - bt.item_begin;
            g.pairs = c->pf_pairs;
            g.top_k = k;
            g.nk = nk;
            if (nm == 2) {
                g.a = c->pf_x16;
                g.a_by_token = 1;
                g.K = c->H;
                g.N = c->I;
                g.mat_off0 = 0;
                g.mat_off1 = mg;
                g.out = c->pf_h16;
            } else {
                g.a = c->pf_h16;
                g.a_by_token = 0;
                g.K = c->I;
                g.N = c->H;
                g.mat_off0 = 2 * mg;
                g.out = c->pf_y;
            }
            g.a_bytes = (nm == 2 ? (size_t)n_tok : rows) * g.K * sizeof(uint16_t);
            g.block_bytes = c->S;
            if (bt.sched_n[nm - 1] > 0) {
                g.sched = c->pf_sched + bt.sched_off[nm - 1];
                g.n_sched = bt.sched_n[nm - 1];
            }
            double rows_b = 0;
            for (int it = bt.item_begin; it < bt.item_end; ++it) rows_b += items[it].rows;
            const double flops = 2.0 * rows_b * g.N * (double)g.K * nm;
            const double bytes = (double)(bt.item_end - bt.item_begin) * nm * matrix_bytes(c->quant, g.N, g.K);
            TimeScope ts(c, 4, bytes, flops);
            if ((err = moe::launch_prefill_gemm(c->quant, nm, g, stream, ts.a, ts.b)) != hipSuccess)
                return hip_fail(err, "prefill GEMM launch");
        }
        if (!bt.uploads.empty() && (err = hipEventRecord(c->arena_read[half], stream)) != hipSuccess)
            return hip_fail(err, "arena event");
    }
    err = moe::launch_combine(x, c->pf_y, c->d_gate, out, n_tok, 0, n_tok, c->H, k, has_shared,
                              (fflags & MOE_FWD_RESIDUAL) ? 1 : 0, stream);
    if (err != hipSuccess) return hip_fail(err, "combine launch");
    return MOE_OK;
}

void free_cache(moe_cache *c) {
    if (!c) return;
    if (c->tier) {
        if (c->copy_stream) hipStreamSynchronize(c->copy_stream);
        if (c->copy_stream2) hipStreamSynchronize(c->copy_stream2);
        if (c->spec_stream) hipStreamSynchronize(c->spec_stream);
        if (c->tier->fd >= 0) close(c->tier->fd);
        if (c->tier->ram) hipHostFree(c->tier->ram);
        delete c->tier;
        c->tier = nullptr;
    }
    for (moe_cache::StepGraph &g : c->sg) {
        if (g.done) {
            hipEventSynchronize(g.done);
            hipEventDestroy(g.done);
        }
        if (g.exec) hipGraphExecDestroy(g.exec);
        if (g.ids) hipHostFree(g.ids);
        if (g.gate) hipHostFree(g.gate);
    }
    if (c->cap_stream) hipStreamDestroy(c->cap_stream);
    if (c->d_gx) hipFree(c->d_gx);
    if (c->d_gids) hipFree(c->d_gids);
    if (c->d_ggate) hipFree(c->d_ggate);
    if (c->h_graph_bad) hipHostFree(c->h_graph_bad);
    if (c->copy_stream) hipStreamSynchronize(c->copy_stream);
    if (c->copy_stream2) hipStreamSynchronize(c->copy_stream2);
    if (c->spec_stream) hipStreamSynchronize(c->spec_stream);
    resolve_timing(c);
    for (hipEvent_t e : c->event_pool) hipEventDestroy(e);
    for (hipEvent_t e : c->reader_ring)
        if (e) hipEventDestroy(e);
    for (hipEvent_t e : c->fill_ring)
        if (e) hipEventDestroy(e);
    if (c->ev_route) hipEventDestroy(c->ev_route);
    for (hipEvent_t ev : c->ev_staged)
        if (ev) hipEventDestroy(ev);
    for (hipEvent_t ev : c->ev_near)
        if (ev) hipEventDestroy(ev);
    if (c->copy_stream) hipStreamDestroy(c->copy_stream);
    if (c->copy_stream2) hipStreamDestroy(c->copy_stream2);
    if (c->ev_copy2) hipEventDestroy(c->ev_copy2);
    if (c->spec_stream) hipStreamDestroy(c->spec_stream);
    if (c->bank) hipFree(c->bank);
    if (c->staging) hipFree(c->staging);
    if (c->d_z) hipFree(c->d_z);
    if (c->d_tickets) hipFree(c->d_tickets);
    if (c->d_fused_sync) hipFree(c->d_fused_sync);
    if (c->d_map) hipFree(c->d_map);
    if (c->h_fused_timeout) hipHostFree(c->h_fused_timeout);
    if (c->d_ids) hipFree(c->d_ids);
    if (c->d_gate) hipFree(c->d_gate);
    if (c->h_ids_base) hipHostFree(c->h_ids_base);
    if (c->h_gate_base) hipHostFree(c->h_gate_base);
    if (c->h_spec_base) hipHostFree(c->h_spec_base);
    if (c->d_h) hipFree(c->d_h);
    if (c->d_y) hipFree(c->d_y);
    if (c->d_xq) hipFree(c->d_xq);
    if (c->pf_x16) hipFree(c->pf_x16);
    if (c->pf_h16) hipFree(c->pf_h16);
    if (c->pf_y) hipFree(c->pf_y);
    if (c->pf_pairs) hipFree(c->pf_pairs);
    if (c->pf_items) hipFree(c->pf_items);
    if (c->pf_sched) hipFree(c->pf_sched);
    if (c->pf_host) hipHostFree(c->pf_host);
    if (c->arena) hipFree(c->arena);
    for (int i = 0; i < 2; ++i) {
        if (c->arena_read[i]) hipEventDestroy(c->arena_read[i]);
        if (c->arena_ready[i]) hipEventDestroy(c->arena_ready[i]);
    }
    if (c->d_stack[0]) hipFree(c->d_stack[0]);
    if (c->d_stack[1]) hipFree(c->d_stack[1]);
    delete c;
}

bool is_pinned_host(const void *p) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return attr.type == hipMemoryTypeHost;
}

}  // namespace

// ============================================================================= C ABI

extern "C" {

size_t moe_expert_bytes(int quant, int hidden, int inter) { return expert_bytes_of(quant, hidden, inter); }

int moe_host_alloc(size_t nbytes, void **out) {
    if (!out || nbytes == 0) return set_error(MOE_ERR_INVALID, "bad arguments");
    *out = nullptr;
    hipError_t e = hipHostMalloc(out, nbytes, hipHostMallocDefault);
    if (e != hipSuccess) {
        *out = nullptr;
        return set_error(MOE_ERR_OOM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
    }
    return MOE_OK;
}

int moe_host_free(void *ptr) {
    if (!ptr) return MOE_OK;
    hipError_t e = hipHostFree(ptr);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "hipHostFree");
}

int moe_cache_create(int E, int K, int top_k, int hidden, int inter, int quant, int n_layers, unsigned flags,
                     moe_cache **out) {
    if (!out) return set_error(MOE_ERR_INVALID, "out is NULL");
    *out = nullptr;
    if (E <= 0 || K <= 0 || top_k <= 0 || hidden <= 0 || inter <= 0 || n_layers <= 0 || top_k > E)
        return set_error(MOE_ERR_INVALID, "sizes must be positive and top_k <= E");
    if (quant != MOE_Q_F32 && quant != MOE_Q_INT4_G32_F16 && quant != MOE_Q_E2M1_E4M3_G16)
        return set_error(MOE_ERR_INVALID, "unknown quant");
    if (K < top_k) return set_error(MOE_ERR_CACHE_TOO_SMALL, "K < top_k: one token's picks cannot all be resident");
    if (top_k > kMaxTopK || E > kMaxExperts) return set_error(MOE_ERR_UNSUPPORTED, "top_k > 16 or E > 1024");
    if (check_shapes(quant, hidden, inter) != MOE_OK)
        return set_error(MOE_ERR_UNSUPPORTED, "hidden/inter must be multiples of 256 (4-bit) or 32 (fp32), "
                                              "with at most 256 16-byte chunks per row");
    const size_t S = expert_bytes_of(quant, hidden, inter);
    if (!S) return set_error(MOE_ERR_INVALID, "bad shape for the format");
    if (flags & ~(MOE_POOL_SHARED | MOE_SHARED_EXPERT | MOE_PREFETCH | MOE_WAVES_UNION | MOE_POLICY_LFU |
                  MOE_ADAPTIVE_CAPACITY))
        return set_error(MOE_ERR_INVALID, "unknown flags");
    if ((flags & MOE_ADAPTIVE_CAPACITY) && (flags & (MOE_POOL_SHARED | MOE_POLICY_LFU)))
        return set_error(MOE_ERR_UNSUPPORTED, "adaptive capacity is defined for per-layer LRU pools");
    const bool shared = (flags & MOE_POOL_SHARED) != 0;
    moe_cache *c = new (std::nothrow)
        moe_cache(E, K, top_k, n_layers, shared, S, (flags & MOE_WAVES_UNION) != 0, (flags & MOE_POLICY_LFU) != 0,
                  (flags & MOE_ADAPTIVE_CAPACITY) != 0);
    if (!c) return set_error(MOE_ERR_OOM, "host allocation failed");
    c->E = E;
    c->K = K;
    c->k = top_k;
    c->H = hidden;
    c->I = inter;
    c->quant = quant;
    c->L = n_layers;
    c->flags = flags;
    c->S = S;
    if (const char *v = getenv("MOE_DEBUG_POISON")) c->debug_poison = v[0] == '1';
    if (const char *v = getenv("MOE_DEBUG_DELAY_US")) c->debug_delay_us = (unsigned)std::min(100000L, std::max(0L, atol(v)));
    hipError_t e;
    if ((e = hipGetDevice(&c->device)) != hipSuccess) {
        free_cache(c);
        return hip_fail(e, "hipGetDevice");
    }
    c->n_pools = shared ? 1 : n_layers;
    c->host_blocks.assign(n_layers, std::vector<const uint8_t *>(E, nullptr));
    c->layer_ready.assign(n_layers, 0);
    c->slot_reader.assign((size_t)c->n_pools * K, -1);
    if ((e = hipMalloc(&c->bank, (size_t)c->n_pools * K * S)) != hipSuccess) {
        free_cache(c);
        return set_error(MOE_ERR_OOM, std::string("slot bank: ") + hipGetErrorString(e));
    }
    if (flags & MOE_PREFETCH) {
        if ((e = hipMalloc(&c->staging, (size_t)kStageSlots * S)) != hipSuccess) {
            c->staging = nullptr;
            free_cache(c);
            return set_error(MOE_ERR_OOM, std::string("staging bank: ") + hipGetErrorString(e));
        }
        c->stage_key.assign(kStageSlots, -1);
        c->stage_used.assign(kStageSlots, 0);
        c->stage_busy.assign(kStageSlots, 0);
    }
    c->max_pairs = 32 * top_k + 32;
    if ((e = hipMalloc(&c->d_h, (size_t)c->max_pairs * inter * sizeof(float))) != hipSuccess ||
        (e = hipMalloc(&c->d_y, (size_t)c->max_pairs * hidden * sizeof(float))) != hipSuccess) {
        free_cache(c);
        return set_error(MOE_ERR_OOM, std::string("activation buffers: ") + hipGetErrorString(e));
    }
    {
        if ((e = hipMalloc(&c->d_xq, (size_t)moe::kMaxTokens * hidden * 2)) != hipSuccess ||
            (e = hipMalloc(&c->d_stack[0], (size_t)moe::kMaxTokens * hidden * sizeof(float))) != hipSuccess ||
            (e = hipMalloc(&c->d_stack[1], (size_t)moe::kMaxTokens * hidden * sizeof(float))) != hipSuccess ||
            (e = hipMalloc(&c->d_tickets, moe::kTicketBytes)) != hipSuccess ||
            (e = hipMemset(c->d_tickets, 0, moe::kTicketBytes)) != hipSuccess ||
            (e = hipMalloc(&c->d_fused_sync, moe::kSyncBytes)) != hipSuccess ||
            (e = hipMemset(c->d_fused_sync, 0, moe::kSyncBytes)) != hipSuccess ||
            (e = hipMalloc(&c->d_map, (size_t)n_layers * E * sizeof(int32_t))) != hipSuccess ||
            (e = hipMemset(c->d_map, 0xFF, (size_t)n_layers * E * sizeof(int32_t))) != hipSuccess) {
            free_cache(c);
            return set_error(MOE_ERR_OOM, std::string("activation/stack buffers: ") + hipGetErrorString(e));
        }
        if ((e = hipHostMalloc((void **)&c->h_fused_timeout, sizeof(int), hipHostMallocMapped | hipHostMallocCoherent)) !=
            hipSuccess) {
            free_cache(c);
            return set_error(MOE_ERR_OOM, std::string("pinned flag: ") + hipGetErrorString(e));
        }
        *c->h_fused_timeout = 0;
        c->map_shadow.assign((size_t)n_layers * E, -1);
        if ((e = hipHostGetDevicePointer((void **)&c->h_fused_timeout_dev, c->h_fused_timeout, 0)) != hipSuccess) {
            free_cache(c);
            return hip_fail(e, "hipHostGetDevicePointer");
        }
    }
    if ((e = hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking)) != hipSuccess ||
        (e = hipStreamCreateWithFlags(&c->spec_stream, hipStreamNonBlocking)) != hipSuccess ||
        (e = hipStreamCreateWithFlags(&c->copy_stream2, hipStreamNonBlocking)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&c->ev_copy2, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&c->ev_route, hipEventDisableTiming)) != hipSuccess) {
        free_cache(c);
        return hip_fail(e, "stream/event creation");
    }
    for (hipEvent_t &ev : c->ev_staged)
        if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
            free_cache(c);
            return hip_fail(e, "event creation");
        }
    for (hipEvent_t &ev : c->ev_near)
        if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
            free_cache(c);
            return hip_fail(e, "event creation");
        }
    c->unit_of.assign(E, -1);
    c->reader_ring.assign(kReaderRing, nullptr);
    c->fill_ring.assign(kFillRing, nullptr);
    for (auto &ev : c->reader_ring)
        if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
            free_cache(c);
            return hip_fail(e, "event creation");
        }
    for (auto &ev : c->fill_ring)
        if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
            free_cache(c);
            return hip_fail(e, "event creation");
        }
    int rc = ensure_route_capacity(c, 32);
    if (rc) {
        free_cache(c);
        return rc;
    }
    *out = c;
    return MOE_OK;
}

int moe_cache_set_layer(moe_cache *c, int layer, const void *host_experts, size_t nbytes) {
    if (!c || !host_experts || layer < 0 || layer >= c->L) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (nbytes != (size_t)c->E * c->S) return set_error(MOE_ERR_INVALID, "nbytes must be E * expert_bytes");
    if (c->tier) return set_error(MOE_ERR_INVALID, "the cache reads a file store");
    if (!is_pinned_host(host_experts))
        return set_error(MOE_ERR_INVALID, "host store must be pinned host memory (moe_host_alloc)");
    const uint8_t *b = (const uint8_t *)host_experts;
    for (int e = 0; e < c->E; ++e) c->host_blocks[layer][e] = b + (size_t)e * c->S;
    c->layer_ready[layer] = 1;
    return MOE_OK;
}

int moe_cache_set_file_store(moe_cache *c, const char *path, int ram_blocks, int n_readers) {
    if (!c || !path || n_readers < 1 || n_readers > 64) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (c->tier) return set_error(MOE_ERR_INVALID, "the cache already has a file store");
    // a wave's uploads (at most min(capacity, 32 * top_k) fills, where a layer's capacity is K,
    // or up to E with adaptive capacity) and a prefill batch (32) must fit at once
    const int cap = c->pl.adaptive() ? std::max(c->K, c->E) : c->K;
    const int need = std::max(32, std::min(cap, 32 * c->k));
    if (ram_blocks < need) return set_error(MOE_ERR_INVALID, "ram_blocks below the uploads of one wave or batch");
    if (int grc = graph_sync(c)) return grc;
    discard_ahead(c);
    FileTier *t = new (std::nothrow) FileTier();
    if (!t) return set_error(MOE_ERR_OOM, "file store");
    t->fd = open(path, O_RDONLY);
    if (t->fd < 0) {
        delete t;
        return set_error(MOE_ERR_IO, std::string("open: ") + strerror(errno));
    }
    const off_t need_bytes = (off_t)c->L * c->E * (off_t)c->S;
    const off_t size = lseek(t->fd, 0, SEEK_END);
    if (size < need_bytes) {
        close(t->fd);
        delete t;
        return set_error(MOE_ERR_INVALID, "the file is shorter than n_layers * E blocks");
    }
    t->R = ram_blocks;
    t->n_readers = n_readers;
    const hipError_t e = hipHostMalloc((void **)&t->ram, (size_t)ram_blocks * c->S, hipHostMallocDefault);
    if (e != hipSuccess) {
        close(t->fd);
        delete t;
        return set_error(MOE_ERR_OOM, std::string("RAM tier: ") + hipGetErrorString(e));
    }
    t->lru = moe::SlotPool(ram_blocks);
    t->block_of.assign((size_t)c->L * c->E, -1);
    t->fence.assign(ram_blocks, {nullptr, nullptr, nullptr});
    c->tier = t;
    for (int l = 0; l < c->L; ++l) c->layer_ready[l] = 1;
    return MOE_OK;
}

int moe_cache_set_expert_ptrs(moe_cache *c, int layer, const void *const *blocks) {
    if (!c || !blocks || layer < 0 || layer >= c->L) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (c->tier) return set_error(MOE_ERR_INVALID, "the cache reads a file store");
    for (int e = 0; e < c->E; ++e) {
        if (!blocks[e]) return set_error(MOE_ERR_INVALID, "null expert block");
        if (!is_pinned_host(blocks[e])) return set_error(MOE_ERR_INVALID, "expert blocks must be pinned host memory");
    }
    for (int e = 0; e < c->E; ++e) c->host_blocks[layer][e] = (const uint8_t *)blocks[e];
    c->layer_ready[layer] = 1;
    return MOE_OK;
}

int moe_layer_forward(moe_cache *c, int layer, const float *x, int n_tokens, const float *router_w,
                      const void *shared_w, const float *next_router_w, float *out, unsigned flags, void *stream) {
    if (!c || !x || !router_w || !out || n_tokens < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (layer < 0 || layer >= c->L) return set_error(MOE_ERR_INVALID, "layer out of range");
    if ((c->flags & MOE_SHARED_EXPERT) && !shared_w)
        return set_error(MOE_ERR_INVALID, "the cache has a shared expert: shared_w is required");
    if (!(c->flags & MOE_SHARED_EXPERT)) shared_w = nullptr;
    if (int grc = graph_sync(c)) return grc;
    if (x == out) return set_error(MOE_ERR_INVALID, "out may not alias x");
    if (!c->layer_ready[layer]) return set_error(MOE_ERR_NOT_READY, "no host store registered for this layer");
    if (n_tokens == 0) return MOE_OK;
    int dev = -1;
    if (hipGetDevice(&dev) == hipSuccess && dev != c->device) hipSetDevice(c->device);
    c->forwards += 1;
    c->last_tokens = n_tokens;
    int rc;
    {
        HostClock hc(c->call_us);
        if (n_tokens <= MOE_DECODE_MAX_TOKENS)
            rc = decode_forward(c, layer, x, n_tokens, router_w, shared_w, &next_router_w, 1, out, flags,
                                (hipStream_t)stream);
        else
            rc = prefill_forward(c, layer, x, n_tokens, router_w, shared_w, out, flags, (hipStream_t)stream);
    }
    if (dev >= 0 && dev != c->device) hipSetDevice(dev);
    return rc;
}

}  // extern "C"

// ----------------------------------------------------------------------------- allocation-free decode calls
//
// moe_layer_forward_noalloc runs the decode path with its per-call device scratch (logits,
// router counters, the fp16 activation copy, h, Y, the device routing ids and gates) in one
// file-scope device array instead of the cache's own buffers, and allocates nothing.  Each
// GPU holds its own copy of the array until the process ends; its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and only that address
// is handed to kernels and copies.
namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};

// The device address of `scratch` on `device` (the current device).
int scratch_address(int device, unsigned char **out) {
    if (device < 0 || device >= kScratchDevices) return set_error(MOE_ERR_UNSUPPORTED, "device index too large");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return set_error(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) gave no address");
        g_scratch_ptr[device] = p;
    }
    *out = (unsigned char *)g_scratch_ptr[device];
    return MOE_OK;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Where each scratch buffer of a decode call sits in the array, sized as the cache sizes its
// own buffers; total bytes in *total.
struct ScratchLayout {
    size_t z, tickets, xq, h, y, ids, gate, total;
};
ScratchLayout scratch_layout(const moe_cache *c) {
    ScratchLayout l{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += round256(bytes);
        return at;
    };
    const size_t nk = (size_t)moe::kMaxTokens * c->k;
    l.z = take((1 + moe::kMaxSpec) * (size_t)moe::kMaxTokens * c->E * sizeof(double));
    l.tickets = take(moe::kTicketBytes);
    l.xq = take((size_t)moe::kMaxTokens * c->H * 2);
    l.h = take((size_t)c->max_pairs * c->I * sizeof(float));
    l.y = take((size_t)c->max_pairs * c->H * sizeof(float));
    l.ids = take(nk * sizeof(int32_t));
    l.gate = take(nk * sizeof(float));
    l.total = off;
    return l;
}

}  // namespace

extern "C" {

int moe_layer_forward_noalloc(moe_cache *c, int layer, const float *x, int n_tokens, const float *router_w,
                              const void *shared_w, const float *next_router_w, float *out, unsigned flags,
                              void *stream) {
    if (!c || !x || !router_w || !out || n_tokens < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (layer < 0 || layer >= c->L) return set_error(MOE_ERR_INVALID, "layer out of range");
    if (n_tokens > MOE_DECODE_MAX_TOKENS)
        return set_error(MOE_ERR_UNSUPPORTED, "the allocation-free call runs decode calls (at most 32 tokens)");
    if ((c->flags & MOE_SHARED_EXPERT) && !shared_w)
        return set_error(MOE_ERR_INVALID, "the cache has a shared expert: shared_w is required");
    if (!(c->flags & MOE_SHARED_EXPERT)) shared_w = nullptr;
    if (x == out) return set_error(MOE_ERR_INVALID, "out may not alias x");
    const ScratchLayout lay = scratch_layout(c);
    if (lay.total > kScratchBytes)
        return set_error(MOE_ERR_UNSUPPORTED, "the decode scratch of this cache's shape exceeds the 32 MiB array");
    if (int grc = graph_sync(c)) return grc;
    if (!c->layer_ready[layer]) return set_error(MOE_ERR_NOT_READY, "no host store registered for this layer");
    if (n_tokens == 0) return MOE_OK;
    if (c->max_route_tokens < n_tokens)      // sized for 32 tokens when the cache was created
        return set_error(MOE_ERR_INVALID, "routing buffers smaller than the call");
    int dev = -1;
    if (hipGetDevice(&dev) == hipSuccess && dev != c->device) hipSetDevice(c->device);
    struct DeviceBack {
        int dev, mine;
        ~DeviceBack() {
            if (dev >= 0 && dev != mine) hipSetDevice(dev);
        }
    } device_back{dev, c->device};
    unsigned char *base = nullptr;
    if (int rc = scratch_address(c->device, &base)) return rc;
    // a router launched ahead by the stack driver wrote the cache's own buffers
    discard_ahead(c);
    // the router's counters start at zero (each launch leaves them at zero; the array keeps
    // whatever the last call on this GPU left)
    hipError_t e = moe::launch_fill_u32((unsigned *)(base + lay.tickets), 0u, moe::kTicketBytes / sizeof(unsigned),
                                        (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "scratch counter clear");
    // the call's kernels take the array's buffers; kernel timing (which creates events) is off
    struct Swap {
        moe_cache *c;
        double *z;
        unsigned *tickets;
        void *xq;
        float *h, *y, *gate;
        int32_t *ids;
        unsigned mask;
        ~Swap() {
            c->d_z = z;
            c->d_tickets = tickets;
            c->d_xq = xq;
            c->d_h = h;
            c->d_y = y;
            c->d_ids = ids;
            c->d_gate = gate;
            c->time_mask = mask;
        }
    } swap{c, c->d_z, c->d_tickets, c->d_xq, c->d_h, c->d_y, c->d_gate, c->d_ids, c->time_mask};
    c->d_z = (double *)(base + lay.z);
    c->d_tickets = (unsigned *)(base + lay.tickets);
    c->d_xq = base + lay.xq;
    c->d_h = (float *)(base + lay.h);
    c->d_y = (float *)(base + lay.y);
    c->d_ids = (int32_t *)(base + lay.ids);
    c->d_gate = (float *)(base + lay.gate);
    c->time_mask = 0;
    c->forwards += 1;
    c->last_tokens = n_tokens;
    HostClock hc(c->call_us);
    return decode_forward(c, layer, x, n_tokens, router_w, shared_w, &next_router_w, 1, out, flags,
                          (hipStream_t)stream);
}

static int stack_layer(moe_cache *c, int layer, const float *x, int n_tokens, const float *router_w,
                       const void *shared_w, const float *const *spec_ws, int n_spec, float *out, void *stream,
                       const NextCall *next) {
    if (!c->layer_ready[layer]) return set_error(MOE_ERR_NOT_READY, "no host store registered for this layer");
    if (n_tokens == 0) return MOE_OK;
    c->forwards += 1;
    c->last_tokens = n_tokens;
    HostClock hc(c->call_us);
    return decode_forward(c, layer, x, n_tokens, router_w, shared_w, spec_ws, n_spec, out, MOE_FWD_RESIDUAL,
                          (hipStream_t)stream, next);
}

int moe_stack_forward(moe_cache *c, const float *x, int n_tokens, const float *const *router_ws,
                      const void *const *shared_ws, float *out, float *layer_inputs, void *stream) {
    if (!c || !x || !router_ws || !out || n_tokens < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (n_tokens > MOE_DECODE_MAX_TOKENS)
        return set_error(MOE_ERR_UNSUPPORTED, "the stack driver runs decode calls (at most 32 tokens)");
    if (x == out) return set_error(MOE_ERR_INVALID, "out may not alias x");
    if ((c->flags & MOE_SHARED_EXPERT) && !shared_ws) return set_error(MOE_ERR_INVALID, "shared_ws is required");
    if (n_tokens == 1) {
        bool done = false;
        const int grc = graph_step(c, x, router_ws, shared_ws, out, layer_inputs, (hipStream_t)stream, &done);
        if (grc || done) return grc;
    }
    if (int grc = graph_sync(c)) return grc;
    const size_t bytes = (size_t)n_tokens * c->H * sizeof(float);
    const float *in = x;
    for (int l = 0; l < c->L; ++l) {
        float *dst = (l == c->L - 1) ? out : c->d_stack[l & 1];
        if (layer_inputs) {
            hipError_t e = hipMemcpyAsync(layer_inputs + (size_t)l * n_tokens * c->H, in, bytes, hipMemcpyDeviceToDevice,
                                          (hipStream_t)stream);
            if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(layer input)");
        }
        const float *spec_ws[moe::kMaxSpec], *next_spec_ws[moe::kMaxSpec];
        int n_spec = 0, n_next_spec = 0;
        while (n_spec < c->pf_ahead && l + n_spec + 1 < c->L) {
            spec_ws[n_spec] = router_ws[l + n_spec + 1];
            ++n_spec;
        }
        while (n_next_spec < c->pf_ahead && l + n_next_spec + 2 < c->L) {
            next_spec_ws[n_next_spec] = router_ws[l + n_next_spec + 2];
            ++n_next_spec;
        }
        // the next layer reads this layer's output; its input copy (layer_inputs) is queued
        // after its router, which leaves that output unchanged
        NextCall next{dst, l + 1 < c->L ? router_ws[l + 1] : nullptr,
                      shared_ws && l + 1 < c->L ? shared_ws[l + 1] : nullptr, next_spec_ws, n_next_spec};
        int rc = stack_layer(c, l, in, n_tokens, router_ws[l], shared_ws ? shared_ws[l] : nullptr, spec_ws, n_spec, dst,
                             stream, l + 1 < c->L && c->layer_ready[l + 1] ? &next : nullptr);
        if (rc) return rc;
        in = dst;
    }
    return MOE_OK;
}

int moe_cache_stats(const moe_cache *c, moe_stats *out) {
    if (!c || !out) return set_error(MOE_ERR_INVALID, "bad arguments");
    const int grc = flush_graph(const_cast<moe_cache *>(c));
    *out = moe_stats();
    moe::planner_stats(c->pl, *out);
    out->graph_steps = c->graph_steps;
    if (c->tier) {
        out->ram_hits = c->tier->hits;
        out->ram_misses = c->tier->misses;
        out->ram_evictions = c->tier->evictions;
        out->bytes_read_file = c->tier->bytes_read;
    }
    out->forwards = c->forwards;
    out->prefetch_issued = c->pf_issued;
    out->prefetch_used = c->pf_used;
    out->prefetch_wasted = c->pf_wasted;
    out->prefetch_candidates = c->pf_candidates;
    out->prefetch_deferred = c->pf_deferred;
    out->bytes_h2d_copied = c->h2d_copied;
    out->bytes_d2d_copied = c->d2d_copied;
    out->host_plan_us = c->plan_us;
    out->host_wait_us = c->wait_us;
    out->host_call_us = c->call_us;
    out->host_upload_us = c->upload_us;
    out->host_launch_us = c->launch_us;
    out->host_prefetch_us = c->prefetch_us;
    out->host_event_us = c->event_us;
    return grc;
}

int moe_cache_reset_stats(moe_cache *c) {
    if (!c) return set_error(MOE_ERR_INVALID, "bad arguments");
    const int grc = flush_graph(c);
    c->pl.reset_stats();
    c->graph_steps = 0;
    if (c->tier) c->tier->hits = c->tier->misses = c->tier->evictions = c->tier->bytes_read = 0;
    c->forwards = c->pf_issued = c->pf_used = c->pf_wasted = c->h2d_copied = c->d2d_copied = 0;
    c->pf_candidates = c->pf_deferred = 0;
    c->plan_us = c->wait_us = c->call_us = c->upload_us = c->launch_us = c->prefetch_us = c->event_us = 0;
    return grc;
}

int moe_cache_set_trace(moe_cache *c, moe_trace_fn fn, void *user) {
    if (!c) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (int grc = flush_graph(c)) return grc;   // the step in flight reports to the callback it ran under
    c->trace_fn = fn;
    c->trace_user = user;
    return MOE_OK;
}

int moe_cache_set_timing(moe_cache *c, unsigned mask) {
    if (!c) return set_error(MOE_ERR_INVALID, "bad arguments");
    c->time_mask = mask;
    // every event a timed launch may take before the next resolve, created here rather
    // than on the launch path
    const size_t want = mask ? 2 * (size_t)kTimedMax + 16 : 0;
    const size_t have = c->event_pool.size() + 2 * c->timed.size();
    for (size_t i = have; i < want; ++i) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return set_error(MOE_ERR_HIP, "hipEventCreate (timing events)");
        c->event_pool.push_back(e);
    }
    return MOE_OK;
}

int moe_cache_set_timing_stride(moe_cache *c, int stride) {
    if (!c || stride < 1) return set_error(MOE_ERR_INVALID, "bad arguments");
    c->time_stride = stride;
    for (uint64_t &n : c->time_count) n = 0;
    return MOE_OK;
}

int moe_cache_set_prefetch(moe_cache *c, int backlog, int layers_ahead) {
    if (!c || backlog < 0 || backlog > kStageSlots / 2 || layers_ahead < 1 || layers_ahead > moe::kMaxSpec)
        return set_error(MOE_ERR_INVALID, "bad arguments");
    c->pf_backlog = backlog;
    c->pf_ahead = layers_ahead;
    return MOE_OK;
}

int moe_cache_set_prelaunch(moe_cache *c, int on) {
    if (!c || (on != 0 && on != 1)) return set_error(MOE_ERR_INVALID, "bad arguments");
    c->prelaunch = on != 0;
    return MOE_OK;
}

int moe_cache_set_adaptive(moe_cache *c, int period, int delta, int pairs, int floor) {
    if (!c) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (!c->pl.adaptive()) return set_error(MOE_ERR_UNSUPPORTED, "the cache was created without adaptive capacity");
    if (int grc = flush_graph(c)) return grc;
    if (c->pl.set_adaptive(period, delta, pairs, floor) != moe::PLAN_OK)
        return set_error(MOE_ERR_INVALID, "bad adaptive parameters");
    return MOE_OK;
}

int moe_cache_layer_capacity(const moe_cache *c, int layer, int *held, int *target) {
    if (!c || !held || !target || layer < 0 || layer >= c->L) return set_error(MOE_ERR_INVALID, "bad arguments");
    flush_graph(const_cast<moe_cache *>(c));
    *held = c->pl.held(layer);
    *target = c->pl.target(layer);
    return MOE_OK;
}

int moe_cache_set_graph(moe_cache *c, int on) {
    if (!c || (on != 0 && on != 1)) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (on && c->pl.adaptive()) return set_error(MOE_ERR_UNSUPPORTED, "captured steps need fixed per-layer capacities");
    const int grc = flush_graph(c);
    c->graph_on = on != 0;
    if (!on) drop_graphs(c);
    return grc;
}

int moe_cache_set_decode_fusion(moe_cache *c, int on) {
    if (!c || (on != 0 && on != 1)) return set_error(MOE_ERR_INVALID, "bad arguments");
    c->fuse_decode = on != 0;
    return MOE_OK;
}

int moe_cache_timing(moe_cache *c, moe_timing *out) {
    if (!c || !out) return set_error(MOE_ERR_INVALID, "bad arguments");
    resolve_timing(c);
    *out = c->timing;
    return MOE_OK;
}

int moe_cache_reset_timing(moe_cache *c) {
    if (!c) return set_error(MOE_ERR_INVALID, "bad arguments");
    resolve_timing(c);
    c->timing = moe_timing{};
    return MOE_OK;
}

int moe_cache_last_routing(const moe_cache *c, int32_t *ids, float *gate, int n_tokens) {
    if (!c || n_tokens <= 0) return set_error(MOE_ERR_INVALID, "bad arguments");
    if (int grc = flush_graph(const_cast<moe_cache *>(c))) return grc;
    if (n_tokens != c->last_tokens) return set_error(MOE_ERR_INVALID, "bad arguments");
    const size_t n = (size_t)n_tokens * c->k;
    if (ids) memcpy(ids, c->h_ids, n * sizeof(int32_t));
    if (gate) memcpy(gate, c->h_gate, n * sizeof(float));
    return MOE_OK;
}

int moe_cache_slot_of(const moe_cache *c, int layer, int expert) {
    if (!c || layer < 0 || layer >= c->L || expert < 0 || expert >= c->E) return -1;
    flush_graph(const_cast<moe_cache *>(c));
    return c->pl.slot_of(layer, expert);
}

int moe_cache_slot_ptr(const moe_cache *c, int layer, int slot, const void **out) {
    const int n_slots = c && c->pl.adaptive() ? c->L * c->K : (c ? c->K : 0);   // adaptive: global numbers
    if (!c || !out || layer < 0 || layer >= c->L || slot < 0 || slot >= n_slots)
        return set_error(MOE_ERR_INVALID, "bad arguments");
    *out = c->slot_ptr(layer, slot);
    return MOE_OK;
}

void moe_cache_destroy(moe_cache *c) {
    if (!c) return;
    const char *log = getenv("MOE_CACHE_LOG");
    if (log && log[0] == '1') {
        moe_stats s;
        moe_cache_stats(c, &s);
        const moe_bucket_stats *bs[2] = {&s.small, &s.large};
        const char *names[2] = {"ubatch <= 8", "ubatch 9..32"};
        for (int i = 0; i < 2; ++i) {
            const uint64_t n = bs[i]->hits + bs[i]->misses;
            fprintf(stderr, "moe_cache: %s: hits = %llu, misses = %llu, hit rate = %.1f%%, uploaded = %.1f MiB\n",
                    names[i], (unsigned long long)bs[i]->hits, (unsigned long long)bs[i]->misses,
                    n ? 100.0 * bs[i]->hits / n : 0.0, bs[i]->bytes_h2d / 1048576.0);
        }
    }
    free_cache(c);
}

int moe_debug_fail_upload(moe_cache *c, int nth) {
    if (!c || nth < -1) return set_error(MOE_ERR_INVALID, "bad arguments");
    c->debug_fail_upload = nth;
    return MOE_OK;
}

int moe_debug_decode(int quant, int what, const uint8_t *codes, int n, float *out, void *stream) {
    if (!codes || !out || n < 0) return set_error(MOE_ERR_INVALID, "bad arguments");
    hipError_t e = moe::launch_debug_decode(quant, what, codes, n, out, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "decode launch");
}

}  // extern "C"
