// Internal interface between the host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>

namespace moe {

// Launch a kernel and return the status of this launch alone (hipGetLastError
// would also report an earlier, unrelated failure).  With events, the dispatch
// itself records ev_start / ev_stop when the kernel starts and ends.
template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, hipEvent_t ev_start,
                         hipEvent_t ev_stop, A... args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    static_assert((std::is_same_v<P, A> && ...), "kernel arguments must match the parameter types exactly");
    void *ptrs[] = {static_cast<void *>(&args)...};
    if (ev_start || ev_stop)
        return hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, stream, ev_start,
                                  ev_stop, 0);
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, stream);
}

enum Quant { Q_F32 = 0, Q_INT4 = 1, Q_E2M1 = 2 };

constexpr int kMaxTokens = 32;   // tokens of a decode call
constexpr int kMaxUnits = 128;
constexpr int kMaxPairs = 128;

// Work list of one expert-GEMV launch, passed by value as a kernel argument.
// A unit is one distinct expert of a wave: where its block is read from, an
// optional pool slot the block is copied into on the way (a fill served from
// the prefetch staging bank), and the (token, pick) pairs routed to it.  A
// pair id is t*top_k + j for routed picks and n_tok*top_k + t for the shared
// expert.  Two capacities: the small one keeps the kernel arguments of a
// single-token call short (the launch copies them).
template <int MU, int MP>
struct UnitListT {
    static constexpr int kUnits = MU, kPairs = MP;
    int32_t n_units;
    int32_t src[MU];                  // >= 0: pool slot; -1: shared expert; <= -2: staging slot (-2 - src)
    int32_t copy_to[MU];              // pool slot receiving the bytes read, or -1
    uint16_t pbeg[MU + 1];            // pairs of unit u: pair[pbeg[u] .. pbeg[u+1])
    uint16_t pad_;                    // keeps pair[] 4-byte aligned (kernels read it by dwords)
    uint16_t pair[MP];
};
using UnitList = UnitListT<kMaxUnits, kMaxPairs>;
using UnitListS = UnitListT<16, 16>;
static_assert(offsetof(UnitList, pair) % 4 == 0 && offsetof(UnitListS, pair) % 4 == 0, "pair[] alignment");

// Activation vectors of the 4-bit formats are fp16, in the pair order the
// weight decoder consumes: int4 -- within every 8 elements the fp16 pairs
// (0,4) (1,5) (2,6) (3,7); e2m1 -- natural order.  fp32 weights take fp32 vectors.
struct GemvArgs {
    const uint8_t *bank;       // slot bank base of the pool
    const uint8_t *staging;    // prefetch staging bank
    const uint8_t *shared_w;   // block of the shared expert (or null)
    uint8_t *copy_bank;        // bank that copy_to slots index (the pool's)
    size_t block_bytes;        // S
    size_t mat_off0;           // byte offset of the (first) matrix inside a block
    size_t mat_off1;           // byte offset of the second matrix (gate/up kernel)
    int rows;                  // R
    int cols;                  // C (reduction)
    const void *vec;           // activation vectors (fp16 pair order, or fp32)
    int vec_by_token;          // 1: row of vec = token of the pair; 0: row = pair id
    int nk;                    // n_tok * top_k (first shared-expert pair id)
    int top_k;
    void *out;                 // gate/up: h (fp16 pair order, or fp32) [pairs x R]; down: Y fp32 [pairs x R]
    int tiles_per_unit;
};

struct GemvShape {             // launch shape chosen for (quant, cols, n_mats)
    int lpr, cpl, u;           // lanes per row, 16-byte chunks per lane, rows in flight per lane
    int rows_per_wg;
    bool ok;
};

GemvShape gemv_shape(int quant, int cols, int n_mats);

// The down projection of a whole wave fused with the weighted combine: the
// grid tiles the hidden dimension, each workgroup computes its rows of Y for
// every unit of the list and then the output rows of every token of the wave,
//   out[t] = sum_j gate[t,j] Y[t*k+j] (+ Y[shared, t]) (+ x[t])
// in the same order and arithmetic as the separate down and combine kernels.
// The list must hold the wave's every unit and pair (one list per wave).
constexpr int kMaxMapUpdates = 32;
struct CombineArgs {
    const float *x;            // residual source [n_tok x H], or null
    const float *gate;         // [n_tok x top_k]
    float *out;                // [n_tok x H]
    int t0, nt;                // tokens of the wave
    int has_shared;
    // entries of the device copy of the slot table that this wave's plan changed:
    // map[upd_key[i]] = upd_val[i] for i < n_upd (workgroup 0 stores them)
    int32_t *map;
    int n_upd;
    int32_t upd_key[kMaxMapUpdates];
    int32_t upd_val[kMaxMapUpdates];
    // one-token launch (k_down_combine_picks) only: a matrix the next launch reads, a router
    // [pf_rows x pf_cols] fp32 read by workgroups of kRouterRowsPerWg rows, requested on the
    // way so that it sits in the cache (each workgroup b takes rows of the reading workgroups
    // congruent to b mod 8, which the dispatch places on the same XCD when both grids are
    // multiples of 8); null: nothing
    const float *pf;
    int pf_rows, pf_cols;
};

// Gate/up of a one-token call's resident picks, launched right after the router and
// before the host has planned: unit u < n_routed is the router's pick u (ids[u]); it is
// computed from the slot the device copy of the slot table gives (map[map_base + id]),
// and skipped when that is -1.  Unit n_routed is the shared expert (if has_shared).
// The plan never moves a resident expert, so these slots are the plan's for every hit.
struct PreArgs {
    const int32_t *ids;        // router output [top_k] (device)
    const int32_t *map;        // device copy of the slot table, [n_layers * E]
    int map_base;              // layer * E
    int n_experts;
    int n_routed;              // top_k
    int has_shared;
};
hipError_t launch_expert_gemv_pre(int quant, const GemvArgs &a, const PreArgs &pa, hipStream_t stream,
                                  hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
// Down + combine of a one-token call whose every pick is resident, its units read on the
// device like the early gate/up's (a captured decode step, or the early launch of an
// uncaptured one): the combine of token 0 with cb.t0 = 0, cb.nt = 1, a.nk = pa.n_routed.  A
// pick out of range or not resident makes the launch write nothing and set *bad
// (device-visible host memory) if bad is not null.
hipError_t launch_down_combine_picks(int quant, const GemvArgs &a, const CombineArgs &cb, const PreArgs &pa, int *bad,
                                     hipStream_t stream, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
hipError_t launch_down_combine(int quant, const GemvArgs &a, const CombineArgs &cb, const UnitList &ul,
                               hipStream_t stream, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Completion signal of the fused decode kernel's gate/up workgroups, counted
// in two levels so that no memory line takes more than a few dozen atomics per
// launch: kSyncGroups group counters, a top counter over the groups, and
// kSyncFlags copies of the flag the down workgroups poll.  Counters are zero
// between launches (the workgroup that completes one resets it); a flag holds
// the epoch of the last launch whose h values are all stored.
constexpr int kSyncGroups = 32;
constexpr int kSyncFlags = 8;
constexpr int kSyncStrideU32 = 64;   // 256 bytes between counters and between flags
constexpr size_t kSyncBytes = (size_t)(kSyncGroups + 1 + 2 * kSyncFlags) * kSyncStrideU32 * 4;
struct FusedSync {
    unsigned *sync;             // kSyncBytes, zeroed once: groups, then top, then the flags (u64)
    unsigned long long epoch;   // this launch's number, from 1, increasing
    int *timed_out;             // host-mapped flag, set if a down workgroup stopped waiting
    int n_gu;                   // gate/up workgroups: ulg.n_units * g.tiles_per_unit
};

// Gate/up of `ulg` (a subset of the wave's units, or all of them) and the down
// projection + combine of the whole wave (`uld`) in one launch; see
// k_expert_fused.  Returns hipErrorNotSupported, having launched nothing, where
// the shape or the list sizes have no fused kernel (the caller then launches
// the two kernels).
hipError_t launch_expert_fused(int quant, const GemvArgs &g, const UnitList &ulg, const GemvArgs &d,
                               const CombineArgs &cb, const UnitList &uld, const FusedSync &fs, hipStream_t stream,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Launch one expert GEMV over `ul` (n_mats = 2: gate/up + SwiGLU, 1: down).
// ev_start/ev_stop (may be null): events the dispatch itself records when the
// kernel starts and ends (hipExtLaunchKernel), for kernel timing.
hipError_t launch_expert_gemv(int quant, int n_mats, const GemvArgs &a, const UnitList &ul, hipStream_t stream,
                              hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Router: float64 logits of this layer's router and of up to kMaxSpec later
// layers' routers (for speculative prefetch), then softmax and top-k.  The
// logits launch also writes the fp16 activation copy of x for the gate/up GEMV.
constexpr int kMaxSpec = 5;
constexpr int kRouterRowsPerWg = 4;   // router rows per workgroup of the row kernels
// The one-launch router (up to kFusedRouterTokens tokens) exchanges the logits through a
// float64 array whose every entry holds kExchangeSentinel between launches: the bit pattern
// of a NaN whose low payload bits are set, which no sum of products of fp32 values widened
// to float64 can produce.  Filled with bytes 0xFF once; each launch leaves it so.
constexpr int kFusedRouterTokens = 4;
constexpr unsigned long long kExchangeSentinel = ~0ull;
inline size_t router_exchange_bytes(int E) { return (size_t)(1 + kMaxSpec) * kFusedRouterTokens * E * sizeof(double); }
// How long the one-launch router's selecting workgroups wait for the other workgroups'
// logits before they give up (microseconds of the GPU's 100 MHz real-time counter): far
// beyond any launch, so that only a workgroup starved by other work on the GPU for that long
// could make a selection give up.
constexpr unsigned kRouterWaitUs = 200000;
struct RouterArgs {
    const float *x;            // [n_tok x H]
    int xq_natural;            // 1: fp16 copy in natural order (prefill GEMM operand)
    void *xq;                  // fp16 activation copy [n_tok x H] (4-bit formats), or null
    int quant;
    const float *w0;           // [E x H]
    const float *wspec[kMaxSpec];   // [E x H]: the routers of layers +1 .. +n_spec
    int n_spec;                // 0 .. kMaxSpec
    int n_tok, E, H, top_k;
    double *z;                 // [n_mats x n_tok x E]
    // selection outputs (second kernel)
    int32_t *ids;              // [n_tok x top_k] device
    float *gate;               // [n_tok x top_k] device
    int32_t *ids_host;         // device-visible pinned copies (may be null)
    float *gate_host;
    int32_t *spec_ids_host;    // picks of wspec[0..n_spec): [n_spec x n_tok x top_k], or null
    double *zx;                // exchange array (router_exchange_bytes(E), every entry the sentinel):
                               // one launch for up to kFusedRouterTokens tokens; null: two launches
    int *timed_out;            // device-visible host flag, set if a selection stopped waiting
    unsigned wait_us;          // microseconds before a selection stops waiting (0: it does not wait)
};
hipError_t launch_router(const RouterArgs &a, hipStream_t stream, hipEvent_t ev_start = nullptr,
                         hipEvent_t ev_stop = nullptr);

// out[t] = (residual ? x[t] : 0) + sum_j gate[t,j] Y[t*k+j] (+ Y[nk+t]), in rank order,
// for tokens t0 .. t0+nt-1 of a call of n_tok tokens.
hipError_t launch_combine(const float *x, const float *y, const float *gate, float *out, int n_tok, int t0, int nt,
                          int H, int top_k, int has_shared, int residual, hipStream_t stream);

// Prefill grouped GEMM.  A work item is up to kPrefillRows pairs of one expert;
// the grid is items x output tiles of 64.
constexpr int kPrefillRows = 128;
struct PrefillItem {
    uint64_t block;            // device address of the expert's packed block (pool slot or arena)
    int32_t pair_off;          // first pair of the item in the expert-sorted pair list
    int32_t rows;              // pairs in the item (<= kPrefillRows)
};
struct PrefillGemmArgs {
    const PrefillItem *items;
    int n_items;
    int n_tiles;               // column tiles per item (set by the launcher)
    const int32_t *pairs;      // pair ids sorted by expert
    const _Float16 *a;         // gate/up: x fp16 [n_tok x K] (row = token); down: h fp16 [pairs x K];
                               // int4: each group of 8 elements in the pair order (0,4,1,5,2,6,3,7)
    size_t a_bytes;            // bytes of a (< 2^31)
    size_t block_bytes;        // bytes of an expert block (< 2^31)
    int a_by_token;            // row of a: pair p -> token p / top_k (p < nk) or p - nk (shared expert)
    int top_k;
    int nk;                    // n_tok * top_k
    int K, N;                  // reduction and output sizes
    size_t mat_off0, mat_off1;
    void *out;                 // gate/up: h fp16 [pairs x N] (int4: pair order as a); down: Y fp32 [pairs x N]
    const int32_t *sched;      // null, or the unit (item * n_tiles + tile) of each workgroup, -1 for none
    int n_sched;               // workgroups when sched is set
};
// Column tiles of one item in a prefill GEMM launch with n_mats matrices of N outputs.
int prefill_tiles(int n_mats, int N);
hipError_t launch_prefill_gemm(int quant, int n_mats, const PrefillGemmArgs &a, hipStream_t stream,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

hipError_t launch_debug_decode(int quant, int what, const uint8_t *codes, int n, float *out, hipStream_t stream);

// map[keys[i]] = vals[i] for i < n, by kernels whose arguments carry the entries (no host
// buffer has to outlive the call; keys must be in range).
hipError_t launch_map_set(int32_t *map, const int32_t *keys, const int32_t *vals, int n, hipStream_t stream);

// p[0 .. n) = v, by a kernel (a fill that a captured graph may hold, unlike a memset node).
hipError_t launch_fill_u32(unsigned *p, unsigned v, size_t n, hipStream_t stream);

// A one-wave kernel that returns after `us` microseconds (at most 100000) of the real-time
// counter: a stream position that completes late, for fence checks.
hipError_t launch_delay_us(unsigned us, hipStream_t stream);

}  // namespace moe
