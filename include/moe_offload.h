/*
 * moe_offload.h -- C ABI of the MI355X offloaded mixture-of-experts layer with
 * an LRU expert cache (library: expert_offload_lru_amd/libmoe_offload.so).
 *
 * The layer (SGLang page "Running an MoE Model Larger Than Your VRAM: SGLang
 * Paged Experts, the PCIe Math, and the 4-Request Cliff", section "What does
 * Paged Experts actually do?"; explainer page "MoE expert offload and the LRU
 * expert cache that llama.cpp and SGLang both merged in October 2026",
 * sections "The model that should not fit" and "Inside llama.cpp PR #29887"):
 * a router picks top_k of E experts per token; a K-slot LRU cache of experts
 * in HBM resolves every pick to a slot, misses are copied from a pinned host
 * store holding every expert; the picked experts' SwiGLU FFNs run on the
 * routed tokens and their outputs are summed with the router's weights.
 *
 * Conventions
 *  - Every function returns an int status (MOE_OK = 0 or a negative MOE_ERR_*)
 *    unless stated otherwise; moe_last_error() gives a message for the calling
 *    thread.  The library never aborts the process.
 *  - "device" pointers are HIP device memory of the GPU that was current when
 *    the cache was created; "host" pointers are ordinary host memory unless
 *    "pinned" is stated (allocated with moe_host_alloc, hipHostMalloc or a
 *    pinned torch tensor).  The library never pins caller memory itself.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - A cache handle is used from one host thread at a time.  Calls on one
 *    cache are ordered by their stream; when a call uses a different stream
 *    than the previous call, the library first waits for the previous stream.
 *
 * Packed expert block (S = moe_expert_bytes(quant, hidden, inter) bytes): the
 * matrices gate [inter x hidden], up [inter x hidden], down [hidden x inter]
 * back to back.  A matrix of R rows and C reduction columns is stored as
 *   MOE_Q_F32:           R*C float32, row-major;
 *   MOE_Q_INT4_G32_F16:  R*C/2 bytes of 4-bit codes, row-major, element 2j in
 *                        the low nibble of byte j and 2j+1 in the high nibble;
 *                        then R*C/32 float16 scales (row-major, one per 32
 *                        consecutive elements of a row); w = (q - 8) * s
 *                        (Q4_0-like: 32 weights share a 2-byte scale, explainer
 *                        page, "The bus problem");
 *   MOE_Q_E2M1_E4M3_G16: R*C/2 bytes of e2m1 codes (sign, 2-bit exponent with
 *                        bias 1, 1-bit mantissa; same nibble order); then R*C/16
 *                        OCP E4M3 scale bytes, one per 16 elements; w = s * q
 *                        (NVFP4-like, 95 GiB page "Decode"; NVMe page "Workflow").
 * The FFN of an expert is y = W_down (silu(W_gate x) * (W_up x)).
 */
#ifndef MOE_OFFLOAD_H
#define MOE_OFFLOAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
#define MOE_OK                    0
#define MOE_ERR_INVALID          -1  /* bad argument, shape or pointer            */
#define MOE_ERR_CACHE_TOO_SMALL  -2  /* K < top_k, or a plan needs more slots     */
#define MOE_ERR_OOM              -3  /* a device or pinned allocation failed      */
#define MOE_ERR_HIP              -4  /* a HIP runtime call failed                 */
#define MOE_ERR_NOT_READY        -5  /* a layer's host store was never set        */
#define MOE_ERR_UNSUPPORTED      -6  /* shape/format the library does not handle  */
#define MOE_ERR_IO               -7  /* opening or reading the expert file failed   */

/* ---------------------------------------------------------------- formats */
#define MOE_Q_F32                 0
#define MOE_Q_INT4_G32_F16        1
#define MOE_Q_E2M1_E4M3_G16       2

/* ---------------------------------------------------------------- create flags */
#define MOE_POOL_SHARED      0x1u  /* one pool of K slots for all layers, key layer*E+e
                                      (T4 page, "What the MoE Cache Actually Caches");
                                      otherwise K slots per layer (SGLang page)        */
#define MOE_SHARED_EXPERT    0x2u  /* layers have an always-on shared expert (weight 1) */
#define MOE_PREFETCH         0x4u  /* speculative next-layer uploads into a staging bank */
#define MOE_WAVES_UNION      0x8u  /* decode calls with tokens*top_k > K split into waves that
                                      take tokens while the union of their experts fits in K
                                      (SGLang page, "Comments"); otherwise waves of K/top_k
                                      tokens (SGLang page, "What happens with more than one
                                      request?")                                         */
#define MOE_POLICY_LFU      0x10u  /* evict the least frequently used expert instead of the
                                      least recently used (95 GiB page, "Decode"): a use
                                      count per expert that survives eviction, +1 per plan
                                      naming it; empty slots first (lowest first), then least
                                      (count, plan of last use, slot) among the experts the
                                      plan does not name                                 */
#define MOE_ADAPTIVE_CAPACITY 0x20u /* per-layer pools that trade capacity at a fixed total
                                      of n_layers*K slots (95 GiB page, "Decode"); slots
                                      are then numbered over all layers (layer l starts
                                      with l*K .. l*K+K-1); see moe_cache_set_adaptive.
                                      Not with MOE_POOL_SHARED or MOE_POLICY_LFU
                                      (MOE_ERR_UNSUPPORTED)                              */

/* ---------------------------------------------------------------- forward flags */
#define MOE_FWD_RESIDUAL     0x1u  /* out = x + y instead of out = y */

/* A call with at most this many tokens is a decode call (LRU path); a larger
 * one is a prefill call (explainer page, "The rules in the code"). */
#define MOE_DECODE_MAX_TOKENS 32

typedef struct moe_cache moe_cache;

typedef struct moe_bucket_stats {
    uint64_t plans;       /* plans (waves) counted in this bucket                  */
    uint64_t hits;        /* distinct experts found resident, summed over plans     */
    uint64_t misses;      /* distinct experts filled (uploaded or staged), summed   */
    uint64_t picks;       /* routed (token, k) picks                                */
    uint64_t pick_hits;   /* picks whose expert was resident before the plan        */
    uint64_t evictions;
    uint64_t bytes_h2d;   /* bytes of expert blocks the plans asked to upload       */
    uint64_t bytes_d2d;   /* prefill: bytes served from cache slots                 */
    uint64_t union_sum;   /* distinct experts per plan, summed                      */
    uint64_t union_max;
} moe_bucket_stats;

typedef struct moe_stats {
    moe_bucket_stats small;    /* plans of <= 8 tokens (ids <= 8 * top_k)           */
    moe_bucket_stats large;    /* decode plans of 9..32 tokens                       */
    moe_bucket_stats prefill;  /* prefill calls: hits = from a slot, misses = uploaded */
    uint64_t waves;            /* decode plans                                       */
    uint64_t forwards;         /* moe_layer_forward calls                            */
    uint64_t prefetch_issued;  /* speculative uploads (experts)                      */
    uint64_t prefetch_used;    /* fills served from the staging bank                 */
    uint64_t prefetch_wasted;  /* staged experts overwritten unused                  */
    uint64_t prefetch_candidates; /* predicted experts neither resident nor staged     */
    uint64_t prefetch_deferred;   /* ... of which not uploaded: the copy queue was full */
    uint64_t bytes_h2d_copied; /* H2D bytes actually copied (demand + speculative)   */
    uint64_t bytes_d2d_copied; /* D2D bytes copied (staging -> slot, slot -> arena)  */
    double   host_plan_us;     /* host time spent in plans                           */
    double   host_wait_us;     /* host time waiting for routing ids                  */
    double   host_call_us;     /* host time inside decode and prefill calls, total   */
    double   host_upload_us;   /* ... of which issuing demand uploads                */
    double   host_launch_us;   /* ... of which kernel launches                       */
    double   host_prefetch_us; /* ... of which issuing speculative uploads           */
    double   host_event_us;    /* ... of which stream waits on copy events (decode)  */
    uint64_t graph_steps;      /* decode steps run as a captured graph (moe_cache_set_graph) */
    uint64_t ram_hits;         /* file store: uploads whose block was in the RAM tier */
    uint64_t ram_misses;       /* ... read from the file first                         */
    uint64_t ram_evictions;    /* ... of which replaced a block held in the RAM tier   */
    uint64_t bytes_read_file;  /* bytes read from the file                             */
} moe_stats;

/* One plan (decode wave), handed to the trace callback during moe_layer_forward.
 * Arrays are valid only during the callback. */
typedef struct moe_plan_record {
    int32_t layer, wave, t0, t1, top_k;
    const int32_t *ids;          /* [(t1-t0)*top_k] picks, token-major, rank order  */
    const float   *gate;         /* [(t1-t0)*top_k] router weight of each pick       */
    const int32_t *slots;        /* [(t1-t0)*top_k] pool slot of each pick            */
    int32_t n_hits;   const int32_t *hits;          /* experts, first-occurrence order */
    int32_t n_fills;  const int32_t *fill_expert;   /* ascending expert                */
                      const int32_t *fill_slot;
    int32_t n_evictions; const int64_t *evict_key;  /* key = expert, or layer*E+expert */
                         const int32_t *evict_slot; /*   for a shared pool             */
} moe_plan_record;

typedef void (*moe_trace_fn)(const moe_plan_record *rec, void *user);

/* Kernel timing (HIP events around each launch on the launch stream). */
typedef struct moe_kernel_timing {
    uint64_t launches;
    double   ms;          /* summed event durations                          */
    double   bytes;       /* algorithmic bytes of the timed launches          */
    double   flops;       /* algorithmic flops of the timed launches          */
} moe_kernel_timing;

typedef struct moe_timing {
    moe_kernel_timing router, gate_up, down, combine, prefill_gemm;
    moe_kernel_timing expert_fused;   /* gate/up + down + combine in one launch */
    moe_kernel_timing gate_up_early;  /* one-token calls: resident picks' gate/up before the plan */
    moe_kernel_timing down_early;     /* one-token calls: resident picks' down + combine before the
                                         plan; a launch whose output the plan did not keep counts
                                         zero bytes */
} moe_timing;

#define MOE_TIME_ROUTER   0x1u
#define MOE_TIME_GATE_UP  0x2u
#define MOE_TIME_DOWN     0x4u
#define MOE_TIME_COMBINE  0x8u
#define MOE_TIME_PREFILL  0x10u
#define MOE_TIME_FUSED    0x20u
#define MOE_TIME_GATE_UP_EARLY 0x40u
#define MOE_TIME_DOWN_EARLY 0x80u

/* ---------------------------------------------------------------- functions */

/* Bytes of one packed expert block; 0 for an unknown format or bad shape. */
size_t moe_expert_bytes(int quant, int hidden, int inter);

/* Pinned (page-locked, device-mapped) host memory for expert stores.
 * Freed with moe_host_free.  MOE_ERR_OOM if the allocation fails. */
int moe_host_alloc(size_t nbytes, void **out);
int moe_host_free(void *ptr);

/* Create a cache on the current HIP device.
 *  E experts per layer, K slots (per layer, or in total with MOE_POOL_SHARED),
 *  top_k picks per token, hidden/inter the expert shape, quant a MOE_Q_*,
 *  n_layers MoE layers.  Allocates the slot bank(s) in HBM (K*S bytes per pool),
 *  the staging bank, routing buffers, a copy stream and events.
 *  Errors: MOE_ERR_INVALID (non-positive sizes, top_k > E, unknown quant),
 *  MOE_ERR_CACHE_TOO_SMALL (K < top_k), MOE_ERR_UNSUPPORTED (hidden or inter
 *  not a multiple of 256 for 4-bit formats, of 4 for fp32; top_k > 16;
 *  E > 1024), MOE_ERR_OOM, MOE_ERR_HIP.  *out is NULL on error. */
int moe_cache_create(int E, int K, int top_k, int hidden, int inter, int quant,
                     int n_layers, unsigned flags, moe_cache **out);

/* Register the host store of `layer`: E packed blocks back to back
 * (nbytes == E * S), in pinned host memory.  Caller-owned; it must outlive
 * the cache and not change while the cache may upload from it.
 * Errors: MOE_ERR_INVALID (bad layer, size, or memory that is not pinned). */
int moe_cache_set_layer(moe_cache *c, int layer, const void *host_experts, size_t nbytes);

/* Same, with one pinned pointer per expert (blocks[e], S bytes each); blocks
 * may alias.  Runs of consecutive experts are merged into one copy only when
 * their blocks are also consecutive in memory. */
int moe_cache_set_expert_ptrs(moe_cache *c, int layer, const void *const *blocks);

/* Two-tier host store for models beyond host RAM (NVMe page, "Workflow": experts
 * repacked into contiguous blocks read with pread into an LRU cache of pinned RAM
 * blocks, fed by reader threads; copies to the GPU from there).  Replaces the host
 * store of every layer; set_layer / set_expert_ptrs are refused afterwards.
 *  path:       file holding block (layer, e) of expert_bytes bytes at byte offset
 *              (layer * E + e) * expert_bytes, for every layer and expert (it may be
 *              longer); opened read-only and read with buffered pread (direct I/O
 *              cannot target pinned memory of the GPU driver).
 *  ram_blocks: pinned RAM blocks of the tier, at least max(32, min(C, 32 * top_k)) with
 *              C = K, or max(K, E) with MOE_ADAPTIVE_CAPACITY (one wave's or one prefill
 *              batch's uploads); a call whose uploads would need more fails with
 *              MOE_ERR_INVALID instead of reusing a block it copies from.
 *  n_readers:  threads that read one wave's or batch's absent blocks in parallel (1..64).
 * The tier is an LRU keyed layer * E + e whose recency follows use by the model: per
 * decode wave the plan's hits make their blocks (if present) the most recently used,
 * then its fills in the plan's order are read from the tier (a present block is a hit;
 * an absent one is read into the least recently used block once the copies that last
 * read that block completed), a fill served from the staging bank only refreshing its
 * block; a prefill call refreshes its resident experts' blocks, then reads its uploads,
 * both ascending.  Speculative copies take only blocks already present and change no
 * recency.
 * Counters: moe_stats.ram_*, bytes_read_file.  Errors: MOE_ERR_INVALID (bad sizes,
 * a file shorter than n_layers * E blocks, a second call), MOE_ERR_IO (open), MOE_ERR_OOM.
 * A failed read later makes the forward call return MOE_ERR_IO. */
int moe_cache_set_file_store(moe_cache *c, const char *path, int ram_blocks, int n_readers);

/* One MoE layer.
 *  x, out:        device fp32 [n_tokens x hidden], row-major; out is overwritten
 *                 (out may not alias x).
 *  router_w:      device fp32 [E x hidden] of this layer.
 *  shared_w:      device packed block of the layer's shared expert (required
 *                 iff the cache has MOE_SHARED_EXPERT), else NULL.
 *  next_router_w: device fp32 [E x hidden] of layer+1, used for speculative
 *                 prefetch when the cache has MOE_PREFETCH; NULL disables it.
 *  flags:         MOE_FWD_RESIDUAL.
 * n_tokens = 0 returns MOE_OK and enqueues nothing.
 * n_tokens <= 32: decode path (router, LRU plan per wave, uploads, expert
 * GEMV, combine).  n_tokens > 32: prefill path (router, experts grouped by
 * token, batches of 32 experts through an arena, grouped MFMA GEMM, combine);
 * the LRU state is read, not changed.
 * Work is enqueued on `stream`; the host blocks only until the routing ids
 * of the call are readable.  out is valid when `stream` completes.
 * Errors: MOE_ERR_INVALID, MOE_ERR_NOT_READY (no host store for the layer),
 * MOE_ERR_CACHE_TOO_SMALL, MOE_ERR_HIP (a failed upload submission rolls
 * back that wave's fills), MOE_ERR_OOM, MOE_ERR_UNSUPPORTED (n_tokens > 32
 * with hidden or inter not a multiple of 64). */
int moe_layer_forward(moe_cache *c, int layer, const float *x, int n_tokens,
                      const float *router_w, const void *shared_w,
                      const float *next_router_w, float *out, unsigned flags,
                      void *stream);

/* moe_layer_forward for callers that cannot allocate device memory during the call (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): a decode
 * call (n_tokens <= 32, arguments, results and errors as moe_layer_forward) whose per-call
 * device scratch -- router logits and counters, the fp16 activation copy, the gate/up
 * output h and the expert outputs Y, the device routing ids and gates -- lives in one
 * 32 MiB device array of the library instead of the cache's buffers.  The call allocates
 * no device or pinned memory (no hipMalloc, hipHostMalloc, hipFree, no event creation:
 * kernel timing does not see its launches); the cache itself is created beforehand by
 * moe_cache_create.  Each GPU holds one copy of the array from its first such call until
 * the process ends, shared by every cache on that GPU and keeping the last call's
 * contents: calls of this function that overlap on one GPU (two streams, two host
 * threads, two caches) race on it and must be ordered by the caller.
 * Errors: as moe_layer_forward, plus MOE_ERR_UNSUPPORTED for n_tokens > 32 or a cache
 * shape whose decode scratch exceeds 32 MiB (it grows with top_k * hidden and
 * top_k * inter; the Qwen3-30B-A3B and Flash-Next shapes take under 5 MiB). */
int moe_layer_forward_noalloc(moe_cache *c, int layer, const float *x, int n_tokens,
                              const float *router_w, const void *shared_w,
                              const float *next_router_w, float *out, unsigned flags,
                              void *stream);

/* A decode step through all n_layers layers, chained by the residual
 * x_{l+1} = x_l + y_l (out = x_{n_layers}); the layer loop runs in the library.
 *  x, out:       device fp32 [n_tokens x hidden], n_tokens <= 32, out != x.
 *  router_ws:    host array of n_layers device pointers (fp32 [E x hidden]).
 *  shared_ws:    host array of n_layers device blocks, or NULL without a shared expert.
 *  layer_inputs: NULL, or device fp32 [n_layers x n_tokens x hidden] that receives x_l.
 * With MOE_PREFETCH, layer l also routes its input through the routers of the
 * next layers (router_ws[l+1] .. router_ws[l+d], d = layers_ahead of
 * moe_cache_set_prefetch, default 3) and uploads their predicted misses.
 * Errors as moe_layer_forward, plus MOE_ERR_UNSUPPORTED for more than 32 tokens. */
int moe_stack_forward(moe_cache *c, const float *x, int n_tokens, const float *const *router_ws,
                      const void *const *shared_ws, float *out, float *layer_inputs, void *stream);

/* Counters since creation or the last reset. */
int moe_cache_stats(const moe_cache *c, moe_stats *out);
int moe_cache_reset_stats(moe_cache *c);

/* Trace callback called synchronously on the host for every plan; NULL off. */
int moe_cache_set_trace(moe_cache *c, moe_trace_fn fn, void *user);

/* Kernel timing: `mask` of MOE_TIME_* kernels to bracket with events (0 = off).
 * moe_cache_timing waits for outstanding timed launches, then reports sums. */
int moe_cache_set_timing(moe_cache *c, unsigned mask);
/* Time one launch in every `stride` (>= 1; default 1) of each selected kernel:
 * an event-timed launch costs the host several microseconds more than a plain
 * one, so sampling keeps a timed run close to an untimed one.  Errors:
 * MOE_ERR_INVALID for stride < 1. */
int moe_cache_set_timing_stride(moe_cache *c, int stride);
int moe_cache_timing(moe_cache *c, moe_timing *out);

/* Speculative prefetch (MOE_PREFETCH) tuning.
 *  backlog:      speculative uploads are issued only while fewer than this many
 *                expert blocks are queued on the copy stream (0..32, default 4):
 *                demand uploads of the next call queue behind them.
 *  layers_ahead: layers moe_stack_forward routes ahead for speculation
 *                (1..5, default 3).
 * Errors: MOE_ERR_INVALID for a value out of range. */
int moe_cache_set_prefetch(moe_cache *c, int backlog, int layers_ahead);
int moe_cache_reset_timing(moe_cache *c);

/* Decode launch shape (off by default).  With on = 1, a wave whose units fit
 * one short launch list runs its expert work as one kernel: the gate/up
 * workgroups first, then the down projection + combine workgroups, which
 * request their weights at once and wait on device counters until every h
 * value is stored (the expert FFN of the SGLang page, "What does Paged
 * Experts actually do?", and the NVMe page's fused 4-bit kernel, "Workflow";
 * putting both projections in one launch is this library's choice).  Shapes
 * without a fused kernel, and larger waves, take the gate/up and down kernels
 * as with on = 0.  Outputs are bitwise the same either way.  Measured on
 * MI355X at one token, the fused launch takes about as long as the two
 * kernels it replaces: the cross-XCD completion signal costs what the kernel
 * boundary did.  Should a down workgroup stop waiting (a bounded wait that, by
 * dispatch order, always ends), later moe_layer_forward / moe_stack_forward
 * calls fail with MOE_ERR_HIP.
 * Errors: MOE_ERR_INVALID for on other than 0 or 1. */
int moe_cache_set_decode_fusion(moe_cache *c, int on);

/* Captured decode steps (opt-in; off by default).  With on = 1, a moe_stack_forward call
 * of one token, made while every expert of every layer holds a slot,
 * runs as one replay of a captured HIP graph: per layer the router, the gate/up of every
 * pick and the down + combine, the units read on the device from the router's ids and the
 * device copy of the slot table, with no host round trip between layers (SGLang page,
 * "What happens with more than one request?": a single-wave decode step is the case a
 * graph can hold; NVMe page, "Workflow": graphs for the one-token layers).  Every pick of
 * such a step is a hit, so nothing is uploaded or evicted; the host replays the step's
 * plans from its routing results at the next call into the cache (or at moe_cache_stats,
 * moe_cache_last_routing, moe_cache_slot_of ...), which gives the same recency order,
 * counters and trace records as the uncaptured path, and outputs bitwise equal to it.
 * x is copied into the cache ahead of each replay; layer_inputs, when given, is written
 * by copies inside the graph; a graph is captured per (out, layer_inputs, router_ws,
 * shared_ws), two in turn, and captured again when one of them changes; other
 * calls take the regular path.  Per-kernel timing does not see the
 * captured launches.  If a captured step finds a pick without a slot (the host's check
 * makes that impossible), it writes nothing and every later forward call returns
 * MOE_ERR_HIP.  Errors: MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED (adaptive capacity). */
int moe_cache_set_graph(moe_cache *c, int on);

/* Early launches for one-token decode calls (on by default).  The library keeps a
 * device copy of its slot table, updated by each wave's down + combine launch;
 * with on = 1, a one-token call launches the gate/up of the picks that copy
 * shows resident (and of the shared expert) right after the router, before
 * the host has read the routing and planned, and behind it their down +
 * combine, which writes the output only if the copy shows every pick resident.
 * The plan never moves a resident expert (explainer page, "The rules in the
 * code": hits are refreshed in place), so the early launches read the slots the
 * plan assigns.  Where the plan has no fill or eviction and the copy showed
 * every pick at its slot, the layer is complete and the host launches nothing
 * more for it; otherwise the plan's own launches cover the rest and compute the
 * output again.  Outputs are bitwise the same either way.
 * Errors: MOE_ERR_INVALID for on other than 0 or 1. */
int moe_cache_set_prelaunch(moe_cache *c, int on);

/* Adaptive per-layer capacity (MOE_ADAPTIVE_CAPACITY), after the 95 GiB
 * page, "Decode": capacity moves from layers with high hit rates to layers
 * with low ones, the total staying n_layers*K.  The page gives no schedule;
 * this library's: a decode step begins with a call of layer 0; every
 * `period` steps the layers with picks since the last rebalance are ranked
 * by pick hit rate (exact ratios, ties by layer), and the i-th highest gives
 * `delta` slots of target capacity to the i-th lowest, for i < pairs, while
 * its rate is strictly higher, it keeps at least `floor` slots and the taker
 * at most E.  A layer follows its target in its next plan: below it, it takes
 * free slots (lowest first) as least recently used; above it, after its hits
 * are refreshed, it releases its least recently used slots (their experts
 * are evicted and appear in that plan's trace record) but keeps as many as
 * the plan's distinct experts.  Waves are sized by min(slots held, target).
 * Defaults: period 8, delta 2, pairs 4, floor max(top_k, K/2).
 * Errors: MOE_ERR_INVALID for period < 1, delta < 0, pairs < 0,
 * floor < top_k or floor > K; MOE_ERR_UNSUPPORTED without the flag. */
int moe_cache_set_adaptive(moe_cache *c, int period, int delta, int pairs, int floor);

/* Slots a layer holds and its current target (both K without adaptive
 * capacity; host table, no GPU work). */
int moe_cache_layer_capacity(const moe_cache *c, int layer, int *held, int *target);

/* Routing of the last moe_layer_forward call, read from the host copies:
 * ids [n_tokens x top_k] and gate [n_tokens x top_k] (host memory; either
 * may be NULL).  n_tokens must equal that call's token count. */
int moe_cache_last_routing(const moe_cache *c, int32_t *ids, float *gate, int n_tokens);

/* Slot of (layer, expert) in its pool, -1 if not resident (host table). */
int moe_cache_slot_of(const moe_cache *c, int layer, int expert);

/* Device address of a pool slot's block (for tests of slot contents). */
int moe_cache_slot_ptr(const moe_cache *c, int layer, int slot, const void **out);

/* Waits for the cache's copy stream, frees what the cache allocated.  Prints
 * a one-line summary of the stats when the environment has MOE_CACHE_LOG=1. */
void moe_cache_destroy(moe_cache *c);

/* Message of the last error on the calling thread ("" if none). */
const char *moe_last_error(void);

/* Decoders of the 4-bit path on the GPU, for checking them against the
 * number formats' definitions: for every byte b of `codes` (device, n bytes),
 * out[2b], out[2b+1] (device fp32) receive
 *   quant MOE_Q_E2M1_E4M3_G16, what = 0: the two e2m1 values of byte b
 *     (low nibble first); what = 1: out[2b] = E4M3 value of byte b;
 *   quant MOE_Q_INT4_G32_F16: the two (q - 8) values of byte b.
 * Uses the same device decode routines as the expert kernels. */
int moe_debug_decode(int quant, int what, const uint8_t *codes, int n, float *out, void *stream);

/* Failure-path check (SGLang page, "Can paging change the model's outputs?": paging bugs
 * produce wrong outputs rather than crashes, so the failure paths are tested): the nth
 * upload submission from now (0 = the next) of this cache -- a demand upload run, a
 * speculative upload or a prefill arena upload -- fails as if its copy call had failed,
 * enqueuing nothing; -1 disarms.  A failed demand upload makes its forward call return
 * MOE_ERR_HIP with that wave's fills rolled back (the filled slots empty and least recently
 * used), so a later call uploads them again.  Two more checks are set by the environment
 * when a cache is created: MOE_DEBUG_POISON=1 fills every block an upload is about to
 * overwrite with all-one bytes (NaN scales) on the upload's stream first, and
 * MOE_DEBUG_DELAY_US=n (at most 100000) puts a kernel that waits n microseconds ahead of
 * every upload; a kernel that reads a block without waiting for its upload then reads NaN
 * or stale bytes.  Outputs and traces are unchanged by both.  MOE_DEBUG_ROUTER_WAIT_US=n
 * sets how many microseconds (at most 200000, the default) the one-launch router's selecting
 * workgroups wait for the other workgroups' logits before giving up (0: they give up at
 * once); a call whose selection gave up returns MOE_ERR_HIP, and so do later forward calls.
 * Errors: MOE_ERR_INVALID for nth < -1. */
int moe_debug_fail_upload(moe_cache *c, int nth);

#ifdef __cplusplus
}
#endif
#endif /* MOE_OFFLOAD_H */
