/*
 * moe_planner.h -- C ABI of the host slot table alone (no GPU), exported by
 * both expert_offload_lru_amd/libmoe_planner.so (built with a plain C++
 * compiler, no HIP) and libmoe_offload.so.  It is the same code the GPU
 * library plans with, exposed so the LRU behaviour can be checked on a CPU.
 *
 * The method (explainer page "MoE expert offload and the LRU expert cache
 * that llama.cpp and SGLang both merged in October 2026", section "Inside
 * llama.cpp PR #29887: slot maps, banks, and only the misses cross PCIe";
 * SGLang page, section "What happens with more than one request?"): per plan,
 * resident experts are refreshed first, then missing experts in ascending
 * order take the least recently used slots; a decode call whose
 * tokens * top_k exceed K runs in waves of K / top_k tokens.
 */
#ifndef MOE_PLANNER_H
#define MOE_PLANNER_H

#include <stddef.h>
#include <stdint.h>

#include "moe_offload.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_planner moe_planner;

/* E experts, K slots (per layer, or total with MOE_POOL_SHARED in flags),
 * top_k, n_layers, block_bytes = S for the byte counters.
 * Errors: MOE_ERR_INVALID, MOE_ERR_CACHE_TOO_SMALL (K < top_k). */
int moe_planner_create(int E, int K, int top_k, int n_layers, unsigned flags,
                       size_t block_bytes, moe_planner **out);
void moe_planner_destroy(moe_planner *p);

/* Plan a decode call: ids [n_tokens x top_k] (host, token-major, rank order).
 * Writes slots [n_tokens x top_k] (host) and calls `fn` once per wave
 * (gate is NULL in those records).  n_waves_out (may be NULL) receives the
 * number of waves.  On error the pools are unchanged for the failing wave.
 * Errors: MOE_ERR_INVALID (ids out of range, bad layer), MOE_ERR_CACHE_TOO_SMALL. */
int moe_planner_decode(moe_planner *p, int layer, const int32_t *ids, int n_tokens,
                       int32_t *slots, moe_trace_fn fn, void *user, int *n_waves_out);

/* Prefill lookup of n_ids ids: the touched experts ascending (experts, at
 * most E entries) and the slot of each or -1 (slots); *n_out receives the
 * count.  The pools are not changed; the prefill bucket is counted. */
int moe_planner_prefill(moe_planner *p, int layer, const int32_t *ids, int n_ids,
                        int32_t *experts, int32_t *slots, int *n_out);

/* Recency order of the pool of `layer` (least recent first): K entries, or
 * with MOE_ADAPTIVE_CAPACITY the slots the layer holds (moe_planner_capacity). */
int moe_planner_order(const moe_planner *p, int layer, int32_t *order);

/* Adaptive capacity parameters and state, as moe_cache_set_adaptive and
 * moe_cache_layer_capacity.  A decode call of layer 0 begins a step. */
int moe_planner_set_adaptive(moe_planner *p, int period, int delta, int pairs, int floor);
int moe_planner_capacity(const moe_planner *p, int layer, int *held, int *target);

/* Coalesced copy runs of the last plan of the last decode call: triples
 * (expert, slot, n) into runs[3*i..], at most max_runs; *n_out = count. */
int moe_planner_last_runs(const moe_planner *p, int32_t *runs, int max_runs, int *n_out);

/* Test hook: undo the fills of the last plan (what the GPU library does when
 * an upload cannot be submitted). */
int moe_planner_rollback_last(moe_planner *p);

int moe_planner_stats(const moe_planner *p, moe_stats *out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PLANNER_H */
