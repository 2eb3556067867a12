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
//
// This file: the cache object's life cycle and the C ABI's set-up, statistics, timing and
// inspection calls; kernel timing.  Decode calls are in decode.cpp, uploads in
// uploads.cpp, the two-tier store in file_tier.cpp, captured steps in graph.cpp, prefill
// calls in prefill_host.cpp.
#include "runtime_internal.hpp"

namespace {

// ----------------------------------------------------------------------------- timing

// ----------------------------------------------------------------------------- unit lists

int check_shapes(int quant, int hidden, int inter) {
    for (int n_mats = 1; n_mats <= 2; ++n_mats) {
        const int cols = n_mats == 2 ? hidden : inter;
        if (!moe::gemv_shape(quant, cols, n_mats).ok) return MOE_ERR_UNSUPPORTED;
    }
    return MOE_OK;
}

// The current call reads its routing from set st.
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
    if (c->d_zx) hipFree(c->d_zx);
    if (c->d_fused_sync) hipFree(c->d_fused_sync);
    if (c->d_map) hipFree(c->d_map);
    if (c->h_wait_timeout) hipHostFree(c->h_wait_timeout);
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
    if (c->pf_plan) hipFree(c->pf_plan);
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

namespace rt {

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
            case 7: k = &c->timing.down_early; break;
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

}  // namespace rt

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
    if (const char *v = getenv("MOE_DEBUG_ROUTER_WAIT_US"))
        c->router_wait_us = (unsigned)std::min((long)moe::kRouterWaitUs, std::max(0L, atol(v)));
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
            (e = hipMalloc(&c->d_zx, moe::router_exchange_bytes(E))) != hipSuccess ||
            (e = hipMemset(c->d_zx, 0xFF, moe::router_exchange_bytes(E))) != hipSuccess ||
            (e = hipMalloc(&c->d_fused_sync, moe::kSyncBytes)) != hipSuccess ||
            (e = hipMemset(c->d_fused_sync, 0, moe::kSyncBytes)) != hipSuccess ||
            (e = hipMalloc(&c->d_map, (size_t)n_layers * E * sizeof(int32_t))) != hipSuccess ||
            (e = hipMemset(c->d_map, 0xFF, (size_t)n_layers * E * sizeof(int32_t))) != hipSuccess) {
            free_cache(c);
            return set_error(MOE_ERR_OOM, std::string("activation/stack buffers: ") + hipGetErrorString(e));
        }
        if ((e = hipHostMalloc((void **)&c->h_wait_timeout, sizeof(int), hipHostMallocMapped | hipHostMallocCoherent)) !=
            hipSuccess) {
            free_cache(c);
            return set_error(MOE_ERR_OOM, std::string("pinned flag: ") + hipGetErrorString(e));
        }
        *c->h_wait_timeout = 0;
        c->map_shadow.assign((size_t)n_layers * E, -1);
        c->map_keys.reserve((size_t)n_layers * E);
        c->map_vals.reserve((size_t)n_layers * E);
        if ((e = hipHostGetDevicePointer((void **)&c->h_wait_timeout_dev, c->h_wait_timeout, 0)) != hipSuccess) {
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

}  // extern "C"

extern "C" {

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
