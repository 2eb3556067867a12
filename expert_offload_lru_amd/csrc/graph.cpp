// Captured decode steps of the host runtime (moe_cache_set_graph).
#include "runtime_internal.hpp"

namespace {

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
    c->map_dirty = false;
    c->resident_checked = c->plan_changes;
    return MOE_OK;
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
        ra.zx = c->d_zx;
        ra.timed_out = c->h_wait_timeout_dev;
        ra.wait_us = c->router_wait_us;
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
        // the next layer's router matrix comes from HBM otherwise (a step streams far more
        // expert bytes than the cache holds): requested into the cache while the down runs
        if (l + 1 < c->L) {
            cb.pf = router_ws[l + 1];
            cb.pf_rows = c->E;
            cb.pf_cols = c->H;
        }
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

}  // namespace

namespace rt {

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
    if (c->h_wait_timeout && *(volatile int *)c->h_wait_timeout)
        return set_error(MOE_ERR_HIP, "a router selection stopped waiting for its logits; outputs since then are "
                                      "not valid");
    return flush_graph(c);
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

}  // namespace rt
