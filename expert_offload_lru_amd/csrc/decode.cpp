// Decode calls of the host runtime (at most 32 tokens): routing buffers and readback, the
// router and expert launches, the wave loop, the layer and stack entry points, and the
// allocation-free decode call.
#include "runtime_internal.hpp"

namespace {

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
        c->map_carried = plan && cb.map != nullptr;
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
    fs.timed_out = c->h_wait_timeout_dev;

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

// One token: the down + combine of the picks that the device copy of the slot table shows
// resident, queued behind their early gate/up.  It writes `out` only where that copy covers
// every pick; the plan then tells whether what it wrote is the layer's output (the host
// launches the down itself otherwise, which overwrites it).
int prelaunch_down(moe_cache *c, int layer, const void *shared_w, const float *x, float *out, unsigned fflags,
                   hipStream_t stream, hipEvent_t *ev_a, hipEvent_t *ev_b) {
    moe::GemvArgs g;
    moe::PreArgs pa;
    pre_args(c, layer, shared_w, nullptr, g, pa);
    moe::GemvArgs d{};
    d.bank = c->pool_base(layer);
    d.staging = c->staging;
    d.shared_w = (const uint8_t *)shared_w;
    d.copy_bank = const_cast<uint8_t *>(c->pool_base(layer));
    d.block_bytes = c->S;
    d.mat_off0 = 2 * matrix_bytes(c->quant, c->I, c->H);
    d.rows = c->H;
    d.cols = c->I;
    d.vec = c->d_h;
    d.vec_by_token = 0;
    d.nk = c->k;
    d.top_k = c->k;
    moe::CombineArgs cb{};
    cb.x = (fflags & MOE_FWD_RESIDUAL) ? x : nullptr;
    cb.gate = c->d_gate;
    cb.out = out;
    cb.t0 = 0;
    cb.nt = 1;
    cb.has_shared = shared_w ? 1 : 0;
    cb.map = c->d_map;
    cb.n_upd = 0;
    TimeScope ts(c, 7, 0.0, 0.0);
    hipError_t err;
    {
        HostClock hc(c->launch_us);
        err = moe::launch_down_combine_picks(c->quant, d, cb, pa, nullptr, stream, ts.a, ts.b);
    }
    *ev_a = ts.a;
    *ev_b = ts.b;
    ts.a = ts.b = nullptr;    // recorded by the caller with the bytes it turns out to have read
    if (err != hipSuccess) {
        if (*ev_a) c->event_pool.push_back(*ev_a);
        if (*ev_b) c->event_pool.push_back(*ev_b);
        *ev_a = *ev_b = nullptr;
        return hip_fail(err, "down+combine launch (resident picks)");
    }
    return MOE_OK;
}

// Make the device copy of the slot table exact: the entries where the shadow differs from
// the host's table are written by small kernels on `stream`, ahead of the kernels that read
// them and after every down launch whose updates they supersede (no allocation, no host
// buffer that must outlive the call).
int sync_map(moe_cache *c, hipStream_t stream) {
    c->map_dirty = false;
    std::vector<int32_t> &keys = c->map_keys, &vals = c->map_vals;
    keys.clear();
    vals.clear();
    for (int l = 0; l < c->L; ++l)
        for (int e = 0; e < c->E; ++e) {
            const size_t key = (size_t)l * c->E + e;
            const int32_t want = c->pl.slot_of(l, e);
            if (c->map_shadow[key] != want) {
                c->map_shadow[key] = want;
                keys.push_back((int32_t)key);
                vals.push_back(want);
            }
        }
    if (keys.empty()) return MOE_OK;
    HostClock hc(c->launch_us);
    const hipError_t e = moe::launch_map_set(c->d_map, keys.data(), vals.data(), (int)keys.size(), stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "slot table update");
}

// Whether a one-token call of `layer`, routed into set st, will likely find every pick
// resident where the device copy of the slot table shows it: from the previous call's
// speculative ids for this layer, where that call was the layer before at one token (else,
// or while they have not landed, yes).  A guess only: it decides whether the early down +
// combine is worth launching, never what the output is.
bool picks_likely_resident(const moe_cache *c, int layer, int st) {
    const moe_cache::RouteSet &prev = c->rs[1 - st];
    if (prev.layer != layer - 1 || prev.n_tok != 1 || prev.n_spec < 1 || !prev.spec) return true;
    const volatile int32_t *spec = prev.spec;    // its first speculated layer is this one
    for (int j = 0; j < c->k; ++j) {
        const int32_t e = spec[j];
        if (e < 0 || e >= c->E) return true;
        const int32_t slot = c->pl.slot_of(layer, e);
        if (slot < 0 || c->map_shadow[(size_t)layer * c->E + e] != slot) return false;
    }
    return true;
}

// Launch a decode call's router, writing its host results into routing set st, and for
// one token the early gate/up of its resident picks and, when they are likely all
// resident, their down + combine; c->ahead describes the call.
int issue_route(moe_cache *c, int layer, const float *x, int n_tok, const float *router_w, const void *shared_w,
                const float *const *spec_ws, int n_spec, float *out, unsigned fflags, hipStream_t stream, int st) {
    const bool f32 = c->quant == MOE_Q_F32;
    const bool early = n_tok == 1 && c->prelaunch && !c->fuse_decode;
    if (early && c->map_dirty) {
        if (int rc = sync_map(c, stream)) return rc;
    }
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
    ra.zx = c->d_zx;
    ra.timed_out = c->h_wait_timeout_dev;
    ra.wait_us = c->router_wait_us;
    mark_routing(c, st, n_tok, n_spec);
    hipError_t err;
    {
        const double bytes = (double)(1 + n_spec) * c->E * c->H * 4 + (double)n_tok * c->H * 4;
        TimeScope ts(c, 0, bytes, 2.0 * (1 + n_spec) * c->E * (double)c->H * n_tok);
        HostClock hc(c->launch_us);
        if ((err = moe::launch_router(ra, stream, ts.a, ts.b)) != hipSuccess) return hip_fail(err, "router launch");
    }
    // before this set's identity changes: the other set holds the previous call's guesses
    const bool down_early = early && picks_likely_resident(c, layer, st);
    c->rs[st].layer = layer;
    c->rs[st].n_tok = n_tok;
    c->rs[st].n_spec = n_spec;
    moe_cache::Ahead a;
    a.on = true;
    a.layer = layer;
    a.n_tok = n_tok;
    a.n_spec = n_spec;
    a.set = st;
    a.x = x;
    a.stream = stream;
    a.out = out;
    a.fflags = fflags;
    // one token: the resident picks' gate/up and down + combine go out at once, before the
    // host trip; the plan then launches only what they did not cover
    a.pre = early;
    if (a.pre) {
        int rc = prelaunch_gate_up(c, layer, shared_w, f32 ? (const void *)x : c->d_xq, stream, &a.pre_a, &a.pre_b);
        if (!rc && down_early) rc = prelaunch_down(c, layer, shared_w, x, out, fflags, stream, &a.pre_da, &a.pre_db);
        if (rc) {
            if (a.pre_a) c->event_pool.push_back(a.pre_a);
            if (a.pre_b) c->event_pool.push_back(a.pre_b);
            return rc;
        }
        a.pre_down = down_early;
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

// The stack driver's next call, whose router the current call launches once its own
// expert kernels are queued.
struct NextCall {
    const float *x;
    const float *router_w;
    const void *shared_w;
    const float *const *spec_ws;
    int n_spec_in;
    float *out;
    unsigned fflags;
};

int decode_forward(moe_cache *c, int layer, const float *x, int n_tok, const float *router_w, const void *shared_w,
                   const float *const *spec_ws, int n_spec_in, float *out, unsigned fflags, hipStream_t stream,
                   const NextCall *next = nullptr) {
    int rc = ensure_route_capacity(c, n_tok);
    if (rc) return rc;
    if (*(volatile int *)c->h_wait_timeout)
        return set_error(MOE_ERR_HIP, "a kernel stopped waiting for other workgroups (a router selection for its "
                                      "logits, or a fused expert launch for its gate/up); outputs since then are "
                                      "not valid");
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
                         c->ahead.stream == stream && c->ahead.n_spec == n_spec && c->ahead.out == out &&
                         c->ahead.fflags == fflags))
        discard_ahead(c);
    if (!c->ahead.on && (rc = issue_route(c, layer, x, n_tok, router_w, shared_w, spec_ws, n_spec, out, fflags,
                                          stream, 1 - c->rcur)) != MOE_OK)
        return rc;
    use_route_set(c, c->ahead.set);
    const bool pre = c->ahead.pre, pre_down = c->ahead.pre_down;
    hipEvent_t pre_a = c->ahead.pre_a, pre_b = c->ahead.pre_b, pre_da = c->ahead.pre_da, pre_db = c->ahead.pre_db;
    c->ahead = moe_cache::Ahead();
    struct EventsBack {      // timing events of the early launches go back to the pool on an early return
        moe_cache *c;
        hipEvent_t &a, &b, &da, &db;
        ~EventsBack() {
            for (hipEvent_t e : {a, b, da, db})
                if (e) c->event_pool.push_back(e);
        }
    } events_back{c, pre_a, pre_b, pre_da, pre_db};
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
        // the early down + combine wrote the layer's output if the early gate/up covered every
        // unit and the plan changed nothing (one wave; no fill, no eviction): then the layer
        // is complete, else the launches below compute it (overwriting what it wrote)
        const bool early_done = pre_down && !multi_wave && p.fills.empty() && p.evictions.empty() && gu->u.empty();
        if (pre_da) {
            const size_t np_all = units.pairs.size();
            c->timed.push_back({7, pre_da, pre_db,
                                early_done ? gemv_bytes(c, (int)units.u.size(), (int)np_all, 1, 0) +
                                                 (double)c->H * 4 * ((fflags & MOE_FWD_RESIDUAL) ? 2 : 1)
                                           : 0.0,
                                early_done ? 2.0 * np_all * (double)c->H * c->I : 0.0});
            pre_da = pre_db = nullptr;
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
        c->map_carried = false;
        if (!fused && !early_done) {
            rc = down_and_combine(c, layer, units, shared_w, n_tok, t0, t1, x, out, residual, has_shared, stream,
                                  c->prelaunch ? &p : nullptr);
            if (rc) return rc;
        }
        if ((!p.fills.empty() || !p.evictions.empty()) && !c->map_carried) c->map_dirty = true;
        // the stack driver's next layer: its router (and early gate/up) go out now, queued behind
        // this layer's kernels, before the host's remaining bookkeeping for this call
        if (next && w + 1 == c->wave_ranges.size() && layer + 1 < c->L) {
            const int nn = spec_count(c, layer + 1, next->spec_ws, next->n_spec_in);
            if ((rc = issue_route(c, layer + 1, next->x, n_tok, next->router_w, next->shared_w, next->spec_ws, nn,
                                  next->out, next->fflags, stream, 1 - c->rcur)) != MOE_OK)
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

}  // namespace

namespace rt {

// Forget a call launched ahead that is not the one now made (only after an error): its
// router may still be queued, so the stream drains before its buffers are reused.
void discard_ahead(moe_cache *c) {
    if (!c->ahead.on) return;
    hipStreamSynchronize(c->ahead.stream);
    for (hipEvent_t e : {c->ahead.pre_a, c->ahead.pre_b, c->ahead.pre_da, c->ahead.pre_db})
        if (e) c->event_pool.push_back(e);
    c->ahead = moe_cache::Ahead();
}

// Captured steps name the routing buffers: they go when those are reallocated (after the
// step in flight, if any, has finished).
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

}  // namespace rt

extern "C" {

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
    size_t z, zx, xq, h, y, ids, gate, total;
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
    l.zx = take(moe::router_exchange_bytes(c->E));
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
    // the router's exchange array starts as all sentinels (each launch leaves it so; the array
    // keeps whatever the last call on this GPU left)
    hipError_t e = moe::launch_fill_u32((unsigned *)(base + lay.zx), 0xFFFFFFFFu,
                                        moe::router_exchange_bytes(c->E) / sizeof(unsigned), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "scratch exchange fill");
    // the call's kernels take the array's buffers; kernel timing (which creates events) is off
    struct Swap {
        moe_cache *c;
        double *z, *zx;
        void *xq;
        float *h, *y, *gate;
        int32_t *ids;
        unsigned mask;
        ~Swap() {
            c->d_z = z;
            c->d_zx = zx;
            c->d_xq = xq;
            c->d_h = h;
            c->d_y = y;
            c->d_ids = ids;
            c->d_gate = gate;
            c->time_mask = mask;
        }
    } swap{c, c->d_z, c->d_zx, c->d_xq, c->d_h, c->d_y, c->d_gate, c->d_ids, c->time_mask};
    c->d_z = (double *)(base + lay.z);
    c->d_zx = (double *)(base + lay.zx);
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
        float *next_dst = (l + 1 == c->L - 1) ? out : c->d_stack[(l + 1) & 1];
        NextCall next{dst, l + 1 < c->L ? router_ws[l + 1] : nullptr,
                      shared_ws && l + 1 < c->L ? shared_ws[l + 1] : nullptr, next_spec_ws, n_next_spec, next_dst,
                      MOE_FWD_RESIDUAL};
        int rc = stack_layer(c, l, in, n_tokens, router_ws[l], shared_ws ? shared_ws[l] : nullptr, spec_ws, n_spec, dst,
                             stream, l + 1 < c->L && c->layer_ready[l + 1] ? &next : nullptr);
        if (rc) return rc;
        in = dst;
    }
    return MOE_OK;
}

}  // extern "C"
