// Prefill calls of the host runtime (more than 32 tokens): grouping by expert, resident
// experts read in place, the others uploaded in batches through the arena, the grouped GEMM
// launches and the combine.
#include "runtime_internal.hpp"

namespace {

// ----------------------------------------------------------------------------- prefill

constexpr int kArenaBatch = 32;       // experts per batch (NVMe page, "Workflow")
constexpr int kSchedSlack = 64;       // dispatch-table entries allowed beyond 3 per (item, tile)

// Dispatch tables of the prefill GEMM launches.  The hardware hands workgroup b to
// XCD b % 8, and each XCD starts its workgroups in index order.  Items go to the
// XCDs longest first, each to the least loaded (an item costs about 1 + its
// 32-row tiles per column tile), and every XCD runs its items longest first, the
// column tiles of an item together; unused entries are -1.
struct XcdLists {
    std::vector<int> of[8];   // items of each XCD, in the order it runs them
};
void assign_xcds(const moe::PrefillItem *items, int n_items, XcdLists &xl) {
    std::vector<int> order(n_items);
    for (int i = 0; i < n_items; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return items[x].rows > items[y].rows; });
    int64_t load[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (auto &l : xl.of) l.clear();
    for (int i : order) {
        const int x = (int)(std::min_element(load, load + 8) - load);
        xl.of[x].push_back(i);
        load[x] += 1 + (items[i].rows + 31) / 32;
    }
}
// The table of one launch with n_tiles column tiles per item.  Returns its length, or 0
// when it would exceed cap (the launch then goes without a table).
int build_sched(const XcdLists &xl, int n_items, int n_tiles, int32_t *out, size_t cap) {
    size_t len = 0;
    for (const auto &l : xl.of) len = std::max(len, l.size() * (size_t)n_tiles);
    const size_t n = 8 * len;
    if (n > cap || n > (size_t)3 * n_items * n_tiles + kSchedSlack) return 0;
    std::fill(out, out + n, -1);
    for (int x = 0; x < 8; ++x)
        for (size_t q = 0; q < xl.of[x].size(); ++q)
            for (int t = 0; t < n_tiles; ++t) out[8 * (q * n_tiles + t) + x] = xl.of[x][q] * n_tiles + t;
    return (int)n;
}

size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

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
    if (c->pf_plan) hipFree(c->pf_plan);
    if (c->pf_host) hipHostFree(c->pf_host);
    c->pf_x16 = nullptr;
    c->pf_h16 = nullptr;
    c->pf_y = nullptr;
    c->pf_plan = nullptr;
    c->pf_host = nullptr;
    c->pf_host_dev = nullptr;
    c->pf_cap = 0;
    const size_t plan_bytes = align16(rows * sizeof(int32_t)) + align16(max_items * sizeof(moe::PrefillItem)) +
                              sched_cap * sizeof(int32_t);
    if ((e = hipMalloc(&c->pf_x16, (size_t)cap * c->H * 2)) != hipSuccess ||
        (e = hipMalloc(&c->pf_h16, rows * c->I * 2)) != hipSuccess ||
        (e = hipMalloc(&c->pf_y, rows * c->H * sizeof(float))) != hipSuccess ||
        (e = hipMalloc(&c->pf_plan, plan_bytes)) != hipSuccess ||
        (e = hipHostMalloc((void **)&c->pf_host, plan_bytes, hipHostMallocMapped | hipHostMallocCoherent)) !=
            hipSuccess)
        return set_error(MOE_ERR_OOM, std::string("prefill workspace: ") + hipGetErrorString(e));
    void *host_dev = nullptr;
    if ((e = hipHostGetDevicePointer(&host_dev, c->pf_host, 0)) != hipSuccess) return hip_fail(e, "hipHostGetDevicePointer");
    c->pf_host_dev = static_cast<const uint8_t *>(host_dev);
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
    std::vector<int32_t> experts, slots, count;
    if (c->pl.prefill_lookup(layer, c->h_ids, nk, experts, slots, &count) != moe::PLAN_OK)
        return set_error(MOE_ERR_INVALID, "router produced an expert id out of range");
    std::vector<int32_t> start(c->E, 0);
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
    // the plan's parts: pairs, items, dispatch tables (same offsets on the device)
    const size_t items_off = align16(rows * sizeof(int32_t));
    moe::PrefillItem *items = reinterpret_cast<moe::PrefillItem *>(c->pf_host + items_off);
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
    const size_t sched_off = items_off + align16(n_items * sizeof(moe::PrefillItem));
    int32_t *sched = reinterpret_cast<int32_t *>(c->pf_host + sched_off);
    size_t n_sched = 0;
    XcdLists xl;
    for (Batch &bt : batches) {
        assign_xcds(items + bt.item_begin, bt.item_end - bt.item_begin, xl);
        for (int nm = 1; nm <= 2; ++nm) {
            const int n = build_sched(xl, bt.item_end - bt.item_begin, moe::prefill_tiles(nm, nm == 2 ? c->I : c->H),
                                      sched + n_sched, c->pf_sched_cap - n_sched);
            bt.sched_off[nm - 1] = (int)n_sched;
            bt.sched_n[nm - 1] = n;
            n_sched += n;
        }
    }
    c->plan_us += now_us() - tp;

    // the plan to the device in one copy, by a kernel ahead of the GEMMs on their stream (a
    // copy-engine transfer would add the hand-over between the engines to every layer)
    HostClock hc_launch(c->launch_us);   // from here on: copies and launches
    if ((err = moe::launch_copy_from_host(c->pf_host_dev, c->pf_plan, sched_off + n_sched * sizeof(int32_t), stream)) !=
        hipSuccess)
        return hip_fail(err, "prefill plan copy");
    const int32_t *d_pairs = reinterpret_cast<const int32_t *>(c->pf_plan);
    const moe::PrefillItem *d_items = reinterpret_cast<const moe::PrefillItem *>(c->pf_plan + items_off);
    const int32_t *d_sched = reinterpret_cast<const int32_t *>(c->pf_plan + sched_off);

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
            g.items = d_items + bt.item_begin;
            g.n_items = bt.item_end - bt.item_begin;
            g.pairs = d_pairs;
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
                g.sched = d_sched + bt.sched_off[nm - 1];
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

}  // namespace

namespace rt {

int prefill_forward(moe_cache *c, int layer, const float *x, int n_tok, const float *router_w, const void *shared_w,
                    float *out, unsigned fflags, hipStream_t stream) {
    discard_ahead(c);
    return prefill_forward_impl(c, layer, x, n_tok, router_w, shared_w, out, fflags, stream);
}

}  // namespace rt
