// Uploads of the host runtime: demand uploads of a wave's fills, speculative uploads into
// the staging bank, the copy queues' backlog, and the fence checks ahead of every upload.
#include "runtime_internal.hpp"

namespace {

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

}  // namespace

namespace rt {

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

}  // namespace rt
