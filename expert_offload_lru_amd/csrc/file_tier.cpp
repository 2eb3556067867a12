// Two-tier store of the host runtime: expert blocks read from a file into an LRU of pinned
// RAM blocks, uploads from there.
#include "runtime_internal.hpp"

namespace {

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

}  // namespace

namespace rt {

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
               const char *touch_only) {
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

}  // namespace rt
