// Router for gfx950: float64 logits, softmax and top-k.
//
// What it computes (explainer page, "The model that should not fit": a small
// router in front of the experts reads each token and picks a few; SGLang
// page, "What does Paged Experts actually do?": top_k of E experts per token):
//   z[t,e] = sum_i W[e,i] x[t,i]       float32 operands, float64 accumulation
//   p[t,:] = softmax(z[t,:])           exp, sum and quotient in float32, from z - max z
//   ids[t,:] = the top_k experts by z, descending, equal z to the lower index
//   gate[t,j] = p[t, ids[t,j]]          (not renormalised over the picks)
// With further matrices (the next layers' routers) the same launch also picks
// those layers' top_k on the same input, for speculative prefetch (NVMe page,
// "Workflow": the next layer's router run on the current layer's input).
//
// Logits: one wave per (matrix, expert row) and block of tokens, streaming the
// row with 16-byte loads; the per-token sums are reduced with a halving
// butterfly (each exchange halves the values a lane holds) and DPP moves.  The
// same launch writes the fp16 copy of x the expert GEMV reads.
// Selection: one wave per (matrix, token): softmax and k rounds of a wave
// arg-max over the heads of per-lane sorted lists of packed (logit, index) keys.
// A round compares the upper 32 bits of the heads (one DPP max per step) and
// accepts the round's lane if it alone holds that maximum, which gives the pick
// the whole key would; a tie in those bits reruns the k rounds on the 64-bit
// keys.  Lane j keeps pick j, and the lanes holding picks compute and store the
// gates together at the end.
//
// Selection needs every logit of its token, which other workgroups produce.
// Up to four tokens, one launch does both.  The logits go to an exchange array
// whose entries hold a sentinel between launches, with agent-scope atomic
// stores (coherent across the eight XCDs without a cache writeback); the
// workgroups that produce them exit.  The last workgroup of each matrix, which
// the dispatcher starts after that matrix's others, computes its own rows and
// then reads its tokens' logits with agent-scope atomic loads until no
// sentinel is left, selects from the values it holds, and puts the sentinels
// back.  (A ticket counter would need each producer to wait for its stores to
// complete and a second round trip for the ticket before the selector could
// read; a release fence would write back a whole L2.)  The wait is bounded:
// after wait_us microseconds the selection stops, marks the token's device ids
// invalid, raises a host flag and writes no results.
// Larger batches use two launches (logits, then selection).
#include <cfloat>

#include "kernels.hpp"

namespace moe {
namespace {

typedef _Float16 f16;
constexpr int kRowsPerWg = kRouterRowsPerWg;

// Logit stores: plain, or relaxed agent-scope atomics (one launch path).
template <bool COHERENT>
__device__ inline void store_z(double *p, double v) {
    if constexpr (COHERENT)
        __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), __builtin_bit_cast(unsigned long long, v),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

__device__ inline int dpp_i(int v, int ctrl) {
    switch (ctrl) {
        case 0: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);    // quad xor 1
        case 1: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);    // quad xor 2
        case 2: return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true);   // half-row mirror
        default: return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, true); // row mirror
    }
}

__device__ inline double dpp_f64(double v, int ctrl) {
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = dpp_i((int)(b & 0xFFFFFFFF), ctrl), hi = dpp_i((int)(b >> 32), ctrl);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

__device__ inline double readlane_f64(double v, int l) {
    const long long b = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFF), l);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

// fp16 copy of x for the gate/up GEMV, a slice per workgroup: 8 elements per item.
__device__ inline void write_xq(const RouterArgs &a, int t0, int nt, int part, int n_parts) {
    if (!a.xq) return;
    const int n8 = a.H / 8;
    const int per = (n8 + n_parts - 1) / n_parts;
    const int b0 = part * per, b1 = min(b0 + per, n8);
    if (b1 <= b0) return;
    for (int item = threadIdx.x; item < nt * (b1 - b0); item += 256) {      // workgroups of 256
        const int t = t0 + item / (b1 - b0);
        const int g = b0 + item % (b1 - b0);
        const float4 lo = *reinterpret_cast<const float4 *>(a.x + (size_t)t * a.H + 8 * g);
        const float4 hi = *reinterpret_cast<const float4 *>(a.x + (size_t)t * a.H + 8 * g + 4);
        const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        f16 o[8];
        if (a.quant == Q_INT4 && !a.xq_natural) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {       // pairs (0,4) (1,5) (2,6) (3,7)
                o[2 * m] = (f16)v[m];
                o[2 * m + 1] = (f16)v[m + 4];
            }
        } else {
#pragma unroll
            for (int m = 0; m < 8; ++m) o[m] = (f16)v[m];
        }
        *reinterpret_cast<uint4 *>(reinterpret_cast<f16 *>(a.xq) + (size_t)t * a.H + 8 * g) =
            __builtin_bit_cast(uint4, o);
    }
}

// Logits of row gr (matrix gr / E, expert gr % E) for tokens t0 .. t0+nt-1 (nt <= TB).
template <int TB, bool COHERENT>
__device__ inline void logits_row(const RouterArgs &a, double *zout, int n_mats, int gr, int t0, int nt, int lane) {
    constexpr int LOG = (TB == 1) ? 0 : (TB == 4 ? 2 : (TB == 8 ? 3 : 5));
    static_assert((1 << LOG) == TB, "TB is 1, 4, 8 or 32");
    if (gr >= n_mats * a.E) return;
    const int m = gr / a.E;
    const int e = gr - m * a.E;
    const float *w = (m == 0 ? a.w0 : a.wspec[m - 1]) + (size_t)e * a.H;
    double v[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) v[t] = 0.0;
    // up to 8 16-byte loads of the row per lane (H <= 2048) in flight at once, then the
    // token FMAs; longer rows take further rounds.  Loads past the row end re-read its
    // first chunk (in bounds, no branch that would split the loads apart) and count zero.
    constexpr int XT = TB <= 4 ? TB : 1;    // tokens whose x chunks load together with the row
    for (int h0 = lane * 4; h0 < a.H; h0 += 2048) {
        float4 wv[8];
        float4 xa[XT][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int h = h0 + 256 * u;
            wv[u] = *reinterpret_cast<const float4 *>(w + (h < a.H ? h : h0));
        }
#pragma unroll
        for (int t = 0; t < XT; ++t) {
            const float *xr = a.x + (size_t)(t0 + (t < nt ? t : 0)) * a.H;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int h = h0 + 256 * u;
                xa[t][u] = *reinterpret_cast<const float4 *>(xr + (h < a.H ? h : h0));
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (h0 + 256 * u >= a.H) wv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < nt) {
                float4 xv[8];
                if constexpr (XT == TB) {
#pragma unroll
                    for (int u = 0; u < 8; ++u) xv[u] = xa[t][u];
                } else {
                    const float *xr = a.x + (size_t)(t0 + t) * a.H;
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int h = h0 + 256 * u;
                        xv[u] = *reinterpret_cast<const float4 *>(xr + (h < a.H ? h : h0));
                    }
                }
                double s = v[t];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    s = fma((double)wv[u].x, (double)xv[u].x, s);
                    s = fma((double)wv[u].y, (double)xv[u].y, s);
                    s = fma((double)wv[u].z, (double)xv[u].z, s);
                    s = fma((double)wv[u].w, (double)xv[u].w, s);
                }
                v[t] = s;
            }
        }
    }
    // halving butterfly: after the step with mask M a lane keeps the half of its
    // values selected by lane bit M; LOG steps leave one value per lane, for the
    // token in lane bits 5 .. 6-LOG
    int n = TB;
#pragma unroll
    for (int st = 0; st < LOG; ++st) {
        const int mask = 32 >> st;
        const bool upper = (lane & mask) != 0;
        n >>= 1;
#pragma unroll
        for (int i = 0; i < TB / 2; ++i) {
            if (i < n) {
                const double send = upper ? v[i] : v[i + n];
                const double keep = upper ? v[i + n] : v[i];
                v[i] = keep + __shfl_xor(send, mask);
            }
        }
    }
    // the remaining lane bits 0 .. 5-LOG: DPP within rows of 16, lane reads across rows
    double s = v[0];
    constexpr int REST = 6 - LOG;
#pragma unroll
    for (int st = 0; st < (REST < 4 ? REST : 4); ++st) s += dpp_f64(s, st);
    if constexpr (REST == 6) s = (readlane_f64(s, 0) + readlane_f64(s, 16)) + (readlane_f64(s, 32) + readlane_f64(s, 48));
    static_assert(REST <= 4 || REST == 6, "token blocks of 1, 4, 8 or 32");
    const int tok = (lane >> REST) & (TB - 1);
    const bool writer = (lane & ((1 << REST) - 1)) == 0;
    if (writer && tok < nt) store_z<COHERENT>(zout + ((size_t)m * a.n_tok + t0 + tok) * a.E + e, s);
}

template <int TB>
__global__ __launch_bounds__(256) void k_router_logits(RouterArgs a, int n_mats) {
    const int t0 = blockIdx.y * TB;
    const int nt = min(TB, a.n_tok - t0);
    // the wave index is uniform: keep it (and the matrix pointer it selects) scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    logits_row<TB, false>(a, a.z, n_mats, blockIdx.x * kRowsPerWg + wave, t0, nt, threadIdx.x & 63);
    write_xq(a, t0, nt, blockIdx.x, gridDim.x);      // after the row loads went out
}

// Logits of more than 32 tokens on the matrix cores: v_mfma_f64_16x16x4_f64 takes
// the fp32 operands widened to float64 (exact) and accumulates in float64, the
// same arithmetic as the row kernel's FMAs up to the order of the sums.  A wave
// computes 16 tokens x 16 experts of one matrix; the 4 waves of a workgroup share
// the tokens (64 experts).  Lane l supplies A[l%16][l/16] (token l%16) and
// B[l/16][l%16] (expert l%16); register r of the result is token l/16 + 4r,
// expert l%16.  Within a round of 32 reduction elements, lane group q = l/16
// holds elements 8q .. 8q+7, step s of the round uses element 8q + s on both
// operands.  Tokens and experts past the ends are clamped for loading and not
// stored.  H must be a multiple of 32.
typedef double d4v __attribute__((ext_vector_type(4)));
constexpr int kMfmaTok = 16;

__global__ __launch_bounds__(256) void k_router_logits_mfma(RouterArgs a, int n_mats) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int eb = (a.E + 63) / 64;
    const int m = blockIdx.y / eb;
    const int e0 = (blockIdx.y - m * eb) * 64 + 16 * wave;
    const int t0 = blockIdx.x * kMfmaTok;
    const int i = lane & 15, q = lane >> 4;
    const float *w = m == 0 ? a.w0 : a.wspec[m - 1];
    const float *xr = a.x + (size_t)min(t0 + i, a.n_tok - 1) * a.H + 8 * q;
    const float *wr = w + (size_t)min(e0 + i, a.E - 1) * a.H + 8 * q;
    d4v acc[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
    float4 xa[4][2], wa[4][2];   // rounds r .. r+3 in flight
    auto load = [&](int set, int k0) {
        xa[set][0] = *reinterpret_cast<const float4 *>(xr + k0);
        xa[set][1] = *reinterpret_cast<const float4 *>(xr + k0 + 4);
        wa[set][0] = *reinterpret_cast<const float4 *>(wr + k0);
        wa[set][1] = *reinterpret_cast<const float4 *>(wr + k0 + 4);
    };
    auto round = [&](int set) {
        const float xv[8] = {xa[set][0].x, xa[set][0].y, xa[set][0].z, xa[set][0].w,
                             xa[set][1].x, xa[set][1].y, xa[set][1].z, xa[set][1].w};
        const float wv[8] = {wa[set][0].x, wa[set][0].y, wa[set][0].z, wa[set][0].w,
                             wa[set][1].x, wa[set][1].y, wa[set][1].z, wa[set][1].w};
#pragma unroll
        for (int st = 0; st < 8; ++st)
            acc[st & 1] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[st], (double)wv[st], acc[st & 1], 0, 0, 0);
    };
    const int n_rounds = a.H / 32;
    load(0, 0);
    load(1, min(1, n_rounds - 1) * 32);
    load(2, min(2, n_rounds - 1) * 32);
    int r = 0;
    for (; r + 4 <= n_rounds; r += 4) {
        load(3, min(r + 3, n_rounds - 1) * 32);
        round(0);
        load(0, min(r + 4, n_rounds - 1) * 32);
        round(1);
        load(1, min(r + 5, n_rounds - 1) * 32);
        round(2);
        load(2, min(r + 6, n_rounds - 1) * 32);
        round(3);
    }
    // the last 1 .. 3 rounds sit in sets 0 .. 2
    if (r < n_rounds) round(0);
    if (r + 1 < n_rounds) round(1);
    if (r + 2 < n_rounds) round(2);
    const int e = e0 + i;
    if (e < a.E) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int t = t0 + q + 4 * k;
            if (t < a.n_tok) a.z[((size_t)m * a.n_tok + t) * a.E + e] = acc[0][k] + acc[1][k];
        }
    }
    // the fp16 copy of x for the expert kernels: the workgroups of a token block share it
    write_xq(a, t0, min(kMfmaTok, a.n_tok - t0), blockIdx.y, gridDim.y);
}

// --- selection -------------------------------------------------------------------------------

constexpr int kSelWaves = 4;       // (matrix, token) items per workgroup, one wave each

// Sortable 64-bit key of (logit, expert): the float64 bits mapped to an unsigned
// order, the low 10 mantissa bits replaced by 1023 - expert.  Larger key = larger
// logit, equal logits to the lower expert.  Logits closer than 2^-42 relative order
// by index, far inside the near-tie window the routing is checked with.
__device__ inline unsigned long long sel_key(double z, int e) {
    unsigned long long b = __builtin_bit_cast(unsigned long long, z);
    b = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
    return (b & ~0x3FFull) | (unsigned long long)(1023 - e);
}

__device__ inline unsigned long long dpp_u64(unsigned long long v, int ctrl) {
    const int lo = (int)(v & 0xFFFFFFFFull), hi = (int)(v >> 32);
    int mlo, mhi;
    switch (ctrl) {
        case 0: mlo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, true);
                mhi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, true); break;     // quad xor 1
        case 1: mlo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, true);
                mhi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, true); break;     // quad xor 2
        case 2: mlo = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xF, 0xF, true);
                mhi = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xF, 0xF, true); break;    // half-row mirror
        case 3: mlo = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xF, 0xF, true);
                mhi = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xF, 0xF, true); break;    // row mirror
        case 4: mlo = __builtin_amdgcn_update_dpp(0, lo, 0x142, 0xA, 0xF, false);
                mhi = __builtin_amdgcn_update_dpp(0, hi, 0x142, 0xA, 0xF, false); break;   // row broadcast 15
        default: mlo = __builtin_amdgcn_update_dpp(0, lo, 0x143, 0xC, 0xF, false);
                 mhi = __builtin_amdgcn_update_dpp(0, hi, 0x143, 0xC, 0xF, false); break;  // row broadcast 31
    }
    return ((unsigned long long)(unsigned)mhi << 32) | (unsigned)mlo;
}

// Wave maximum of a key; every lane gets it (lane 63 holds it after the broadcasts).
__device__ inline unsigned long long wave_max_key(unsigned long long k) {
#pragma unroll
    for (int st = 0; st < 6; ++st) {
        const unsigned long long o = dpp_u64(k, st);
        k = o > k ? o : k;
    }
    const int lo = __builtin_amdgcn_readlane((int)(k & 0xFFFFFFFFull), 63);
    const int hi = __builtin_amdgcn_readlane((int)(k >> 32), 63);
    return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
}

// Wave maximum of a 32-bit value (every lane gets it).
__device__ inline unsigned wave_max_u32(unsigned k) {
    k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0xB1, 0xF, 0xF, true));    // quad xor 1
    k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0x4E, 0xF, 0xF, true));    // quad xor 2
    k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0x141, 0xF, 0xF, true));   // half-row mirror
    k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0x140, 0xF, 0xF, true));   // row mirror
    k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0x142, 0xA, 0xF, false));  // row broadcast 15
    k = max(k, (unsigned)__builtin_amdgcn_update_dpp(0, (int)k, 0x143, 0xC, 0xF, false));  // row broadcast 31
    return (unsigned)__builtin_amdgcn_readlane((int)k, 63);
}

// Selection for (matrix m, token t) by one wave from the logits zv[i] of experts
// lane + 64 i (E <= 64 * PER; entries past E are ignored).  Pick j is kept by lane j
// (top_k <= 16) and the lanes holding picks write them together at the end.
template <int PER>
__device__ inline void select_item(const RouterArgs &a, int m, int t, int lane, double (&zv)[PER]) {
    // this lane's candidates, sorted by key (descending) once
    unsigned long long key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        if (e >= a.E) zv[i] = -DBL_MAX;
        key[i] = e < a.E ? sel_key(zv[i], e) : 0ull;
    }
#pragma unroll
    for (int i = 1; i < PER; ++i)
#pragma unroll
        for (int j = i; j > 0; --j)
            if (key[j] > key[j - 1]) {
                const unsigned long long tk = key[j];
                key[j] = key[j - 1];
                key[j - 1] = tk;
                const double tz = zv[j];
                zv[j] = zv[j - 1];
                zv[j - 1] = tz;
            }
    // softmax denominator: exp in fp32 of z - max, summed over the wave.  The max is the
    // largest head of the sorted lists; the sum runs over the lists (a permutation of the
    // lane's logits: the same fp32 terms in a fixed order per lane).
    double mx = zv[0];
#pragma unroll
    for (int st = 0; st < 4; ++st) mx = fmax(mx, dpp_f64(mx, st));
    mx = fmax(fmax(readlane_f64(mx, 0), readlane_f64(mx, 16)), fmax(readlane_f64(mx, 32), readlane_f64(mx, 48)));
    float fs = 0.f;
    if (m == 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (key[i]) fs += __expf((float)(zv[i] - mx));
#pragma unroll
        for (int st = 0; st < 4; ++st) fs += __builtin_bit_cast(float, dpp_i(__builtin_bit_cast(int, fs), st));
        fs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), 0)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), 16)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), 32)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), 48));
    }
    int my_e = 0;
    double my_z = 0.0;
    // k rounds on the upper 32 bits of the list heads: their wave maximum and the lanes
    // holding it.  If one lane holds it, that lane's head is the largest remaining key
    // (every other head, and so every other key, is already smaller in those bits), the
    // same pick as a round on the whole key; it pops its list.
    bool exact = true;
    {
        unsigned h32[PER];
        int he[PER];
        double hz[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            h32[i] = (unsigned)(key[i] >> 32);
            he[i] = 1023 - (int)(key[i] & 0x3FFull);
            hz[i] = zv[i];
        }
        for (int j = 0; j < a.top_k; ++j) {
            const unsigned best = wave_max_u32(h32[0]);
            const unsigned long long at = __builtin_amdgcn_ballot_w64(h32[0] == best);
            if (__builtin_popcountll(at) != 1) {
                exact = false;
                break;
            }
            const int owner = __builtin_ctzll(at);
            const int be = __builtin_amdgcn_readlane(he[0], owner);
            const double bz = readlane_f64(hz[0], owner);
            if (lane == j) {
                my_e = be;
                my_z = bz;
            }
            if (lane == owner) {
#pragma unroll
                for (int i = 0; i + 1 < PER; ++i) {
                    h32[i] = h32[i + 1];
                    he[i] = he[i + 1];
                    hz[i] = hz[i + 1];
                }
                h32[PER - 1] = 0u;
            }
        }
    }
    // two lanes' heads equal in the upper bits (equal or nearly equal logits): k rounds
    // on the whole keys, each the wave's largest head key
    if (!exact) {
        for (int j = 0; j < a.top_k; ++j) {
            const unsigned long long best = wave_max_key(key[0]);
            const int be = 1023 - (int)(best & 0x3FFull);
            const int owner = be & 63;
            const double bz = readlane_f64(zv[0], owner);
            if (lane == j) {
                my_e = be;
                my_z = bz;
            }
            if (lane == owner) {
#pragma unroll
                for (int i = 0; i + 1 < PER; ++i) {
                    key[i] = key[i + 1];
                    zv[i] = zv[i + 1];
                }
                key[PER - 1] = 0ull;
            }
        }
    }
    if (lane < a.top_k) {
        const size_t o = (size_t)t * a.top_k + lane;
        if (m == 0) {
            const float g = __expf((float)(my_z - mx)) / fs;
            a.ids[o] = my_e;
            a.gate[o] = g;
            if (a.ids_host) {
                a.ids_host[o] = my_e;
                a.gate_host[o] = g;
            }
        } else if (a.spec_ids_host) {
            a.spec_ids_host[((size_t)(m - 1) * a.n_tok + t) * a.top_k + lane] = my_e;
        }
    }
}

template <int PER>
__global__ __launch_bounds__(64 * kSelWaves) void k_router_select(RouterArgs a, int n_items) {
    const int item = blockIdx.x * kSelWaves + (threadIdx.x >> 6);
    if (item >= n_items) return;
    const int m = item / a.n_tok;
    const int t = item - m * a.n_tok;
    const int lane = threadIdx.x & 63;
    const double *zr = a.z + ((size_t)m * a.n_tok + t) * a.E;
    double zv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) zv[i] = lane + 64 * i < a.E ? zr[lane + 64 * i] : 0.0;
    select_item<PER>(a, m, t, lane, zv);
}

// The logits of (matrix m, token t) from the exchange array, read until no sentinel is
// left (false: wait_us passed first); the entries then hold the sentinel again.
template <int PER>
__device__ inline bool take_exchanged(const RouterArgs &a, int m, int t, int lane, double (&zv)[PER]) {
    unsigned long long *zr = reinterpret_cast<unsigned long long *>(a.zx + ((size_t)m * a.n_tok + t) * a.E);
    bool done = false;
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime(), ticks = 100ull * a.wait_us;
    while (a.wait_us != 0) {
        bool have = true;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + 64 * i;
            if (e < a.E) {
                const unsigned long long b = __hip_atomic_load(zr + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                zv[i] = __builtin_bit_cast(double, b);
                have = have && b != kExchangeSentinel;
            }
        }
        if (__builtin_amdgcn_ballot_w64(!have) == 0) {
            done = true;
            break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) break;
        __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        if (e < a.E) __hip_atomic_store(zr + e, kExchangeSentinel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return done;
}

// One launch for up to kFusedRouterTokens tokens (E a multiple of kRowsPerWg, so a
// workgroup's rows belong to one matrix; tokens <= kRowsPerWg, one selecting wave each).
template <int TB, int PER>
__global__ __launch_bounds__(256) void k_router_fused(RouterArgs a, int n_mats) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    logits_row<TB, true>(a, a.zx, n_mats, blockIdx.x * kRowsPerWg + wave, 0, a.n_tok, lane);
    write_xq(a, 0, a.n_tok, blockIdx.x, gridDim.x);  // after the row loads went out
    const int per_mat = a.E / kRowsPerWg;
    const int m = blockIdx.x / per_mat;
    if ((int)blockIdx.x != (m + 1) * per_mat - 1 || wave >= a.n_tok) return;
    double zv[PER];
    if (take_exchanged<PER>(a, m, wave, lane, zv)) {
        select_item<PER>(a, m, wave, lane, zv);
        return;
    }
    // the wait ended without every logit: no results (the host's read of them fails), the
    // token's device ids marked invalid (kernels that read them on the device skip them),
    // and the host flag raised
    if (lane == 0) {
        if (m == 0)
            for (int j = 0; j < a.top_k; ++j) a.ids[(size_t)wave * a.top_k + j] = -1;
        __hip_atomic_store(a.timed_out, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// --- weighted combine ------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_combine(const float *x, const float *y, const float *gate, float *out,
                                                 int n_tok, int t0, int H, int top_k, int has_shared, int residual) {
    const int t = t0 + blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= H) return;
    float4 yv[16];
    float g[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j < top_k) {
            g[j] = gate[t * top_k + j];
            yv[j] = *reinterpret_cast<const float4 *>(y + ((size_t)t * top_k + j) * H + c);
        }
    }
    const float4 sv = has_shared ? *reinterpret_cast<const float4 *>(y + ((size_t)n_tok * top_k + t) * H + c)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 xv = residual ? *reinterpret_cast<const float4 *>(x + (size_t)t * H + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (j < top_k) {
            acc.x = fmaf(g[j], yv[j].x, acc.x);
            acc.y = fmaf(g[j], yv[j].y, acc.y);
            acc.z = fmaf(g[j], yv[j].z, acc.z);
            acc.w = fmaf(g[j], yv[j].w, acc.w);
        }
    }
    acc.x += sv.x;
    acc.y += sv.y;
    acc.z += sv.z;
    acc.w += sv.w;
    acc.x += xv.x;
    acc.y += xv.y;
    acc.z += xv.z;
    acc.w += xv.w;
    *reinterpret_cast<float4 *>(out + (size_t)t * H + c) = acc;
}

// --- fill -------------------------------------------------------------------------------------

constexpr int kMapSetMax = 120;
struct MapSet {
    int n;
    int32_t key[kMapSetMax];
    int32_t val[kMapSetMax];
};

__global__ __launch_bounds__(128) void k_map_set(int32_t *map, MapSet s) {
    if ((int)threadIdx.x < s.n) map[s.key[threadIdx.x]] = s.val[threadIdx.x];
}

__global__ __launch_bounds__(256) void k_fill_u32(unsigned *p, unsigned v, unsigned n) {
    const unsigned i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// One thread waits until `ticks` of the 100 MHz real-time counter have passed (a bounded
// wait: it always ends).
__global__ __launch_bounds__(64) void k_delay(unsigned long long ticks) {
    if (threadIdx.x != 0) return;
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

}  // namespace

hipError_t launch_delay_us(unsigned us, hipStream_t stream) {
    if (us == 0) return hipSuccess;
    const unsigned long long ticks = 100ull * (us > 100000u ? 100000u : us);   // at most 0.1 s
    return launch(k_delay, dim3(1), dim3(64), stream, nullptr, nullptr, ticks);
}

hipError_t launch_map_set(int32_t *map, const int32_t *keys, const int32_t *vals, int n, hipStream_t stream) {
    for (int i0 = 0; i0 < n; i0 += kMapSetMax) {
        MapSet s;
        s.n = n - i0 < kMapSetMax ? n - i0 : kMapSetMax;
        for (int i = 0; i < s.n; ++i) {
            s.key[i] = keys[i0 + i];
            s.val[i] = vals[i0 + i];
        }
        const hipError_t e = launch(k_map_set, dim3(1), dim3(128), stream, nullptr, nullptr, map, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_fill_u32(unsigned *p, unsigned v, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    if (n > 0xFFFFFFFFull) return hipErrorInvalidValue;
    return launch(k_fill_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), stream, nullptr, nullptr, p, v, (unsigned)n);
}

hipError_t launch_router(const RouterArgs &a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
    if (a.n_tok <= 0) return hipSuccess;
    const int n_mats = 1 + a.n_spec;
    const dim3 block(kRowsPerWg * 64);
    const int gx = (n_mats * a.E + kRowsPerWg - 1) / kRowsPerWg;
    const int per = (a.E + 63) / 64;
    if (a.zx && a.timed_out && a.n_tok <= kFusedRouterTokens && a.n_tok <= kRowsPerWg && a.E % kRowsPerWg == 0) {
        if (a.n_tok == 1) {
            if (per <= 1) return launch(k_router_fused<1, 1>, dim3(gx), block, stream, e0, e1, a, n_mats);
            if (per <= 2) return launch(k_router_fused<1, 2>, dim3(gx), block, stream, e0, e1, a, n_mats);
            if (per <= 4) return launch(k_router_fused<1, 4>, dim3(gx), block, stream, e0, e1, a, n_mats);
            if (per <= 8) return launch(k_router_fused<1, 8>, dim3(gx), block, stream, e0, e1, a, n_mats);
            return launch(k_router_fused<1, 16>, dim3(gx), block, stream, e0, e1, a, n_mats);
        }
        if (per <= 1) return launch(k_router_fused<4, 1>, dim3(gx), block, stream, e0, e1, a, n_mats);
        if (per <= 2) return launch(k_router_fused<4, 2>, dim3(gx), block, stream, e0, e1, a, n_mats);
        if (per <= 4) return launch(k_router_fused<4, 4>, dim3(gx), block, stream, e0, e1, a, n_mats);
        if (per <= 8) return launch(k_router_fused<4, 8>, dim3(gx), block, stream, e0, e1, a, n_mats);
        return launch(k_router_fused<4, 16>, dim3(gx), block, stream, e0, e1, a, n_mats);
    }
    hipError_t e;
    if (a.n_tok == 1) e = launch(k_router_logits<1>, dim3(gx, 1), block, stream, e0, nullptr, a, n_mats);
    else if (a.n_tok <= 4) e = launch(k_router_logits<4>, dim3(gx, 1), block, stream, e0, nullptr, a, n_mats);
    else if (a.n_tok <= 8) e = launch(k_router_logits<8>, dim3(gx, 1), block, stream, e0, nullptr, a, n_mats);
    else if (a.n_tok <= 32 || a.H % 32 != 0)
        e = launch(k_router_logits<32>, dim3(gx, (a.n_tok + 31) / 32), block, stream, e0, nullptr, a, n_mats);
    else
        e = launch(k_router_logits_mfma, dim3((a.n_tok + kMfmaTok - 1) / kMfmaTok, n_mats * ((a.E + 63) / 64)), block,
                   stream, e0, nullptr, a, n_mats);
    if (e != hipSuccess) return e;
    const int n_items = n_mats * a.n_tok;
    const dim3 sg((n_items + kSelWaves - 1) / kSelWaves), sb(64 * kSelWaves);
    if (per <= 1) return launch(k_router_select<1>, sg, sb, stream, nullptr, e1, a, n_items);
    if (per <= 2) return launch(k_router_select<2>, sg, sb, stream, nullptr, e1, a, n_items);
    if (per <= 4) return launch(k_router_select<4>, sg, sb, stream, nullptr, e1, a, n_items);
    if (per <= 8) return launch(k_router_select<8>, sg, sb, stream, nullptr, e1, a, n_items);
    return launch(k_router_select<16>, sg, sb, stream, nullptr, e1, a, n_items);
}

hipError_t launch_combine(const float *x, const float *y, const float *gate, float *out, int n_tok, int t0, int nt,
                          int H, int top_k, int has_shared, int residual, hipStream_t stream) {
    if (nt <= 0) return hipSuccess;
    const dim3 grid((H / 4 + 255) / 256, nt);
    return launch(k_combine, grid, dim3(256), stream, nullptr, nullptr, x, y, gate, out, n_tok, t0, H, top_k, has_shared,
                  residual);
}

}  // namespace moe
