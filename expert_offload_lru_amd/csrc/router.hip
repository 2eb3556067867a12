// Router for gfx950: float64 logits, softmax and top-k.
//
// What it computes (explainer page, "The model that should not fit": a small
// router in front of the experts reads each token and picks a few; SGLang
// page, "What does Paged Experts actually do?": top_k of E experts per token):
//   z[t,e] = sum_i W[e,i] x[t,i]       float32 operands, float64 accumulation
//   p[t,:] = softmax(z[t,:])           exp in fp32, normalised in float64, stored as float32
//   ids[t,:] = the top_k experts by z, descending, equal z to the lower index
//   gate[t,j] = p[t, ids[t,j]]          (not renormalised over the picks)
// With a second matrix (the next layer's router) the same launches also pick
// that layer's top_k on the same input, for speculative prefetch (NVMe page,
// "Workflow": the next layer's router run on the current layer's input).
//
// Two launches, no device-wide fence: across the eight XCDs of the chip a
// release fence writes back a whole L2, which costs more than a kernel
// boundary.  (1) logits: one wave per (matrix, expert row) and block of up to
// 32 tokens, streaming the row with 16-byte loads; the per-token sums are
// reduced with a halving butterfly (each exchange halves the values a lane
// holds).  The same launch writes the fp16 copy of x the expert GEMV reads.
// (2) select: one wave per (matrix, token): softmax and k rounds of a wave
// arg-max built from DPP moves and lane reads (no barriers, no LDS).
#include <cfloat>
#include <climits>

#include "kernels.hpp"

namespace moe {
namespace {

typedef _Float16 f16;
constexpr int kRowsPerWg = 4;

template <int TB>
__global__ __launch_bounds__(256) void k_router_logits(RouterArgs a, int n_mats) {
    constexpr int LOG = (TB == 1) ? 0 : (TB == 8 ? 3 : 5);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int gr = blockIdx.x * kRowsPerWg + wave;
    const int t0 = blockIdx.y * TB;
    const int nt = min(TB, a.n_tok - t0);

    // fp16 activation copy, a slice per workgroup: 8 elements per item
    if (a.xq) {
        const int n8 = a.H / 8;
        const int per = (n8 + gridDim.x - 1) / gridDim.x;
        const int b0 = blockIdx.x * per, b1 = min(b0 + per, n8);
        for (int item = threadIdx.x; item < nt * (b1 - b0); item += blockDim.x) {
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

    if (gr >= n_mats * a.E) return;
    const int m = gr / a.E;
    const int e = gr - m * a.E;
    const float *w = (m == 0 ? a.w0 : (m == 1 ? a.w1 : a.w2)) + (size_t)e * a.H;
    double v[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) v[t] = 0.0;
    // up to 8 16-byte loads of the row per lane (H <= 2048) in flight at once, then the
    // token FMAs; longer rows take further rounds
    for (int h0 = lane * 4; h0 < a.H; h0 += 2048) {
        float4 wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int h = h0 + 256 * u;
            wv[u] = h < a.H ? *reinterpret_cast<const float4 *>(w + h) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < nt) {
                const float *xr = a.x + (size_t)(t0 + t) * a.H;
                float4 xv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int h = h0 + 256 * u;
                    xv[u] = h < a.H ? *reinterpret_cast<const float4 *>(xr + h) : make_float4(0.f, 0.f, 0.f, 0.f);
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
    // values selected by lane bit M; LOG steps leave one value per lane
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
    double s = v[0];
#pragma unroll
    for (int mask = 32 >> LOG; mask >= 1; mask >>= 1) s += __shfl_xor(s, mask);
    const int tok = (lane >> (6 - LOG)) & (TB - 1);
    const bool writer = (lane & ((64 >> LOG) - 1)) == 0;
    if (writer && tok < nt) a.z[((size_t)m * a.n_tok + t0 + tok) * a.E + e] = s;
}

// --- workgroup arg-max: largest z, equal z to the lower index -------------------------------

__device__ inline bool better(double za, int ea, double zb, int eb) { return za > zb || (za == zb && ea < eb); }

__device__ inline int dpp_i(int v, int ctrl) {
    switch (ctrl) {
        case 0: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);    // quad xor 1
        case 1: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);    // quad xor 2
        case 2: return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true);   // half-row mirror
        default: return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, true); // row mirror
    }
}

// Every lane ends with the wave's best (z, e).
__device__ inline void wave_argmax(double &z, int &e) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const long long zb = __builtin_bit_cast(long long, z);
        const int lo = dpp_i((int)(zb & 0xFFFFFFFF), st);
        const int hi = dpp_i((int)(zb >> 32), st);
        const double oz = __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
        const int oe = dpp_i(e, st);
        if (better(oz, oe, z, e)) {
            z = oz;
            e = oe;
        }
    }
    // one candidate per row of 16 lanes: compare the four rows through lane reads
    double bz = z;
    int be = e;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const long long zb = __builtin_bit_cast(long long, z);
        const int lo = __builtin_amdgcn_readlane((int)(zb & 0xFFFFFFFF), 16 * r);
        const int hi = __builtin_amdgcn_readlane((int)(zb >> 32), 16 * r);
        const double rz = __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
        const int re = __builtin_amdgcn_readlane(e, 16 * r);
        if (r == 0 || better(rz, re, bz, be)) {
            bz = rz;
            be = re;
        }
    }
    z = bz;
    e = be;
}

// Every lane ends with the wave's combined value (fmax or sum) via DPP within rows
// of 16 lanes, then lane reads of the four rows.
template <bool MAX>
__device__ inline double wave_reduce(double v) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const long long b = __builtin_bit_cast(long long, v);
        const int lo = dpp_i((int)(b & 0xFFFFFFFF), st);
        const int hi = dpp_i((int)(b >> 32), st);
        const double o = __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
        v = MAX ? fmax(v, o) : v + o;
    }
    double r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const long long b = __builtin_bit_cast(long long, v);
        const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFF), 16 * q);
        const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 16 * q);
        r[q] = __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
    }
    return MAX ? fmax(fmax(r[0], r[1]), fmax(r[2], r[3])) : (r[0] + r[1]) + (r[2] + r[3]);
}

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

__device__ inline unsigned long long dpp_u64(unsigned long long v, int ctrl, int row_mask) {
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
    (void)row_mask;
    return ((unsigned long long)(unsigned)mhi << 32) | (unsigned)mlo;
}

// Wave maximum of a key; every lane gets it (lane 63 holds it after the broadcasts).
__device__ inline unsigned long long wave_max_key(unsigned long long k) {
#pragma unroll
    for (int st = 0; st < 6; ++st) {
        const unsigned long long o = dpp_u64(k, st, 0);
        k = o > k ? o : k;
    }
    const int lo = __builtin_amdgcn_readlane((int)(k & 0xFFFFFFFFull), 63);
    const int hi = __builtin_amdgcn_readlane((int)(k >> 32), 63);
    return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
}

// One wave per (matrix, token), PER candidates per lane (E <= 64 * PER).
template <int PER>
__global__ __launch_bounds__(64 * kSelWaves) void k_router_select(RouterArgs a, int n_items) {
    const int item = blockIdx.x * kSelWaves + (threadIdx.x >> 6);
    if (item >= n_items) return;
    const int lane = threadIdx.x & 63;
    const int m = item / a.n_tok;
    const int t = item - m * a.n_tok;
    const double *zr = a.z + ((size_t)m * a.n_tok + t) * a.E;

    // this lane's candidates, sorted by key (descending) once
    unsigned long long key[PER];
    double zv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        zv[i] = e < a.E ? zr[e] : -DBL_MAX;
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
    // softmax denominator: exp in fp32 of z - max, summed over the wave
    double mx = zv[0];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const long long b = __builtin_bit_cast(long long, mx);
        const int lo = dpp_i((int)(b & 0xFFFFFFFF), st), hi = dpp_i((int)(b >> 32), st);
        mx = fmax(mx, __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo));
    }
    {
        double r = mx;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const long long b = __builtin_bit_cast(long long, mx);
            const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFF), 16 * q);
            const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 16 * q);
            r = fmax(r, __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo));
        }
        mx = r;
    }
    float fs = 0.f;
    if (m == 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (lane + 64 * i < a.E) fs += __expf((float)(zr[lane + 64 * i] - mx));
#pragma unroll
        for (int st = 0; st < 4; ++st) fs += __builtin_bit_cast(float, dpp_i(__builtin_bit_cast(int, fs), st));
        fs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), 0)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), 16)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), 32)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), 48));
    }
    // k rounds: the wave's largest head key; its lane pops its list
    for (int j = 0; j < a.top_k; ++j) {
        const unsigned long long best = wave_max_key(key[0]);
        const int be = 1023 - (int)(best & 0x3FFull);
        const bool mine = (be & 63) == lane;
        const double bz_l = zv[0];
        if (mine) {
#pragma unroll
            for (int i = 0; i + 1 < PER; ++i) {
                key[i] = key[i + 1];
                zv[i] = zv[i + 1];
            }
            key[PER - 1] = 0ull;
        }
        if (m == 0) {
            const long long zb = __builtin_bit_cast(long long, bz_l);
            const int zlo = __builtin_amdgcn_readlane((int)(zb & 0xFFFFFFFF), be & 63);
            const int zhi = __builtin_amdgcn_readlane((int)(zb >> 32), be & 63);
            const double bz = __builtin_bit_cast(double, ((long long)zhi << 32) | (unsigned int)zlo);
            if (lane == 0) {
                const size_t o = (size_t)t * a.top_k + j;
                const float g = __expf((float)(bz - mx)) / fs;
                a.ids[o] = be;
                a.gate[o] = g;
                if (a.ids_host) {
                    a.ids_host[o] = be;
                    a.gate_host[o] = g;
                }
            }
        } else if (lane == 0 && a.spec_ids_host) {
            a.spec_ids_host[((size_t)(m - 1) * a.n_tok + t) * a.top_k + j] = be;
        }
    }
}

// --- weighted combine ------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_combine(const float *x, const float *y, const float *gate, float *out,
                                                 int n_tok, int H, int top_k, int has_shared, int residual) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
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

}  // namespace

hipError_t launch_router(const RouterArgs &a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
    if (a.n_tok <= 0) return hipSuccess;
    const int n_mats = a.w1 ? (a.w2 ? 3 : 2) : 1;
    const dim3 block(kRowsPerWg * 64);
    const int gx = (n_mats * a.E + kRowsPerWg - 1) / kRowsPerWg;
    if (a.n_tok == 1) {
        if (e0 || e1) hipExtLaunchKernelGGL(k_router_logits<1>, dim3(gx, 1), block, 0, stream, e0, nullptr, 0, a, n_mats);
        else hipLaunchKernelGGL(k_router_logits<1>, dim3(gx, 1), block, 0, stream, a, n_mats);
    } else if (a.n_tok <= 8) {
        if (e0 || e1) hipExtLaunchKernelGGL(k_router_logits<8>, dim3(gx, 1), block, 0, stream, e0, nullptr, 0, a, n_mats);
        else hipLaunchKernelGGL(k_router_logits<8>, dim3(gx, 1), block, 0, stream, a, n_mats);
    } else {
        const dim3 g(gx, (a.n_tok + 31) / 32);
        if (e0 || e1) hipExtLaunchKernelGGL(k_router_logits<32>, g, block, 0, stream, e0, nullptr, 0, a, n_mats);
        else hipLaunchKernelGGL(k_router_logits<32>, g, block, 0, stream, a, n_mats);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_items = n_mats * a.n_tok;
    const dim3 sg((n_items + kSelWaves - 1) / kSelWaves), sb(64 * kSelWaves);
    const int per = (a.E + 63) / 64;
#define MOE_SEL(P)                                                                                      \
    do {                                                                                                \
        if (e1) hipExtLaunchKernelGGL(k_router_select<P>, sg, sb, 0, stream, nullptr, e1, 0, a, n_items); \
        else hipLaunchKernelGGL(k_router_select<P>, sg, sb, 0, stream, a, n_items);                     \
    } while (0)
    if (per <= 1) MOE_SEL(1);
    else if (per <= 2) MOE_SEL(2);
    else if (per <= 4) MOE_SEL(4);
    else if (per <= 8) MOE_SEL(8);
    else MOE_SEL(16);
#undef MOE_SEL
    return hipGetLastError();
}

hipError_t launch_combine(const float *x, const float *y, const float *gate, float *out, int n_tok, int H, int top_k,
                          int has_shared, int residual, hipStream_t stream) {
    if (n_tok <= 0) return hipSuccess;
    const dim3 grid((H / 4 + 255) / 256, n_tok);
    hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, stream, x, y, gate, out, n_tok, H, top_k, has_shared, residual);
    return hipGetLastError();
}

}  // namespace moe
