// Router for gfx950: float64 logits, softmax and top-k.
//
// What it computes (explainer page, "The model that should not fit": a small
// router in front of the experts reads each token and picks a few; SGLang
// page, "What does Paged Experts actually do?": top_k of E experts per token):
//   z[t,e] = sum_i W[e,i] x[t,i]       float32 operands, float64 accumulation
//   p[t,:] = softmax(z[t,:])           float64, stored as float32
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
// (2) select: one workgroup per (matrix, token): softmax and k rounds of a
// workgroup arg-max built from DPP moves and lane reads.
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
    const float *w = (m == 0 ? a.w0 : a.w1) + (size_t)e * a.H;
    double v[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) v[t] = 0.0;
    // four 16-byte loads of the row per lane in flight, then the token FMAs
    for (int h0 = lane * 4; h0 < a.H; h0 += 1024) {
        float4 wv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int h = h0 + 256 * u;
            wv[u] = h < a.H ? *reinterpret_cast<const float4 *>(w + h) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < nt) {
                const float *xr = a.x + (size_t)(t0 + t) * a.H;
                float4 xv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int h = h0 + 256 * u;
                    xv[u] = h < a.H ? *reinterpret_cast<const float4 *>(xr + h) : make_float4(0.f, 0.f, 0.f, 0.f);
                }
                double s = v[t];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
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

__device__ inline double wave_max(double v) {
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) v = fmax(v, __shfl_xor(v, mask));
    return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) v += __shfl_xor(v, mask);
    return v;
}

constexpr int kSelThreads = 256;
constexpr int kPerThread = 4;      // E <= 1024

__global__ __launch_bounds__(kSelThreads) void k_router_select(RouterArgs a) {
    const int m = blockIdx.x / a.n_tok;
    const int t = blockIdx.x - m * a.n_tok;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const double *zr = a.z + ((size_t)m * a.n_tok + t) * a.E;
    __shared__ double s_z[2][4];
    __shared__ int s_e[2][4];
    __shared__ double s_red[4];

    double zv[kPerThread];
    double mx = -DBL_MAX;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int e = threadIdx.x + kSelThreads * i;
        zv[i] = e < a.E ? zr[e] : -DBL_MAX;
        mx = fmax(mx, zv[i]);
    }
    mx = wave_max(mx);
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    mx = fmax(fmax(s_red[0], s_red[1]), fmax(s_red[2], s_red[3]));
    double sum = 0.0;
    if (m == 0) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i)
            if ((int)threadIdx.x + kSelThreads * i < a.E) sum += exp(zv[i] - mx);
        sum = wave_sum(sum);
        __syncthreads();
        if (lane == 0) s_red[wave] = sum;
        __syncthreads();
        sum = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    }
    unsigned taken = 0;
    for (int j = 0; j < a.top_k; ++j) {
        double bz = -DBL_MAX;
        int be = INT_MAX;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int e = threadIdx.x + kSelThreads * i;
            if (e < a.E && !(taken & (1u << i)) && better(zv[i], e, bz, be)) {
                bz = zv[i];
                be = e;
            }
        }
        wave_argmax(bz, be);
        const int buf = j & 1;
        if (lane == 0) {
            s_z[buf][wave] = bz;
            s_e[buf][wave] = be;
        }
        __syncthreads();
        bz = s_z[buf][0];
        be = s_e[buf][0];
#pragma unroll
        for (int w = 1; w < 4; ++w)
            if (better(s_z[buf][w], s_e[buf][w], bz, be)) {
                bz = s_z[buf][w];
                be = s_e[buf][w];
            }
        if (be >= 0 && be < a.E && (be % kSelThreads) == (int)threadIdx.x) taken |= 1u << (be / kSelThreads);
        if (threadIdx.x == 0) {
            const size_t o = (size_t)t * a.top_k + j;
            if (m == 0) {
                const float g = (float)(exp(bz - mx) / sum);
                a.ids[o] = be;
                a.gate[o] = g;
                if (a.ids_host) {
                    a.ids_host[o] = be;
                    a.gate_host[o] = g;
                }
            } else if (a.spec_ids_host) {
                a.spec_ids_host[o] = be;
            }
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
    const int n_mats = a.w1 ? 2 : 1;
    const dim3 block(kRowsPerWg * 64);
    const int gx = (n_mats * a.E + kRowsPerWg - 1) / kRowsPerWg;
    if (a.n_tok == 1) {
        hipExtLaunchKernelGGL(k_router_logits<1>, dim3(gx, 1), block, 0, stream, e0, nullptr, 0, a, n_mats);
    } else if (a.n_tok <= 8) {
        hipExtLaunchKernelGGL(k_router_logits<8>, dim3(gx, 1), block, 0, stream, e0, nullptr, 0, a, n_mats);
    } else {
        hipExtLaunchKernelGGL(k_router_logits<32>, dim3(gx, (a.n_tok + 31) / 32), block, 0, stream, e0, nullptr, 0, a,
                              n_mats);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipExtLaunchKernelGGL(k_router_select, dim3(n_mats * a.n_tok), dim3(kSelThreads), 0, stream, nullptr, e1, 0, a);
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
