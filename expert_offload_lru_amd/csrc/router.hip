// Fused router for gfx950: logits, softmax and top-k in one launch.
//
// What it computes (explainer page, "The model that should not fit": a small
// router in front of the experts reads each token and picks a few; SGLang
// page, "What does Paged Experts actually do?": top_k of E experts per token):
//   z[t,e] = sum_i W[e,i] x[t,i]       float32 operands, float64 accumulation
//   p[t,:] = softmax(z[t,:])           float64, stored as float32
//   ids[t,:] = the top_k experts by z, descending, equal z to the lower index
//   gate[t,j] = p[t, ids[t,j]]          (not renormalised over the picks)
// With a second matrix (the next layer's router) the same launch also picks
// that layer's top_k on the same input, for speculative prefetch (NVMe page,
// "Workflow": the next layer's router run on the current layer's input).
//
// Shape: one wave per (matrix, expert row) and block of up to 32 tokens,
// streaming the row with 16-byte loads; the per-token partial sums are
// reduced with a halving butterfly (each exchange step halves the values a
// lane holds), so a wave finishes 32 token sums in 32 exchanges.  The
// workgroup that finishes last for a token block (a ticket counter; no
// waiting) then runs softmax and a wave-wide arg-max k times per token.
#include <cfloat>
#include <climits>

#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kRowsPerWg = 4;

template <int TB>
__global__ __launch_bounds__(256) void k_router(RouterArgs a, int n_mats) {
    constexpr int LOG = (TB == 1) ? 0 : (TB == 8 ? 3 : 5);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int gr = blockIdx.x * kRowsPerWg + wave;
    const int t0 = blockIdx.y * TB;
    const int nt = min(TB, a.n_tok - t0);

    if (gr < n_mats * a.E) {
        const int m = gr / a.E;
        const int e = gr - m * a.E;
        const float *w = (m == 0 ? a.w0 : a.w1) + (size_t)e * a.H;
        double v[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) v[t] = 0.0;
        for (int h = lane * 4; h < a.H; h += 256) {
            const float4 wv = *reinterpret_cast<const float4 *>(w + h);
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                if (t < nt) {
                    const float4 xv = *reinterpret_cast<const float4 *>(a.x + (size_t)(t0 + t) * a.H + h);
                    double s = v[t];
                    s = fma((double)wv.x, (double)xv.x, s);
                    s = fma((double)wv.y, (double)xv.y, s);
                    s = fma((double)wv.z, (double)xv.z, s);
                    s = fma((double)wv.w, (double)xv.w, s);
                    v[t] = s;
                }
            }
        }
        // halving butterfly: after the step with mask M a lane keeps the half of
        // its values selected by lane bit M; LOG steps leave one value per lane
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

    // ticket: the last workgroup of this token block does the selection
    __shared__ int last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned ticket = atomicAdd(&a.counters[blockIdx.y], 1u);
        last = (ticket == gridDim.x - 1);
    }
    __syncthreads();
    if (!last) return;
    __threadfence();

    for (int item = wave; item < n_mats * nt; item += 4) {
        const int m = item / nt;
        const int t = t0 + (item - m * nt);
        const double *zr = a.z + ((size_t)m * a.n_tok + t) * a.E;
        double zv[16];
        double mx = -DBL_MAX;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = lane + 64 * i;
            zv[i] = e < a.E ? zr[e] : -DBL_MAX;
            mx = fmax(mx, zv[i]);
        }
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1) mx = fmax(mx, __shfl_xor(mx, mask));
        double sum = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (lane + 64 * i < a.E) sum += exp(zv[i] - mx);
#pragma unroll
        for (int mask = 32; mask >= 1; mask >>= 1) sum += __shfl_xor(sum, mask);
        unsigned taken = 0;
        for (int j = 0; j < a.top_k; ++j) {
            double bz = -DBL_MAX;
            int be = INT_MAX;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int e = lane + 64 * i;
                if (e < a.E && !(taken & (1u << i)) && (zv[i] > bz || (zv[i] == bz && e < be))) {
                    bz = zv[i];
                    be = e;
                }
            }
#pragma unroll
            for (int mask = 32; mask >= 1; mask >>= 1) {
                const double oz = __shfl_xor(bz, mask);
                const int oe = __shfl_xor(be, mask);
                if (oz > bz || (oz == bz && oe < be)) {
                    bz = oz;
                    be = oe;
                }
            }
            if ((be & 63) == lane) taken |= 1u << (be >> 6);
            if (lane == 0) {
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
    if (threadIdx.x == 0) a.counters[blockIdx.y] = 0u;
}

}  // namespace

hipError_t launch_router(const RouterArgs &a, hipStream_t stream) {
    if (a.n_tok <= 0) return hipSuccess;
    const int n_mats = a.w1 ? 2 : 1;
    const dim3 block(kRowsPerWg * 64);
    const int gx = (n_mats * a.E + kRowsPerWg - 1) / kRowsPerWg;
    if (a.n_tok == 1) {
        hipLaunchKernelGGL(k_router<1>, dim3(gx, 1), block, 0, stream, a, n_mats);
    } else if (a.n_tok <= 8) {
        hipLaunchKernelGGL(k_router<8>, dim3(gx, 1), block, 0, stream, a, n_mats);
    } else {
        hipLaunchKernelGGL(k_router<32>, dim3(gx, (a.n_tok + 31) / 32), block, 0, stream, a, n_mats);
    }
    return hipGetLastError();
}

// --- weighted combine ------------------------------------------------------------------------
// out[t] = (residual ? x[t] : 0) + y[t], y[t] = sum_j gate[t,j] Y[t*k+j] (+ Y[nk+t]), summed in
// rank order j so the result does not depend on which launch produced which row of Y.

namespace {
__global__ __launch_bounds__(256) void k_combine(const float *x, const float *y, const float *gate, float *out,
                                                 int n_tok, int H, int top_k, int has_shared, int residual) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (c >= H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < top_k; ++j) {
        const float g = gate[t * top_k + j];
        const float4 v = *reinterpret_cast<const float4 *>(y + ((size_t)t * top_k + j) * H + c);
        acc.x = fmaf(g, v.x, acc.x);
        acc.y = fmaf(g, v.y, acc.y);
        acc.z = fmaf(g, v.z, acc.z);
        acc.w = fmaf(g, v.w, acc.w);
    }
    if (has_shared) {
        const float4 v = *reinterpret_cast<const float4 *>(y + ((size_t)n_tok * top_k + t) * H + c);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    if (residual) {
        const float4 xv = *reinterpret_cast<const float4 *>(x + (size_t)t * H + c);
        acc.x += xv.x;
        acc.y += xv.y;
        acc.z += xv.z;
        acc.w += xv.w;
    }
    *reinterpret_cast<float4 *>(out + (size_t)t * H + c) = acc;
}
}  // namespace

hipError_t launch_combine(const float *x, const float *y, const float *gate, float *out, int n_tok, int H, int top_k,
                          int has_shared, int residual, hipStream_t stream) {
    if (n_tok <= 0) return hipSuccess;
    const dim3 grid((H / 4 + 255) / 256, n_tok);
    hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, stream, x, y, gate, out, n_tok, H, top_k, has_shared, residual);
    return hipGetLastError();
}

}  // namespace moe
