// Prefill expert FFN on gfx950: grouped MFMA GEMM over the experts of a batch.
//
// What it computes (explainer page, "The rules in the code": calls of more than
// 32 tokens take the large-batch path; 95 GiB page, "Prefill": the layer's
// experts are loaded into an arena in a batch and computed there; NVMe page,
// "Workflow": the whole prompt goes through a layer at once, experts read in
// batches of 32): for every expert e of a batch and the (token, pick) pairs
// routed to it,
//   gate/up kernel: h[p] = silu(X_p Wg^T) * (X_p Wu^T)       (a row per pair)
//   down kernel:    Y[p] = h[p] Wd^T
// With tens to hundreds of tokens per expert this is a dense contraction:
// the work runs on the MFMA matrix cores (v_mfma_f32_32x32x16_f16).
//
// Tiles: a workgroup of 4 waves computes 64 tokens x 64 outputs of one expert
// (per matrix), stepping the reduction 32 elements at a time (one int4 scale
// group).  Activation rows are gathered by pair id into LDS; 4-bit weights are
// dequantised into LDS as fp16 with the block scale folded in (e2m1 x E4M3 is
// exact in fp16; int4 x fp16 scale rounds once to fp16).  Global loads of the
// next step are issued before the MFMAs of the current one.  Activations are
// fp16: the same MFMA rate as bf16 on gfx950, and with bf16 activations the
// layer output misses the stated 2e-3 max|ref| tolerance.
#include "kernels.hpp"

namespace moe {
namespace {

typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));
typedef f16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32;

constexpr int BM = 64, BN = 64, BK = 32;
constexpr int LDA = BK + 8;      // fp16 row stride in LDS (80 bytes): spreads rows over banks

__device__ inline h2 as_h2(u32 v) { return __builtin_bit_cast(h2, v); }

// 16 consecutive weights (8 bytes of codes) of row n, elements k0..k0+15 of the group, to fp16.
template <int FMT>
__device__ inline void dequant16(uint2 codes, u32 sbits, int half_idx, f16 *out) {
    if constexpr (FMT == Q_INT4) {
        const f16 s = __builtin_bit_cast(f16, (unsigned short)(sbits & 0xFFFFu));
        const h2 ss = {s, s};
        const h2 bias = {(f16)1032.0f, (f16)1032.0f};
        const u32 wd[2] = {codes.x, codes.y};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const u32 v = wd[d];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // codes m and m+4 of this dword into fp16 (1024 + q), minus 1032, times s
                const h2 q = as_h2(((v >> (4 * m)) & 0x000F000Fu) | 0x64006400u);
                const h2 w = (q - bias) * ss;
                out[8 * d + m] = w.x;
                out[8 * d + m + 4] = w.y;
            }
        }
    } else {
        // e2m1: two groups of 16 per 32 elements; this half uses scale byte half_idx
        const float sf = __builtin_amdgcn_cvt_f32_fp8((int)sbits, 0);
        const f16 s = (f16)sf;
        const h2 ss = {s, s};
        const u32 wd[2] = {codes.x, codes.y};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[d], 1.0f, 0) * ss;
            const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[d], 1.0f, 1) * ss;
            const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[d], 1.0f, 2) * ss;
            const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wd[d], 1.0f, 3) * ss;
            out[8 * d + 0] = p0.x;
            out[8 * d + 1] = p0.y;
            out[8 * d + 2] = p1.x;
            out[8 * d + 3] = p1.y;
            out[8 * d + 4] = p2.x;
            out[8 * d + 5] = p2.y;
            out[8 * d + 6] = p3.x;
            out[8 * d + 7] = p3.y;
        }
        (void)half_idx;
    }
}

template <int FMT, int NMAT>
__global__ __launch_bounds__(256) void k_prefill_gemm(PrefillGemmArgs a) {
    __shared__ __align__(16) f16 As[BM * LDA];
    __shared__ __align__(16) f16 Bs[NMAT * BN * LDA];
    const int item = blockIdx.x / a.n_tiles;
    const int tile = blockIdx.x - item * a.n_tiles;
    const PrefillItem it = a.items[item];
    const uint8_t *blk = reinterpret_cast<const uint8_t *>(it.block);
    const int n0 = tile * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const size_t row_bytes = (FMT == Q_F32) ? (size_t)a.K * 4 : (size_t)a.K / 2;
    const size_t nib_bytes = row_bytes * a.N;
    const int n_groups = a.K / 32;

    // A: thread -> (row r = tid / 4, 8 halfs at 8 * (tid % 4))
    const int ar = tid >> 2, ap = (tid & 3) * 8;
    const bool a_ok = ar < it.rows;
    size_t a_row = 0;
    if (a_ok) {
        const int p = a.pairs[it.pair_off + ar];
        a_row = a.a_by_token ? (size_t)(p < a.nk ? p / a.top_k : p - a.nk) : (size_t)p;
    }
    const f16 *a_src = a.a + a_row * a.K + ap;
    // B: thread -> (matrix m, row n, 16-element half of the group)
    const int bm = tid / 128, bn = (tid & 127) >> 1, bh = tid & 1;
    const bool b_ok = bm < NMAT && (n0 + bn) < a.N;
    const uint8_t *b_mat = blk + (bm == 0 ? a.mat_off0 : a.mat_off1);

    uint4 a_reg = make_uint4(0, 0, 0, 0);
    uint2 b_codes = make_uint2(0, 0);
    float4 b_f32[4];
    u32 b_scale = 0;
    auto load = [&](int g) {
        if (a_ok) a_reg = *reinterpret_cast<const uint4 *>(a_src + g * 32);
        if (b_ok) {
            const size_t r = (size_t)(n0 + bn);
            if constexpr (FMT == Q_F32) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    b_f32[i] = *reinterpret_cast<const float4 *>(b_mat + r * row_bytes + (size_t)(g * 32 + bh * 16 + 4 * i) * 4);
            } else {
                b_codes = *reinterpret_cast<const uint2 *>(b_mat + r * row_bytes + (size_t)g * 16 + bh * 8);
                if constexpr (FMT == Q_INT4)
                    b_scale = *reinterpret_cast<const unsigned short *>(b_mat + nib_bytes + (r * n_groups + g) * 2);
                else
                    b_scale = b_mat[nib_bytes + (r * n_groups + g) * 2 + bh];
            }
        }
    };

    float16v acc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;

    load(0);
    for (int g = 0; g < n_groups; ++g) {
        // registers -> LDS
        *reinterpret_cast<uint4 *>(&As[ar * LDA + ap]) = a_reg;
        if (bm < NMAT) {
            f16 w[16];
            if (b_ok) {
                if constexpr (FMT == Q_F32) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        w[4 * i] = (f16)b_f32[i].x;
                        w[4 * i + 1] = (f16)b_f32[i].y;
                        w[4 * i + 2] = (f16)b_f32[i].z;
                        w[4 * i + 3] = (f16)b_f32[i].w;
                    }
                } else {
                    dequant16<FMT>(b_codes, b_scale, bh, w);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) w[i] = (f16)0.0f;
            }
            uint4 *dst = reinterpret_cast<uint4 *>(&Bs[(bm * BN + bn) * LDA + bh * 16]);
            dst[0] = __builtin_bit_cast(uint4, *reinterpret_cast<half8 *>(&w[0]));
            dst[1] = __builtin_bit_cast(uint4, *reinterpret_cast<half8 *>(&w[8]));
        }
        __syncthreads();
        if (g + 1 < n_groups) load(g + 1);
        // 2 x (32x32x16) MFMA per matrix per 32-element step
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const half8 av = *reinterpret_cast<const half8 *>(&As[(32 * wm + (lane & 31)) * LDA + 16 * kh + 8 * (lane >> 5)]);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const half8 bv =
                    *reinterpret_cast<const half8 *>(&Bs[(m * BN + 32 * wn + (lane & 31)) * LDA + 16 * kh + 8 * (lane >> 5)]);
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[m], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // epilogue: register i of lane l is row (i/4)*8 + (l/32)*4 + i%4, column l%32 of the wave's 32x32
    const int col = n0 + 32 * wn + (lane & 31);
    if (col >= a.N) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 32 * wm + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (r >= it.rows) continue;
        const int p = a.pairs[it.pair_off + r];
        if constexpr (NMAT == 2) {
            const float gv = acc[0][i];
            const float h = gv / (1.0f + __expf(-gv)) * acc[1][i];
            static_cast<f16 *>(a.out)[(size_t)p * a.N + col] = (f16)h;
        } else {
            static_cast<float *>(a.out)[(size_t)p * a.N + col] = acc[0][i];
        }
    }
}

}  // namespace

hipError_t launch_prefill_gemm(int quant, int n_mats, const PrefillGemmArgs &a, hipStream_t stream, hipEvent_t e0,
                               hipEvent_t e1) {
    if (a.n_items <= 0) return hipSuccess;
    const dim3 grid(a.n_items * a.n_tiles), block(256);
    if (quant == Q_INT4) return n_mats == 2 ? launch(k_prefill_gemm<Q_INT4, 2>, grid, block, stream, e0, e1, a)
                                            : launch(k_prefill_gemm<Q_INT4, 1>, grid, block, stream, e0, e1, a);
    if (quant == Q_E2M1) return n_mats == 2 ? launch(k_prefill_gemm<Q_E2M1, 2>, grid, block, stream, e0, e1, a)
                                            : launch(k_prefill_gemm<Q_E2M1, 1>, grid, block, stream, e0, e1, a);
    return n_mats == 2 ? launch(k_prefill_gemm<Q_F32, 2>, grid, block, stream, e0, e1, a)
                       : launch(k_prefill_gemm<Q_F32, 1>, grid, block, stream, e0, e1, a);
}

}  // namespace moe
