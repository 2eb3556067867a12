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
// Tiles: a workgroup of 4 waves computes 128 pairs x 64 outputs of one expert
// (per matrix); each wave a 64 x 32 block, two MFMA tiles stacked.  The
// reduction steps 64 elements at a time (two int4 scale groups) through a
// double-buffered LDS: while the MFMAs read one buffer the other receives the
// next step (activation rows gathered by pair id; 4-bit weights dequantised to
// fp16 with the block scale folded in; e2m1 x E4M3 is exact in fp16, int4 x
// fp16 scale rounds once), and the global loads of the step after that are in
// flight.  One barrier per step.  Activations are fp16: the same MFMA rate as
// bf16 on gfx950, and with bf16 activations the layer output misses the
// stated 2e-3 max|ref| tolerance.
#include "kernels.hpp"

namespace moe {
namespace {

typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));
typedef f16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32;

constexpr int BM = kPrefillRows, BN = 64, BK = 64;
static_assert(BM == 128, "thread mapping assumes 128-row items");
constexpr int LDA = BK + 8;      // fp16 row stride in LDS (144 bytes): spreads rows over banks

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
    __shared__ __align__(16) f16 As[2][BM * LDA];
    __shared__ __align__(16) f16 Bs[2][NMAT * BN * LDA];
    const int item = blockIdx.x / a.n_tiles;
    const int tile = blockIdx.x - item * a.n_tiles;
    const PrefillItem it = a.items[item];
    const uint8_t *blk = reinterpret_cast<const uint8_t *>(it.block);
    const int n0 = tile * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const size_t row_bytes = (FMT == Q_F32) ? (size_t)a.K * 4 : (size_t)a.K / 2;
    const size_t nib_bytes = row_bytes * a.N;
    const int n_groups = a.K / 32;            // scale groups
    const int n_steps = a.K / BK;

    // A: thread -> rows ar and ar + 64, 8 halfs at 8 * (tid % 4) and 32 further
    const int ar = tid >> 2, ap = (tid & 3) * 8;
    const f16 *a_src[2];
    bool a_ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = ar + 64 * h;
        a_ok[h] = r < it.rows;
        size_t a_row = 0;
        if (a_ok[h]) {
            const int p = a.pairs[it.pair_off + r];
            a_row = a.a_by_token ? (size_t)(p < a.nk ? p / a.top_k : p - a.nk) : (size_t)p;
        }
        a_src[h] = a.a + a_row * a.K + ap;
    }
    // B: thread -> (matrix m, row n, 16-element half of the group)
    const int bm = tid / 128, bn = (tid & 127) >> 1, bh = tid & 1;
    const bool b_ok = bm < NMAT && (n0 + bn) < a.N;
    const uint8_t *b_mat = blk + (bm == 0 ? a.mat_off0 : a.mat_off1);

    // step g covers reduction elements 64g .. 64g+63: thread B half bh takes scale group 2g+bh
    uint4 a_reg[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) a_reg[h][0] = a_reg[h][1] = make_uint4(0, 0, 0, 0);
    uint4 b_codes = make_uint4(0, 0, 0, 0);
    float4 b_f32[8];
    u32 b_scale = 0;
    auto load = [&](int g) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if (a_ok[h]) {
                a_reg[h][0] = *reinterpret_cast<const uint4 *>(a_src[h] + g * BK);
                a_reg[h][1] = *reinterpret_cast<const uint4 *>(a_src[h] + g * BK + 32);
            }
        if (b_ok) {
            const size_t r = (size_t)(n0 + bn);
            const int sg = 2 * g + bh;
            if constexpr (FMT == Q_F32) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    b_f32[i] = *reinterpret_cast<const float4 *>(b_mat + r * row_bytes + (size_t)(sg * 32 + 4 * i) * 4);
            } else {
                b_codes = *reinterpret_cast<const uint4 *>(b_mat + r * row_bytes + (size_t)sg * 16);
                b_scale = *reinterpret_cast<const unsigned short *>(b_mat + nib_bytes + (r * n_groups + sg) * 2);
            }
        }
    };
    // registers -> LDS buffer `buf`
    auto store = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            *reinterpret_cast<uint4 *>(&As[buf][(ar + 64 * h) * LDA + ap]) = a_reg[h][0];
            *reinterpret_cast<uint4 *>(&As[buf][(ar + 64 * h) * LDA + ap + 32]) = a_reg[h][1];
        }
        if (bm < NMAT) {
            f16 w[32];
            if (b_ok) {
                if constexpr (FMT == Q_F32) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        w[4 * i] = (f16)b_f32[i].x;
                        w[4 * i + 1] = (f16)b_f32[i].y;
                        w[4 * i + 2] = (f16)b_f32[i].z;
                        w[4 * i + 3] = (f16)b_f32[i].w;
                    }
                } else if constexpr (FMT == Q_INT4) {
                    dequant16<FMT>(make_uint2(b_codes.x, b_codes.y), b_scale, 0, &w[0]);
                    dequant16<FMT>(make_uint2(b_codes.z, b_codes.w), b_scale, 0, &w[16]);
                } else {   // e2m1: one E4M3 scale byte per 16 elements
                    dequant16<FMT>(make_uint2(b_codes.x, b_codes.y), b_scale & 0xFFu, 0, &w[0]);
                    dequant16<FMT>(make_uint2(b_codes.z, b_codes.w), b_scale >> 8, 1, &w[16]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 32; ++i) w[i] = (f16)0.0f;
            }
            uint4 *dst = reinterpret_cast<uint4 *>(&Bs[buf][(bm * BN + bn) * LDA + bh * 32]);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = __builtin_bit_cast(uint4, *reinterpret_cast<half8 *>(&w[8 * q]));
        }
    };

    float16v acc[NMAT][2];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;

    load(0);
    store(0);
    if (n_steps > 1) load(1);
    __syncthreads();
    for (int g = 0; g < n_steps; ++g) {
        const int cur = g & 1;
        // 4 x (32x32x16) MFMA per row tile and matrix per 64-element step, from buffer cur
#pragma unroll
        for (int kh = 0; kh < BK / 16; ++kh) {
            half8 av[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                av[t] = *reinterpret_cast<const half8 *>(
                    &As[cur][(64 * wm + 32 * t + (lane & 31)) * LDA + 16 * kh + 8 * (lane >> 5)]);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
                const half8 bv = *reinterpret_cast<const half8 *>(
                    &Bs[cur][(m * BN + 32 * wn + (lane & 31)) * LDA + 16 * kh + 8 * (lane >> 5)]);
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    acc[m][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[t], bv, acc[m][t], 0, 0, 0);
            }
        }
        // step g+1 into the other buffer (its last readers were before the previous barrier),
        // then the loads of step g+2
        if (g + 1 < n_steps) {
            store(cur ^ 1);
            if (g + 2 < n_steps) load(g + 2);
        }
        __syncthreads();
    }

    // epilogue: register i of lane l is row (i/4)*8 + (l/32)*4 + i%4, column l%32 of a 32x32 tile
    const int col = n0 + 32 * wn + (lane & 31);
    if (col >= a.N) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 64 * wm + 32 * t + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
            if (r >= it.rows) continue;
            const int p = a.pairs[it.pair_off + r];
            if constexpr (NMAT == 2) {
                const float gv = acc[0][t][i];
                const float h = gv / (1.0f + __expf(-gv)) * acc[1][t][i];
                static_cast<f16 *>(a.out)[(size_t)p * a.N + col] = (f16)h;
            } else {
                static_cast<float *>(a.out)[(size_t)p * a.N + col] = acc[0][t][i];
            }
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
