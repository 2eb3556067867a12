// Slot-indexed dequant-SwiGLU expert GEMV for decode calls (gfx950).
//
// What it computes (SGLang page, "What does Paged Experts actually do?": the
// expert math runs on the GPU over the resident slots; explainer page, "The
// bus problem": an expert is gate, up and down projections; NVMe page,
// "Workflow": a fused 4-bit SwiGLU matrix-vector kernel): for every unit (a
// distinct expert of the wave, read from its cache slot) and every
// (token, pick) pair routed to it,
//   gate/up kernel: h[p][r] = silu(Wg[r] . x_t) * (Wu[r] . x_t),  r < inter
//   down kernel:    Y[p][r] = Wd[r] . h[p],                       r < hidden
// with silu(z) = z / (1 + e^-z).
//
// MI355X design.  The work is bound by HBM bandwidth (one read of each
// picked expert's bytes per call), so the kernel is built around streaming
// the packed weights once with 16-byte loads:
//  * a 64-lane wave covers 64/LPR rows at a time; LPR lanes split a row's
//    16-byte chunks (CPL chunks per lane), so each load instruction reads a
//    contiguous 16*LPR-byte stretch of a row; U rows per lane are loaded up
//    front to keep enough bytes in flight;
//  * activation vectors arrive in fp16, already in the pair order the
//    weight decoding below consumes (written by the router for x and by the
//    gate/up epilogue for h), and go straight from L2 into registers;
//  * 4-bit weights are never expanded to fp32: int4 codes become fp16 by
//    OR-ing them into the mantissa of 1024.0 (two codes per instruction),
//    e2m1 codes go through gfx950's packed fp4 -> fp16 conversion, and the
//    products are accumulated in fp32 by v_dot2 (two MACs per lane-op);
//    the int4 offset (-8) and the 1024 bias are removed once per 32-element
//    group with a constant each lane derives from its vector chunk;
//  * a miss served from the prefetch staging bank is read from there and
//    written into its pool slot by the same loads (no separate copy);
//  * partial sums are reduced across the LPR lanes of a row with DPP moves.
// Every (pair, row) result depends only on the expert's bytes and the
// pair's vector, never on the slot, the unit order or the batch, so outputs
// are bitwise independent of the cache state.
#include "kernels.hpp"

namespace moe {
namespace {

typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32;

constexpr int kWaves = 4;       // waves per workgroup
constexpr int kRsrcWord3 = 0x00020000;   // buffer resource flags of the gfx9 family (raw, untyped)

// Buffer resource over one expert block: loads take the block base and size
// from scalar registers, a per-lane offset from one VGPR, and the per-row part
// of the address as a scalar offset.
__device__ inline __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t *blk, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(blk), (short)0, (int)bytes, kRsrcWord3);
}
__device__ inline uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ inline u32 buf_load2(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return (u32)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// Rows each wave keeps in flight.  Gate/up at one chunk per lane (hidden 2048 for 4-bit
// weights) takes 3: a 768-row expert is then 64 workgroups, so the 8 experts of one
// token are 512 workgroups, two per CU of the 256 (4 rows: 384, one or two per CU).
constexpr int rows_in_flight(int n_mats, int cpl) {
    return (n_mats == 2 && cpl == 1) ? 3 : ((8 / (n_mats * cpl)) >= 4 ? 4 : ((8 / (n_mats * cpl)) >= 2 ? 2 : 1));
}

// The streaming variant for large launches keeps two row blocks in flight per wave; with
// one chunk per lane, two rows per block and two blocks per workgroup (110 VGPRs, 4 waves
// per SIMD) streamed faster at 32 tokens than three rows (140 VGPRs), one row (85 VGPRs,
// 5 waves) with two or four blocks, or two rows with three, four or six blocks (0.42 of
// HBM peak against 0.33 - 0.41), and as fast at 4 tokens.
constexpr int stream_rows_in_flight(int n_mats, int cpl) {
    return (n_mats == 2 && cpl == 1) ? 2 : rows_in_flight(n_mats, cpl);
}

__device__ inline float dpp_add(float v, int ctrl_sel) {
    int src = __builtin_bit_cast(int, v);
    int moved;
    switch (ctrl_sel) {
        case 0: moved = __builtin_amdgcn_update_dpp(0, src, 0xB1, 0xF, 0xF, true); break;   // quad xor 1
        case 1: moved = __builtin_amdgcn_update_dpp(0, src, 0x4E, 0xF, 0xF, true); break;   // quad xor 2
        case 2: moved = __builtin_amdgcn_update_dpp(0, src, 0x141, 0xF, 0xF, true); break;  // half-row mirror
        default: moved = __builtin_amdgcn_update_dpp(0, src, 0x140, 0xF, 0xF, true); break; // row mirror
    }
    return v + __builtin_bit_cast(float, moved);
}

// Sum over aligned segments of LPR lanes; every lane of a segment gets the sum.
template <int LPR>
__device__ inline float seg_sum(float v) {
    if constexpr (LPR >= 2) v = dpp_add(v, 0);
    if constexpr (LPR >= 4) v = dpp_add(v, 1);
    if constexpr (LPR >= 8) v = dpp_add(v, 2);
    if constexpr (LPR >= 16) v = dpp_add(v, 3);
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16);
    if constexpr (LPR >= 64) v += __shfl_xor(v, 32);
    return v;
}

__device__ inline h2 as_h2(u32 v) { return __builtin_bit_cast(h2, v); }

// (a & mask) | (b & ~mask) in one instruction.  The int4 codes' masks and the fp16
// bias 0x6400 share no bits, so this is (a & mask) | bias; written with literal
// operands it takes an AND and an OR (gfx9's three-operand forms take no literals).
__device__ inline u32 bfi(u32 mask, u32 a, u32 b) {
    u32 r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(a), "v"(b));
    return r;
}

// --- one 16-byte chunk of a row times the staged vector chunk -------------------------------
//
// Each adds its product into `acc` with every rounding step written out
// (fmaf), so that no kernel inlining it can contract the arithmetic
// differently: every kernel that computes a (pair, row) value computes it
// bit for bit the same way.

// int4, 32 codes; xp: 16 fp16 pairs ordered per dword as (x0,x4) (x1,x5) (x2,x6) (x3,x7);
// kc = 1032 * sum(even x) + 72 * sum(odd x) of the chunk.
__device__ inline float chunk_int4(float acc, uint4 w, u32 sbits, const uint4 *xp4, float kc) {
    const u32 wd[4] = {w.x, w.y, w.z, w.w};
    float acc_a = 0.f, acc_b = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint4 xv = xp4[d];
        const u32 v = wd[d];
        const u32 v8 = v >> 8;
        acc_a = __builtin_amdgcn_fdot2(as_h2(bfi(0x000F000Fu, v, 0x64006400u)), as_h2(xv.x), acc_a, false);
        acc_b = __builtin_amdgcn_fdot2(as_h2(bfi(0x00F000F0u, v, 0x64006400u)), as_h2(xv.y), acc_b, false);
        acc_a = __builtin_amdgcn_fdot2(as_h2(bfi(0x000F000Fu, v8, 0x64006400u)), as_h2(xv.z), acc_a, false);
        acc_b = __builtin_amdgcn_fdot2(as_h2(bfi(0x00F000F0u, v8, 0x64006400u)), as_h2(xv.w), acc_b, false);
    }
    const float s = (float)__builtin_bit_cast(f16, (unsigned short)(sbits & 0xFFFFu));
    return fmaf(s, fmaf(0.0625f, acc_b, acc_a) - kc, acc);
}

// e2m1, 32 codes in two groups of 16 with E4M3 scales in the two bytes of sbits;
// xp: 16 fp16 pairs in natural order.
__device__ inline float chunk_e2m1(float acc, uint4 w, u32 sbits, const uint4 *xp4) {
    float g0 = 0.f, g1 = 0.f;
    {
        const uint4 x0 = xp4[0], x1 = xp4[1];
        g0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.x, 1.0f, 0), as_h2(x0.x), g0, false);
        g0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.x, 1.0f, 1), as_h2(x0.y), g0, false);
        g0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.x, 1.0f, 2), as_h2(x0.z), g0, false);
        g0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.x, 1.0f, 3), as_h2(x0.w), g0, false);
        g0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.y, 1.0f, 0), as_h2(x1.x), g0, false);
        g0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.y, 1.0f, 1), as_h2(x1.y), g0, false);
        g0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.y, 1.0f, 2), as_h2(x1.z), g0, false);
        g0 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.y, 1.0f, 3), as_h2(x1.w), g0, false);
    }
    {
        const uint4 x2 = xp4[2], x3 = xp4[3];
        g1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.z, 1.0f, 0), as_h2(x2.x), g1, false);
        g1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.z, 1.0f, 1), as_h2(x2.y), g1, false);
        g1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.z, 1.0f, 2), as_h2(x2.z), g1, false);
        g1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.z, 1.0f, 3), as_h2(x2.w), g1, false);
        g1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.w, 1.0f, 0), as_h2(x3.x), g1, false);
        g1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.w, 1.0f, 1), as_h2(x3.y), g1, false);
        g1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.w, 1.0f, 2), as_h2(x3.z), g1, false);
        g1 = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w.w, 1.0f, 3), as_h2(x3.w), g1, false);
    }
    const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sbits, 0);
    const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sbits, 1);
    return fmaf(s1, g1, fmaf(s0, g0, acc));
}

__device__ inline float chunk_f32(float acc, uint4 w, const float4 &x) {
    acc = fmaf(__builtin_bit_cast(float, w.x), x.x, acc);
    acc = fmaf(__builtin_bit_cast(float, w.y), x.y, acc);
    acc = fmaf(__builtin_bit_cast(float, w.z), x.z, acc);
    acc = fmaf(__builtin_bit_cast(float, w.w), x.w, acc);
    return acc;
}

// --- the expert GEMV kernel ------------------------------------------------------------------

__device__ inline int vec_row(const GemvArgs &a, int p) {
    if (!a.vec_by_token) return p;
    return p < a.nk ? p / a.top_k : p - a.nk;
}

// Position of element i of a vector in the fp16 pair order of the format.
template <int FMT>
__device__ inline int pair_pos(int i) {
    if constexpr (FMT == Q_INT4) {
        const int m = i & 7;                        // (0,4) (1,5) (2,6) (3,7) within 8 elements
        return (i & ~7) | ((m & 3) << 1) | (m >> 2);
    } else {
        return i;
    }
}

// Entry i (uniform over the workgroup) of a 16-bit list in the kernel
// arguments, read as the dword that holds it: a scalar load, where a 16-bit
// read would be a vector load the wave has to wait for.
__device__ inline int list_u16(const uint16_t *arr, int i) {
    const uint32_t w = reinterpret_cast<const uint32_t *>(arr)[i >> 1];
    return (i & 1) ? (int)(w >> 16) : (int)(w & 0xFFFFu);
}

// The vector chunks of one pair a lane needs: CPL 16-byte weight chunks, each
// against 32 vector elements (4-bit formats: 64 bytes of fp16) or 4 (fp32).
template <int FMT, int CPL>
struct VecChunks {
    static constexpr int N = (FMT == Q_F32) ? 1 : 4;
    uint4 v[CPL][N];
};

// COH: the vectors were written earlier in the same launch by workgroups that
// may sit on another XCD, whose L2 this one does not see.  The loads then carry
// the agent-scope coherence bit (sc1), as agent-scope atomic loads do, so they
// are served from the point where every XCD's stores meet.
template <int FMT, int CPL, bool COH = false>
__device__ inline void load_vec(VecChunks<FMT, CPL> &x, const GemvArgs &a, int p, int sub, int lpr) {
    const int vrow = vec_row(a, p);
    if constexpr (COH) {
        constexpr int kSc1 = 16;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.vec), (short)0, 0x7FFFFFFF, kRsrcWord3);
        if constexpr (FMT == Q_F32) {
            const int base = vrow * a.cols * 4;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                x.v[i][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, base + (sub + lpr * i) * 16,
                                                                                             0, kSc1));
        } else {
            const int base = vrow * a.cols * 2;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    x.v[i][d] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, base + ((sub + lpr * i) * 4 + d) * 16, 0, kSc1));
        }
        return;
    }
    if constexpr (FMT == Q_F32) {
        const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const float *>(a.vec) + (size_t)vrow * a.cols);
#pragma unroll
        for (int i = 0; i < CPL; ++i) x.v[i][0] = src[sub + lpr * i];
    } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const f16 *>(a.vec) + (size_t)vrow * a.cols);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int d = 0; d < 4; ++d) x.v[i][d] = src[(sub + lpr * i) * 4 + d];
    }
}

// A fill served from the staging bank: the rows this lane loaded are written to
// the fill's pool slot on the way (copy-through).
template <int FMT, int LPR, int CPL, int NMAT, int U>
__device__ __forceinline__ void copy_rows(const GemvArgs &a, uint8_t *cpy, int row0, int sub, size_t row_bytes,
                                          size_t nib_bytes, const uint4 (&wq)[NMAT][U][CPL],
                                          const u32 (&ws)[NMAT][U][CPL]) {
    constexpr int RPW = 64 / LPR;
    constexpr int NC = LPR * CPL;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const size_t moff = (m == 0 ? a.mat_off0 : a.mat_off1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = row0 + u * RPW;
            if (r < a.rows) {
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = sub + LPR * i;
                    *reinterpret_cast<uint4 *>(cpy + moff + (size_t)r * row_bytes + (size_t)c * 16) = wq[m][u][i];
                    if constexpr (FMT != Q_F32)
                        *reinterpret_cast<unsigned short *>(cpy + moff + nib_bytes + ((size_t)r * NC + c) * 2) =
                            (unsigned short)ws[m][u][i];
                }
            }
        }
    }
}

// Every (token, pick) pair p0 .. p1-1 of a unit against the rows this lane holds
// (row0 + u*RPW): dot products, lane reduction, SwiGLU or plain store.  xnext
// holds the first pair's vector chunks on entry; the next pair's load during
// this one's math, and with `again` the first pair's again at the end (for the
// lane's next block of rows).
template <int FMT, int LPR, int CPL, int NMAT, int U, bool COH = false, typename PairAt>
__device__ __forceinline__ void gemv_pairs(const GemvArgs &a, PairAt pair_at, int p0, int p1, int sub, int row0,
                                           const uint4 (&wq)[NMAT][U][CPL], const u32 (&ws)[NMAT][U][CPL],
                                           VecChunks<FMT, CPL> &xnext, bool again) {
    constexpr int RPW = 64 / LPR;
    for (int pp = p0; pp < p1; ++pp) {
        const int p = pair_at(pp);
        const VecChunks<FMT, CPL> xv = xnext;
        if (pp + 1 < p1) load_vec<FMT, CPL>(xnext, a, pair_at(pp + 1), sub, LPR);
        else if (again) load_vec<FMT, CPL>(xnext, a, pair_at(p0), sub, LPR);
        float acc[NMAT][U];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u) acc[m][u] = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            if constexpr (FMT == Q_F32) {
                const float4 x4 = __builtin_bit_cast(float4, xv.v[i][0]);
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int u = 0; u < U; ++u) acc[m][u] = chunk_f32(acc[m][u], wq[m][u][i], x4);
            } else if constexpr (FMT == Q_INT4) {
                // 1032 * sum(even elements) + 72 * sum(odd elements) of the chunk
                const h2 ce = {(f16)1032.0f, (f16)1032.0f}, co = {(f16)72.0f, (f16)72.0f};
                float kc = 0.f;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    kc = __builtin_amdgcn_fdot2(as_h2(xv.v[i][d].x), ce, kc, false);
                    kc = __builtin_amdgcn_fdot2(as_h2(xv.v[i][d].y), co, kc, false);
                    kc = __builtin_amdgcn_fdot2(as_h2(xv.v[i][d].z), ce, kc, false);
                    kc = __builtin_amdgcn_fdot2(as_h2(xv.v[i][d].w), co, kc, false);
                }
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int u = 0; u < U; ++u) acc[m][u] = chunk_int4(acc[m][u], wq[m][u][i], ws[m][u][i], xv.v[i], kc);
            } else {
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int u = 0; u < U; ++u) acc[m][u] = chunk_e2m1(acc[m][u], wq[m][u][i], ws[m][u][i], xv.v[i]);
            }
        }
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int u = 0; u < U; ++u) acc[m][u] = seg_sum<LPR>(acc[m][u]);
        if (sub == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = row0 + u * RPW;
                if (r < a.rows) {
                    if constexpr (NMAT == 2) {
                        const float g = acc[0][u];
                        const float h = g / (1.0f + __expf(-g)) * acc[1][u];
                        if constexpr (COH) {
                            // read later in this launch by other workgroups: store at the
                            // agent's coherence point (an agent-scope store carries sc1)
                            if constexpr (FMT == Q_F32)
                                __hip_atomic_store(static_cast<float *>(a.out) + (size_t)p * a.rows + r, h,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            else
                                __hip_atomic_store(static_cast<unsigned short *>(a.out) + (size_t)p * a.rows +
                                                       pair_pos<FMT>(r),
                                                   __builtin_bit_cast(unsigned short, (f16)h), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                        } else if constexpr (FMT == Q_F32) {
                            static_cast<float *>(a.out)[(size_t)p * a.rows + r] = h;
                        } else {
                            static_cast<f16 *>(a.out)[(size_t)p * a.rows + pair_pos<FMT>(r)] = (f16)h;
                        }
                    } else {
                        static_cast<float *>(a.out)[(size_t)p * a.rows + r] = acc[0][u];
                    }
                }
            }
        }
    }
}

// EXACT: the rows tile the matrix exactly (no partial tile), so every load of a
// lane shares one offset register and the row block goes in a scalar offset.
// One workgroup's tile `tile` of a unit read from `src` (pool slot, -1 shared expert,
// <= -2 staging slot), its pairs p0 .. p1-1 given by pair_at, copied on the way to `cpy`
// if not null.
template <int FMT, int LPR, int CPL, int NMAT, bool EXACT, bool COH, typename PairAt>
__device__ __forceinline__ void gemv_unit_tile(const GemvArgs &a, int tile, int src, uint8_t *cpy, int p0, int p1,
                                               PairAt pair_at) {
    constexpr int U = rows_in_flight(NMAT, CPL);
    constexpr int RPW = 64 / LPR;
    constexpr int NC = LPR * CPL;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int seg = lane / LPR;
    const int sub = lane - seg * LPR;
    const uint8_t *blk = src >= 0 ? a.bank + (size_t)src * a.block_bytes
                                  : (src == -1 ? a.shared_w : a.staging + (size_t)(-2 - src) * a.block_bytes);
    const int row0 = tile * (kWaves * RPW * U) + wave * (RPW * U) + seg;
    const size_t row_bytes = (FMT == Q_F32) ? (size_t)a.cols * 4 : (size_t)a.cols / 2;
    const size_t nib_bytes = row_bytes * a.rows;

    // 0. the first pair's vector chunks (L2-resident) go out ahead of the weights
    VecChunks<FMT, CPL> xnext;
    if (p0 < p1) load_vec<FMT, CPL>(xnext, a, pair_at(p0), sub, LPR);

    // 1. every weight load of this lane (NMAT matrices x U rows x CPL chunks); rows past
    //    the end re-read the last row (always in bounds) and are never stored
    uint4 wq[NMAT][U][CPL];
    u32 ws[NMAT][U][CPL];
    if constexpr (EXACT) {
        const __amdgpu_buffer_rsrc_t rs = block_rsrc(blk, a.block_bytes);
        const int wrow = __builtin_amdgcn_readfirstlane(tile * (kWaves * RPW * U) + wave * (RPW * U));
        const int vo_w = seg * (int)row_bytes + sub * 16;
        const int vo_s = (seg * NC + sub) * 2;
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const int moff = (int)(m == 0 ? a.mat_off0 : a.mat_off1);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int rb = wrow + u * RPW;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    wq[m][u][i] = buf_load16(rs, vo_w, moff + rb * (int)row_bytes + LPR * 16 * i);
                    if constexpr (FMT != Q_F32)
                        ws[m][u][i] = buf_load2(rs, vo_s, moff + (int)nib_bytes + (rb * NC + LPR * i) * 2);
                    else
                        ws[m][u][i] = 0u;
                }
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const size_t moff = (m == 0 ? a.mat_off0 : a.mat_off1);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = row0 + u * RPW;
                const int rr = r < a.rows ? r : a.rows - 1;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = sub + LPR * i;
                    wq[m][u][i] = *reinterpret_cast<const uint4 *>(blk + moff + (size_t)rr * row_bytes + (size_t)c * 16);
                    if constexpr (FMT != Q_F32)
                        ws[m][u][i] = *reinterpret_cast<const unsigned short *>(blk + moff + nib_bytes +
                                                                                ((size_t)rr * NC + c) * 2);
                    else
                        ws[m][u][i] = 0u;
                }
            }
        }
    }
    // 2. a fill served from the staging bank is written to its pool slot on the way
    if (cpy) copy_rows<FMT, LPR, CPL, NMAT, U>(a, cpy, row0, sub, row_bytes, nib_bytes, wq, ws);
    // 3. every (token, pick) pair of the unit
    gemv_pairs<FMT, LPR, CPL, NMAT, U, COH>(a, pair_at, p0, p1, sub, row0, wq, ws, xnext, false);
}

// One workgroup's tile of a launch list (bid = unit * tiles_per_unit + tile).  COH: h is
// read later in the same launch (the fused decode kernel).
template <int FMT, int LPR, int CPL, int NMAT, typename UL, bool EXACT, bool COH>
__device__ __forceinline__ void gemv_tile(const GemvArgs &a, const UL &ul, int bid) {
    // the unit is uniform over the workgroup: keep it (and the list reads it indexes) scalar
    const int unit = __builtin_amdgcn_readfirstlane(bid / a.tiles_per_unit);
    const int tile = bid - unit * a.tiles_per_unit;
    uint8_t *cpy = ul.copy_to[unit] >= 0 ? a.copy_bank + (size_t)ul.copy_to[unit] * a.block_bytes : nullptr;
    gemv_unit_tile<FMT, LPR, CPL, NMAT, EXACT, COH>(a, tile, ul.src[unit], cpy, list_u16(ul.pbeg, unit),
                                                    list_u16(ul.pbeg, unit + 1),
                                                    [&](int pp) { return list_u16(ul.pair, pp); });
}

template <int FMT, int LPR, int CPL, int NMAT, typename UL, bool EXACT>
__global__ __launch_bounds__(256) void k_expert_gemv(GemvArgs a, UL ul) {
    gemv_tile<FMT, LPR, CPL, NMAT, UL, EXACT, false>(a, ul, blockIdx.x);
}

// The same GEMV for large launches: a workgroup streams BPW consecutive blocks
// of rows of its unit, the loads of block b+1 in flight while block b is
// computed (twice the bytes in flight per workgroup at the same occupancy).
// Rows must tile exactly (BPW blocks per tile).
template <int FMT, int LPR, int CPL, int NMAT, int BPW>
__global__ __launch_bounds__(256) void k_expert_gemv_stream(GemvArgs a, UnitList ul) {
    constexpr int U = stream_rows_in_flight(NMAT, CPL);
    constexpr int RPW = 64 / LPR;
    constexpr int NC = LPR * CPL;
    constexpr int BLK = kWaves * RPW * U;     // rows of one block
    const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x / a.tiles_per_unit);
    const int tile = blockIdx.x - unit * a.tiles_per_unit;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int seg = lane / LPR;
    const int sub = lane - seg * LPR;
    const int src = ul.src[unit];
    const int p0 = list_u16(ul.pbeg, unit), p1 = list_u16(ul.pbeg, unit + 1);
    const uint8_t *blk = src >= 0 ? a.bank + (size_t)src * a.block_bytes
                                  : (src == -1 ? a.shared_w : a.staging + (size_t)(-2 - src) * a.block_bytes);
    uint8_t *cpy = ul.copy_to[unit] >= 0 ? a.copy_bank + (size_t)ul.copy_to[unit] * a.block_bytes : nullptr;
    const size_t row_bytes = (FMT == Q_F32) ? (size_t)a.cols * 4 : (size_t)a.cols / 2;
    const size_t nib_bytes = row_bytes * a.rows;
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(blk, a.block_bytes);
    const int vo_w = seg * (int)row_bytes + sub * 16;
    const int vo_s = (seg * NC + sub) * 2;

    VecChunks<FMT, CPL> xnext;
    if (p0 < p1) load_vec<FMT, CPL>(xnext, a, list_u16(ul.pair, p0), sub, LPR);

    uint4 wq[2][NMAT][U][CPL];
    u32 ws[2][NMAT][U][CPL];
    auto load_block = [&](int buf, int b) {
        const int wrow = __builtin_amdgcn_readfirstlane((tile * BPW + b) * BLK + wave * (RPW * U));
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            const int moff = (int)(m == 0 ? a.mat_off0 : a.mat_off1);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int rb = wrow + u * RPW;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    wq[buf][m][u][i] = buf_load16(rs, vo_w, moff + rb * (int)row_bytes + LPR * 16 * i);
                    if constexpr (FMT != Q_F32)
                        ws[buf][m][u][i] = buf_load2(rs, vo_s, moff + (int)nib_bytes + (rb * NC + LPR * i) * 2);
                    else
                        ws[buf][m][u][i] = 0u;
                }
            }
        }
    };
    load_block(0, 0);
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
        const int cur = b & 1;
        if (b + 1 < BPW) load_block(cur ^ 1, b + 1);
        const int row0 = (tile * BPW + b) * BLK + wave * (RPW * U) + seg;
        if (cpy) copy_rows<FMT, LPR, CPL, NMAT, U>(a, cpy, row0, sub, row_bytes, nib_bytes, wq[cur], ws[cur]);
        gemv_pairs<FMT, LPR, CPL, NMAT, U>(a, [&](int pp) { return list_u16(ul.pair, pp); }, p0, p1, sub, row0,
                                           wq[cur], ws[cur], xnext, b + 1 < BPW);
    }
}

// The units of a one-token call read on the device (a captured decode step, every pick
// resident): unit u < n_routed is the router's pick u at the slot the device copy of the
// slot table gives, unit n_routed the shared expert.  At one token unit u's only pair is
// pair u (the shared expert's is nk = n_routed).  Indexed like a launch list's arrays.
struct PickSrc {
    const int32_t *ids, *map;
    int base, n_routed;
    __device__ int operator[](int u) const { return u < n_routed ? map[base + ids[u]] : -1; }
};
struct NoCopy {
    __device__ int operator[](int) const { return -1; }
};
struct PairIota {};
__device__ inline int list_u16(PairIota, int i) { return i; }
struct PickList {
    static constexpr int kUnits = 16, kPairs = 16;
    int n_units;
    PickSrc src;
    NoCopy copy_to;
    PairIota pbeg, pair;
};

// Down projection of every unit of a wave for RPW output rows, then the
// weighted combine of those rows for every token of the wave.  Wave w of the
// workgroup takes units w*UF .. w*UF+UF-1, then every W*UF-th group after; a
// wave's next group's weights are requested while it computes the current group.
// The first group's weights are requested before `ready()`, which every thread
// of the workgroup calls once: in the fused decode kernel it waits until h is
// complete, so the down weights stream while the gate/up workgroups still run.
// COH: h was written earlier in the same launch.
template <int FMT, int LPR, int CPL, typename UL, bool EXACT, bool COH, int W = kWaves, int UF = 2, typename Ready>
__device__ __forceinline__ void down_tile(const GemvArgs &a, const CombineArgs &cb, const UL &ul, int bid,
                                          Ready ready) {
    constexpr int RPW = 64 / LPR;       // output rows of the workgroup (one per lane segment)
    constexpr int NC = LPR * CPL;
    __shared__ float ys[UL::kPairs][RPW];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int seg = lane / LPR;
    const int sub = lane - seg * LPR;
    const int row = bid * RPW + seg;
    const int rr = row < a.rows ? row : a.rows - 1;
    const size_t row_bytes = (FMT == Q_F32) ? (size_t)a.cols * 4 : (size_t)a.cols / 2;
    const size_t nib_bytes = row_bytes * a.rows;
    const int k = a.top_k;
    const int pt0 = cb.t0 * k;            // first routed pair of the wave
    if (bid == 0 && (int)threadIdx.x < cb.n_upd) cb.map[cb.upd_key[threadIdx.x]] = cb.upd_val[threadIdx.x];

    // two sets of weight registers: a wave's next group of units is requested while it
    // computes the current one, so at large batches every wave keeps two groups in flight
    uint4 wq[2][UF][CPL];
    u32 ws[2][UF][CPL];
    auto load_group = [&](auto B, int u0) {
        constexpr int bb = decltype(B)::value;
#pragma unroll
        for (int f = 0; f < UF; ++f) {
            const int u = u0 + f < ul.n_units ? u0 + f : u0;
            const int src = ul.src[u];
            const uint8_t *blk = src >= 0 ? a.bank + (size_t)src * a.block_bytes
                                          : (src == -1 ? a.shared_w : a.staging + (size_t)(-2 - src) * a.block_bytes);
            if constexpr (EXACT) {
                const __amdgpu_buffer_rsrc_t rs = block_rsrc(blk, a.block_bytes);
                const int rb = bid * RPW;
                const int moff = (int)a.mat_off0;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    wq[bb][f][i] = buf_load16(rs, seg * (int)row_bytes + sub * 16,
                                              moff + rb * (int)row_bytes + LPR * 16 * i);
                    if constexpr (FMT != Q_F32)
                        ws[bb][f][i] = buf_load2(rs, (seg * NC + sub) * 2,
                                                 moff + (int)nib_bytes + (rb * NC + LPR * i) * 2);
                    else
                        ws[bb][f][i] = 0u;
                }
            } else {
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = sub + LPR * i;
                    wq[bb][f][i] = *reinterpret_cast<const uint4 *>(blk + a.mat_off0 + (size_t)rr * row_bytes +
                                                                    (size_t)c * 16);
                    if constexpr (FMT != Q_F32)
                        ws[bb][f][i] = *reinterpret_cast<const unsigned short *>(blk + a.mat_off0 + nib_bytes +
                                                                                  ((size_t)rr * NC + c) * 2);
                    else
                        ws[bb][f][i] = 0u;
                }
            }
        }
    };

    // the units of group u0, from weight set B
    auto compute_group = [&](auto B, int u0) {
        constexpr int bb = decltype(B)::value;
#pragma unroll
        for (int f = 0; f < UF; ++f) {
            const int u = u0 + f;
            if (u >= ul.n_units) break;
            // a fill served from the staging bank: this workgroup's rows go to the pool slot
            if (ul.copy_to[u] >= 0 && row < a.rows) {
                uint8_t *cpy = a.copy_bank + (size_t)ul.copy_to[u] * a.block_bytes + a.mat_off0;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int c = sub + LPR * i;
                    *reinterpret_cast<uint4 *>(cpy + (size_t)row * row_bytes + (size_t)c * 16) = wq[bb][f][i];
                    if constexpr (FMT != Q_F32)
                        *reinterpret_cast<unsigned short *>(cpy + nib_bytes + ((size_t)row * NC + c) * 2) =
                            (unsigned short)ws[bb][f][i];
                }
            }
            const int p0 = list_u16(ul.pbeg, u), p1 = list_u16(ul.pbeg, u + 1);
            for (int pp = p0; pp < p1; ++pp) {
                const int p = list_u16(ul.pair, pp);
                VecChunks<FMT, CPL> xv;
                load_vec<FMT, CPL, COH>(xv, a, p, sub, LPR);
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    if constexpr (FMT == Q_F32) {
                        acc = chunk_f32(acc, wq[bb][f][i], __builtin_bit_cast(float4, xv.v[i][0]));
                    } else if constexpr (FMT == Q_INT4) {
                        const h2 ce = {(f16)1032.0f, (f16)1032.0f}, co = {(f16)72.0f, (f16)72.0f};
                        float kc = 0.f;
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            kc = __builtin_amdgcn_fdot2(as_h2(xv.v[i][d].x), ce, kc, false);
                            kc = __builtin_amdgcn_fdot2(as_h2(xv.v[i][d].y), co, kc, false);
                            kc = __builtin_amdgcn_fdot2(as_h2(xv.v[i][d].z), ce, kc, false);
                            kc = __builtin_amdgcn_fdot2(as_h2(xv.v[i][d].w), co, kc, false);
                        }
                        acc = chunk_int4(acc, wq[bb][f][i], ws[bb][f][i], xv.v[i], kc);
                    } else {
                        acc = chunk_e2m1(acc, wq[bb][f][i], ws[bb][f][i], xv.v[i]);
                    }
                }
                acc = seg_sum<LPR>(acc);
                // pair slot in the wave: routed (t - t0)*k + j, shared nt*k + (t - t0)
                const int lp = p < a.nk ? p - pt0 : cb.nt * k + (p - a.nk - cb.t0);
                if (sub == 0) ys[lp][seg] = acc;
            }
        }
    };

    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    constexpr int step = W * UF;
    int u0 = wave * UF;
    if (u0 < ul.n_units) load_group(B0{}, u0);
    ready();
    while (u0 < ul.n_units) {
        if (u0 + step < ul.n_units) load_group(B1{}, u0 + step);
        compute_group(B0{}, u0);
        u0 += step;
        if (u0 >= ul.n_units) break;
        if (u0 + step < ul.n_units) load_group(B0{}, u0 + step);
        compute_group(B1{}, u0);
        u0 += step;
    }
    __syncthreads();
    // combine, in the order of the separate kernel: sum_j g*Y, then the shared expert, then x
    for (int i = threadIdx.x; i < cb.nt * RPW; i += W * 64) {
        const int t = i / RPW;
        const int r = i - t * RPW;
        const int orow = bid * RPW + r;
        if (orow >= a.rows) continue;
        const int tg = cb.t0 + t;
        float acc = 0.f;
        for (int j = 0; j < k; ++j) acc = fmaf(cb.gate[tg * k + j], ys[t * k + j][r], acc);
        acc += cb.has_shared ? ys[cb.nt * k + t][r] : 0.f;
        acc += cb.x ? cb.x[(size_t)tg * a.rows + orow] : 0.f;
        cb.out[(size_t)tg * a.rows + orow] = acc;
    }
}

template <int FMT, int LPR, int CPL, bool EXACT>
__global__ __launch_bounds__(256) void k_expert_gemv_pre(GemvArgs a, PreArgs pa) {
    const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x / a.tiles_per_unit);
    const int tile = blockIdx.x - unit * a.tiles_per_unit;
    int src = -1, pair = a.nk;                    // the shared expert: pair nk + token 0
    if (unit < pa.n_routed) {
        const int e = pa.ids[unit];
        if (e < 0 || e >= pa.n_experts) return;
        src = pa.map[pa.map_base + e];
        if (src < 0) return;                      // not resident: the host's fill launch computes it
        pair = unit;
    }
    gemv_unit_tile<FMT, LPR, CPL, 2, EXACT, false>(a, tile, src, nullptr, 0, 1, [&](int) { return pair; });
}

// The down + combine launch: 8 waves a workgroup, one unit each at a time, so at one token
// every unit's weights and vector are requested at once.
constexpr int kDownWaves = 8;
template <int FMT, int LPR, int CPL, typename UL, bool EXACT>
__global__ __launch_bounds__(kDownWaves * 64) void k_down_combine(GemvArgs a, CombineArgs cb, UL ul) {
    down_tile<FMT, LPR, CPL, UL, EXACT, false, kDownWaves, 1>(a, cb, ul, blockIdx.x, [] {});
}

// Down + combine of a one-token call, its units read on the device (a captured step, or
// the early launch of an uncaptured one).  Every pick must be in range and resident; if one
// is not, no workgroup writes anything and the launch raises *bad (host memory), if given.
// Workgroup b's share of cb.pf (the rows of the reading workgroups congruent to b mod 8),
// 16 bytes a thread, requested now; the returned value only keeps the load alive.
__device__ inline float request_rows(const CombineArgs &cb, int b, int n_wg) {
    if (!cb.pf || cb.pf_cols % 4 != 0) return 0.f;
    const int r = b & 7;
    const int i = b >> 3, n_i = (n_wg - r + 7) >> 3;           // this workgroup's index in its class
    const int n_rwg = (cb.pf_rows + kRouterRowsPerWg - 1) / kRouterRowsPerWg;
    const int n_j = (n_rwg - r + 7) >> 3;                       // reading workgroups in the class
    const size_t wg_f4 = (size_t)kRouterRowsPerWg * cb.pf_cols / 4;
    const size_t set_f4 = (size_t)n_j * wg_f4;
    float v = 0.f;
    for (size_t o = (size_t)i * blockDim.x + threadIdx.x; o < set_f4; o += (size_t)n_i * blockDim.x) {
        const size_t rwg = (size_t)r + 8 * (o / wg_f4);
        const size_t f4 = rwg * wg_f4 + o % wg_f4;                // within the matrix
        if (f4 * 4 < (size_t)cb.pf_rows * cb.pf_cols) v += reinterpret_cast<const float4 *>(cb.pf)[f4].x;
    }
    return v;
}

template <int FMT, int LPR, int CPL, bool EXACT>
__global__ __launch_bounds__(kDownWaves * 64) void k_down_combine_picks(GemvArgs a, CombineArgs cb, PreArgs pa,
                                                                        int *bad) {
    const float keep = request_rows(cb, blockIdx.x, gridDim.x);
    bool ok = true;
    if ((int)threadIdx.x < pa.n_routed) {
        const int e = pa.ids[threadIdx.x];
        ok = e >= 0 && e < pa.n_experts && pa.map[pa.map_base + e] >= 0;
    }
    if (__syncthreads_or(!ok)) {
        if (bad && blockIdx.x == 0 && threadIdx.x == 0)
            __hip_atomic_store(bad, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        return;
    }
    const PickList ul{pa.n_routed + pa.has_shared, {pa.ids, pa.map, pa.map_base, pa.n_routed}, {}, {}, {}};
    down_tile<FMT, LPR, CPL, PickList, EXACT, false, kDownWaves, 1>(a, cb, ul, blockIdx.x, [] {});
    asm volatile("" ::"v"(keep));
}

// One launch for the whole expert work of a single-list wave: workgroups
// [0, n_gu) are the gate/up tiles, the rest the down + combine tiles.  A
// gate/up workgroup stores its h values at the agent's coherence point and
// waits until they are complete there; then it counts itself in its group
// (bid % kSyncGroups); the workgroup completing a group counts the group at
// the top, and the one completing the last group publishes the launch's epoch
// in every flag copy.  A down workgroup requests its weights, then polls its
// flag copy until the epoch appears, and reads h coherently.  Workgroups are
// dispatched in index order, so every gate/up workgroup is running or done
// before any down workgroup can occupy a compute unit, and gate/up workgroups
// wait for nothing: the wait always ends.  It is still bounded: after
// kSpinLimit polls it raises fs.timed_out (host memory) and goes on, so the
// kernel exits in any case.
constexpr unsigned kSpinLimit = 1u << 21;

__device__ inline void fused_gate_up_done(const FusedSync &fs) {
    const int g = blockIdx.x % kSyncGroups;
    const int n_groups = min(kSyncGroups, fs.n_gu);
    const unsigned n_g = (unsigned)(fs.n_gu / kSyncGroups + (g < fs.n_gu % kSyncGroups ? 1 : 0));
    unsigned *gc = fs.sync + g * kSyncStrideU32;
    unsigned *top = fs.sync + kSyncGroups * kSyncStrideU32;
    unsigned long long *flags = reinterpret_cast<unsigned long long *>(top + kSyncStrideU32);
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != n_g - 1) return;
    __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (unsigned)(n_groups - 1)) return;
    __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int r = 0; r < kSyncFlags; ++r)
        __hip_atomic_store(flags + r * (kSyncStrideU32 / 2), fs.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int GL, int GC, int DL, int DC, bool GX, bool DX>
__global__ __launch_bounds__(256) void k_expert_fused(GemvArgs g, GemvArgs d, CombineArgs cb, UnitListS ulg,
                                                      UnitListS uld, FusedSync fs) {
    if ((int)blockIdx.x < fs.n_gu) {
        gemv_tile<FMT, GL, GC, 2, UnitListS, GX, true>(g, ulg, blockIdx.x);
        // this wave's h stores have completed at the coherence point before the count
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) fused_gate_up_done(fs);
        return;
    }
    down_tile<FMT, DL, DC, UnitListS, DX, true>(d, cb, uld, blockIdx.x - fs.n_gu, [&] {
        if (threadIdx.x == 0) {
            const unsigned long long *flag = reinterpret_cast<const unsigned long long *>(
                                                 fs.sync + (kSyncGroups + 1) * kSyncStrideU32) +
                                             (blockIdx.x % kSyncFlags) * (kSyncStrideU32 / 2);
            unsigned it = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < fs.epoch) {
                if (++it == kSpinLimit) {
                    __hip_atomic_store(fs.timed_out, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __syncthreads();
    });
}

// A list that fits the small capacity is launched with the short kernel arguments.
bool to_small(const UnitList &ul, UnitListS &s) {
    const int np = ul.pbeg[ul.n_units];
    if (ul.n_units > UnitListS::kUnits || np > UnitListS::kPairs) return false;
    s.n_units = ul.n_units;
    for (int u = 0; u < ul.n_units; ++u) {
        s.src[u] = ul.src[u];
        s.copy_to[u] = ul.copy_to[u];
    }
    for (int u = 0; u <= ul.n_units; ++u) s.pbeg[u] = ul.pbeg[u];
    s.pad_ = 0;
    for (int i = 0; i < np; ++i) s.pair[i] = ul.pair[i];
    return true;
}

constexpr int kStreamMinWgs = 1536;   // launches at least this large stream two blocks per workgroup

template <int FMT, int LPR, int CPL, int NMAT>
hipError_t launch_t(const GemvArgs &a, const UnitList &ul, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const dim3 grid(ul.n_units * a.tiles_per_unit), block(kWaves * 64);
    const int blk_rows = kWaves * (64 / LPR) * rows_in_flight(NMAT, CPL);
    const bool exact = a.rows % blk_rows == 0;
    if constexpr (NMAT == 2 && FMT != Q_F32) {
        const int sblk_rows = kWaves * (64 / LPR) * stream_rows_in_flight(NMAT, CPL);
        if (a.rows % (2 * sblk_rows) == 0 && (int)grid.x >= kStreamMinWgs) {
            GemvArgs a2 = a;
            a2.tiles_per_unit = a.rows / (2 * sblk_rows);
            return launch(k_expert_gemv_stream<FMT, LPR, CPL, NMAT, 2>, dim3(ul.n_units * a2.tiles_per_unit), block, s,
                          e0, e1, a2, ul);
        }
    }
    UnitListS small;
    if (to_small(ul, small))
        return exact ? launch(k_expert_gemv<FMT, LPR, CPL, NMAT, UnitListS, true>, grid, block, s, e0, e1, a, small)
                     : launch(k_expert_gemv<FMT, LPR, CPL, NMAT, UnitListS, false>, grid, block, s, e0, e1, a, small);
    return exact ? launch(k_expert_gemv<FMT, LPR, CPL, NMAT, UnitList, true>, grid, block, s, e0, e1, a, ul)
                 : launch(k_expert_gemv<FMT, LPR, CPL, NMAT, UnitList, false>, grid, block, s, e0, e1, a, ul);
}

template <int FMT, int LPR, int CPL>
hipError_t launch_dc(const GemvArgs &a, const CombineArgs &cb, const UnitList &ul, dim3 grid, hipStream_t s,
                     hipEvent_t e0, hipEvent_t e1) {
    const bool exact = a.rows % (64 / LPR) == 0;
    const dim3 block(kDownWaves * 64);
    UnitListS small;
    if (to_small(ul, small))
        return exact ? launch(k_down_combine<FMT, LPR, CPL, UnitListS, true>, grid, block, s, e0, e1, a, cb, small)
                     : launch(k_down_combine<FMT, LPR, CPL, UnitListS, false>, grid, block, s, e0, e1, a, cb, small);
    return exact ? launch(k_down_combine<FMT, LPR, CPL, UnitList, true>, grid, block, s, e0, e1, a, cb, ul)
                 : launch(k_down_combine<FMT, LPR, CPL, UnitList, false>, grid, block, s, e0, e1, a, cb, ul);
}

template <int FMT, int GL, int GC, int DL, int DC>
hipError_t launch_fused_t(const GemvArgs &g, const UnitListS &ulg, const GemvArgs &d, const CombineArgs &cb,
                          const UnitListS &uld, const FusedSync &fs, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const int blk_rows = kWaves * (64 / GL) * rows_in_flight(2, GC);
    const bool gx = g.rows % blk_rows == 0, dx = d.rows % (64 / DL) == 0;
    const int n_dc = (d.rows + 64 / DL - 1) / (64 / DL);
    const dim3 grid(fs.n_gu + n_dc), block(kWaves * 64);
    if (gx && dx)
        return launch(k_expert_fused<FMT, GL, GC, DL, DC, true, true>, grid, block, s, e0, e1, g, d, cb, ulg, uld, fs);
    if (gx)
        return launch(k_expert_fused<FMT, GL, GC, DL, DC, true, false>, grid, block, s, e0, e1, g, d, cb, ulg, uld, fs);
    if (dx)
        return launch(k_expert_fused<FMT, GL, GC, DL, DC, false, true>, grid, block, s, e0, e1, g, d, cb, ulg, uld, fs);
    return launch(k_expert_fused<FMT, GL, GC, DL, DC, false, false>, grid, block, s, e0, e1, g, d, cb, ulg, uld, fs);
}

template <int FMT, int NMAT>
hipError_t launch_fmt(int lpr, int cpl, const GemvArgs &a, const UnitList &ul, hipStream_t s, hipEvent_t e0,
                      hipEvent_t e1) {
#define MOE_CASE(L, C) \
    if (lpr == L && cpl == C) return launch_t<FMT, L, C, NMAT>(a, ul, s, e0, e1);
    MOE_CASE(64, 1) MOE_CASE(64, 2) MOE_CASE(64, 3) MOE_CASE(64, 4)
    MOE_CASE(32, 1) MOE_CASE(32, 2) MOE_CASE(32, 3) MOE_CASE(32, 4)
    MOE_CASE(16, 1) MOE_CASE(16, 2) MOE_CASE(16, 3) MOE_CASE(16, 4)
    MOE_CASE(8, 1) MOE_CASE(8, 2) MOE_CASE(8, 3) MOE_CASE(8, 4)
#undef MOE_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_down_combine(int quant, const GemvArgs &a, const CombineArgs &cb, const UnitList &ul,
                               hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const GemvShape sh = gemv_shape(quant, a.cols, 1);
    if (!sh.ok || ul.n_units <= 0) return hipErrorInvalidValue;
    const dim3 grid((a.rows + 64 / sh.lpr - 1) / (64 / sh.lpr));
#define MOE_DC(F, L, C) \
    if (sh.lpr == L && sh.cpl == C) return launch_dc<F, L, C>(a, cb, ul, grid, s, e0, e1);
#define MOE_DC_FMT(F) \
    MOE_DC(F, 64, 1) MOE_DC(F, 64, 2) MOE_DC(F, 64, 3) MOE_DC(F, 64, 4) \
    MOE_DC(F, 32, 1) MOE_DC(F, 32, 2) MOE_DC(F, 32, 3) MOE_DC(F, 32, 4) \
    MOE_DC(F, 16, 1) MOE_DC(F, 16, 2) MOE_DC(F, 16, 3) MOE_DC(F, 16, 4) \
    MOE_DC(F, 8, 1) MOE_DC(F, 8, 2) MOE_DC(F, 8, 3) MOE_DC(F, 8, 4)
    if (quant == Q_INT4) { MOE_DC_FMT(Q_INT4) }
    else if (quant == Q_E2M1) { MOE_DC_FMT(Q_E2M1) }
    else { MOE_DC_FMT(Q_F32) }
#undef MOE_DC_FMT
#undef MOE_DC
    return hipErrorInvalidValue;
}

template <int FMT, int LPR, int CPL>
hipError_t launch_dcp_t(const GemvArgs &a, const CombineArgs &cb, const PreArgs &pa, int *bad, hipStream_t s,
                        hipEvent_t e0, hipEvent_t e1) {
    const dim3 grid((a.rows + 64 / LPR - 1) / (64 / LPR)), block(kDownWaves * 64);
    if (a.rows % (64 / LPR) == 0)
        return launch(k_down_combine_picks<FMT, LPR, CPL, true>, grid, block, s, e0, e1, a, cb, pa, bad);
    return launch(k_down_combine_picks<FMT, LPR, CPL, false>, grid, block, s, e0, e1, a, cb, pa, bad);
}

hipError_t launch_down_combine_picks(int quant, const GemvArgs &a, const CombineArgs &cb, const PreArgs &pa, int *bad,
                                     hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
    const GemvShape sh = gemv_shape(quant, a.cols, 1);
    if (!sh.ok || pa.n_routed <= 0 || !pa.ids || !pa.map) return hipErrorInvalidValue;
    if (pa.n_routed + pa.has_shared > PickList::kPairs || a.nk != pa.n_routed || cb.nt != 1 || cb.t0 != 0 ||
        pa.n_routed > kDownWaves * 64)
        return hipErrorInvalidValue;
#define MOE_DCP(F, L, C) \
    if (sh.lpr == L && sh.cpl == C) return launch_dcp_t<F, L, C>(a, cb, pa, bad, stream, e0, e1);
#define MOE_DCP_FMT(F) \
    MOE_DCP(F, 64, 1) MOE_DCP(F, 64, 2) MOE_DCP(F, 64, 3) MOE_DCP(F, 64, 4) \
    MOE_DCP(F, 32, 1) MOE_DCP(F, 32, 2) MOE_DCP(F, 32, 3) MOE_DCP(F, 32, 4) \
    MOE_DCP(F, 16, 1) MOE_DCP(F, 16, 2) MOE_DCP(F, 16, 3) MOE_DCP(F, 16, 4) \
    MOE_DCP(F, 8, 1) MOE_DCP(F, 8, 2) MOE_DCP(F, 8, 3) MOE_DCP(F, 8, 4)
    if (quant == Q_INT4) { MOE_DCP_FMT(Q_INT4) }
    else if (quant == Q_E2M1) { MOE_DCP_FMT(Q_E2M1) }
    else { MOE_DCP_FMT(Q_F32) }
#undef MOE_DCP_FMT
#undef MOE_DCP
    return hipErrorInvalidValue;
}

template <int FMT, int LPR, int CPL>
hipError_t launch_pre_t(const GemvArgs &a, const PreArgs &pa, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    const int blk_rows = kWaves * (64 / LPR) * rows_in_flight(2, CPL);
    const dim3 grid((pa.n_routed + pa.has_shared) * a.tiles_per_unit), block(kWaves * 64);
    if (a.rows % blk_rows == 0) return launch(k_expert_gemv_pre<FMT, LPR, CPL, true>, grid, block, s, e0, e1, a, pa);
    return launch(k_expert_gemv_pre<FMT, LPR, CPL, false>, grid, block, s, e0, e1, a, pa);
}

hipError_t launch_expert_gemv_pre(int quant, const GemvArgs &a, const PreArgs &pa, hipStream_t stream, hipEvent_t e0,
                                  hipEvent_t e1) {
    const GemvShape sh = gemv_shape(quant, a.cols, 2);
    if (!sh.ok || pa.n_routed <= 0 || !pa.ids || !pa.map) return hipErrorInvalidValue;
    if (a.tiles_per_unit != (a.rows + sh.rows_per_wg - 1) / sh.rows_per_wg) return hipErrorInvalidValue;
#define MOE_PRE(F, L, C) \
    if (sh.lpr == L && sh.cpl == C) return launch_pre_t<F, L, C>(a, pa, stream, e0, e1);
#define MOE_PRE_FMT(F) \
    MOE_PRE(F, 64, 1) MOE_PRE(F, 64, 2) MOE_PRE(F, 64, 3) MOE_PRE(F, 64, 4) \
    MOE_PRE(F, 32, 1) MOE_PRE(F, 32, 2) MOE_PRE(F, 32, 3) MOE_PRE(F, 32, 4) \
    MOE_PRE(F, 16, 1) MOE_PRE(F, 16, 2) MOE_PRE(F, 16, 3) MOE_PRE(F, 16, 4) \
    MOE_PRE(F, 8, 1) MOE_PRE(F, 8, 2) MOE_PRE(F, 8, 3) MOE_PRE(F, 8, 4)
    if (quant == Q_INT4) { MOE_PRE_FMT(Q_INT4) }
    else if (quant == Q_E2M1) { MOE_PRE_FMT(Q_E2M1) }
    else { MOE_PRE_FMT(Q_F32) }
#undef MOE_PRE_FMT
#undef MOE_PRE
    return hipErrorInvalidValue;
}

hipError_t launch_expert_fused(int quant, const GemvArgs &g, const UnitList &ulg, const GemvArgs &d,
                               const CombineArgs &cb, const UnitList &uld, const FusedSync &fs, hipStream_t stream,
                               hipEvent_t e0, hipEvent_t e1) {
    if (ulg.n_units <= 0 || uld.n_units <= 0) return hipErrorInvalidValue;
    if (fs.n_gu != ulg.n_units * g.tiles_per_unit || !fs.sync || !fs.timed_out || fs.epoch == 0)
        return hipErrorInvalidValue;
    UnitListS sg, sd;
    if (!to_small(ulg, sg) || !to_small(uld, sd)) return hipErrorNotSupported;
    const GemvShape gs = gemv_shape(quant, g.cols, 2), ds = gemv_shape(quant, d.cols, 1);
    if (!gs.ok || !ds.ok) return hipErrorInvalidValue;
    if (g.tiles_per_unit != (g.rows + gs.rows_per_wg - 1) / gs.rows_per_wg) return hipErrorInvalidValue;
    // the shapes of the workloads run here; others take the two kernels
    if (quant == Q_INT4 && gs.lpr == 64 && gs.cpl == 1 && ds.lpr == 8 && ds.cpl == 3)
        return launch_fused_t<Q_INT4, 64, 1, 8, 3>(g, sg, d, cb, sd, fs, stream, e0, e1);
    if (quant == Q_E2M1 && gs.lpr == 32 && gs.cpl == 3 && ds.lpr == 16 && ds.cpl == 1)
        return launch_fused_t<Q_E2M1, 32, 3, 16, 1>(g, sg, d, cb, sd, fs, stream, e0, e1);
    if (quant == Q_F32 && gs.lpr == 64 && gs.cpl == 1 && ds.lpr == 32 && ds.cpl == 1)
        return launch_fused_t<Q_F32, 64, 1, 32, 1>(g, sg, d, cb, sd, fs, stream, e0, e1);
    return hipErrorNotSupported;
}

GemvShape gemv_shape(int quant, int cols, int n_mats) {
    GemvShape s{};
    const int per_chunk = (quant == Q_F32) ? 4 : 32;
    if (cols <= 0 || cols % per_chunk) return s;
    const int nc = cols / per_chunk;
    if (nc % 8) return s;
    for (int lpr = 64; lpr >= 8; lpr /= 2) {
        if (nc % lpr == 0 && nc / lpr <= 4) {
            s.lpr = lpr;
            s.cpl = nc / lpr;
            break;
        }
    }
    if (!s.lpr) return s;
    s.u = rows_in_flight(n_mats, s.cpl);
    s.rows_per_wg = kWaves * (64 / s.lpr) * s.u;
    s.ok = true;
    return s;
}

hipError_t launch_expert_gemv(int quant, int n_mats, const GemvArgs &a, const UnitList &ul, hipStream_t stream,
                              hipEvent_t e0, hipEvent_t e1) {
    if (ul.n_units <= 0) return hipSuccess;
    const GemvShape sh = gemv_shape(quant, a.cols, n_mats);
    if (!sh.ok) return hipErrorInvalidValue;
    if (quant == Q_INT4)
        return n_mats == 2 ? launch_fmt<Q_INT4, 2>(sh.lpr, sh.cpl, a, ul, stream, e0, e1)
                           : launch_fmt<Q_INT4, 1>(sh.lpr, sh.cpl, a, ul, stream, e0, e1);
    if (quant == Q_E2M1)
        return n_mats == 2 ? launch_fmt<Q_E2M1, 2>(sh.lpr, sh.cpl, a, ul, stream, e0, e1)
                           : launch_fmt<Q_E2M1, 1>(sh.lpr, sh.cpl, a, ul, stream, e0, e1);
    if (quant == Q_F32)
        return n_mats == 2 ? launch_fmt<Q_F32, 2>(sh.lpr, sh.cpl, a, ul, stream, e0, e1)
                           : launch_fmt<Q_F32, 1>(sh.lpr, sh.cpl, a, ul, stream, e0, e1);
    return hipErrorInvalidValue;
}

// --- decoder self-check ----------------------------------------------------------------------

__global__ void k_debug_decode(int quant, int what, const uint8_t *codes, int n, float *out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const u32 b = codes[i];
    if (quant == Q_E2M1 && what == 0) {
        const h2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(b, 1.0f, 0);
        out[2 * i] = (float)v.x;
        out[2 * i + 1] = (float)v.y;
    } else if (quant == Q_E2M1 && what == 1) {
        out[2 * i] = __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
        out[2 * i + 1] = 0.f;
    } else {
        // int4 through the same 1024-bias construction as chunk_int4
        const h2 lo = as_h2((b & 0x000Fu) | 0x64006400u);
        const h2 hi = as_h2((b & 0x00F0u) | 0x64006400u);
        out[2 * i] = (float)lo.x - 1032.0f;
        out[2 * i + 1] = ((float)hi.x - 1024.0f) * 0.0625f - 8.0f;
    }
}

hipError_t launch_debug_decode(int quant, int what, const uint8_t *codes, int n, float *out, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    return launch(k_debug_decode, dim3((n + 255) / 256), dim3(256), stream, nullptr, nullptr, quant, what, codes, n, out);
}

}  // namespace moe
