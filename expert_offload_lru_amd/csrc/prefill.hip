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
// Tiles: a workgroup of 2 waves computes 128 pairs of one expert against 64
// output columns of both gate and up (gate/up kernel) or 128 output columns
// (down kernel); each wave takes all 128 rows and 32 columns of each of its two
// column slots, so every weight a lane dequantises feeds four MFMAs.  The
// reduction steps 64 elements at a time.
//   weights: each lane loads the 32 codes (16 bytes, one int4 scale group or
//     two e2m1 groups) that it supplies to the MFMA itself, four steps ahead,
//     straight into registers, and dequantises them there just before use;
//     no LDS, no barrier.  For int4 the 8 codes of a dword come out as the
//     pairs (k, k+4), so the reduction index inside each group of 8 runs in
//     that pair order on both operands: the activations are stored in the
//     same order (the router writes x that way, this kernel writes h that
//     way), and a contraction does not depend on the order of its terms.
//   activations: rows gathered by pair id into registers two steps ahead,
//     then into a double-buffered LDS tile whose 16-byte chunks are XOR-
//     swizzled by row (conflict-free reads of 32 rows at one chunk); one
//     barrier per step.
// Activations are fp16: the same MFMA rate as bf16 on gfx950, and with bf16
// activations the layer output misses the stated 2e-3 max|ref| tolerance.
#include "kernels.hpp"

namespace moe {
namespace {

typedef _Float16 f16;
typedef f16 h2 __attribute__((ext_vector_type(2)));
typedef f16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32;

__device__ inline h2 as_h2(u32 v) { return __builtin_bit_cast(h2, v); }

constexpr int BM = kPrefillRows;   // rows (pairs) per item
constexpr int KS = 64;             // reduction elements per step
constexpr int kWavesP = 4;         // waves per workgroup
constexpr int kBRows = kWavesP * 64;   // weight rows of a workgroup (4 waves x 2 slots x 32 columns)
static_assert(BM == 128, "thread mapping assumes 128-row items");

constexpr int kRsrcWord3 = 0x00020000;   // buffer resource flags of the gfx9 family (raw, untyped)

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ inline uint4 ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ inline u32 ld2(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return (u32)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// Swizzle of the 16-byte chunks of LDS row r: 32 consecutive rows read at one
// logical chunk land on distinct banks (for 32- and for 64-bank LDS).
__device__ inline int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// (a & mask) | (b & ~mask) in one instruction.
__device__ inline u32 bfi(u32 mask, u32 a, u32 b) {
    u32 r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(a), "v"(b));
    return r;
}

// Swizzle of the four 16-byte chunks of LDS weight row r (bits 1-3 of r): the 16-byte
// reads of 32 consecutive rows, two chunks per row, are conflict-free whether the LDS
// serves 8 or 16 lanes per pass and whether a pass pairs lanes l and l+32.
__device__ inline int bswz(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | ((((r >> 1) ^ (r >> 2)) & 1) << 1); }

// Column position of natural column c inside the pair order of its group of 8.
__device__ inline int pair_pos(int c) { return (c & ~7) | ((c & 3) << 1) | ((c >> 2) & 1); }

// Raw weights of one lane, one step, its two column slots.
template <int FMT>
struct BRaw {
    uint4 q[2];
    u32 s[2];
};
template <>
struct BRaw<Q_F32> {
    uint4 f[2][8];
};

// 8 weights (reduction elements 8kh .. 8kh+7 of the lane's 32) of slot cs as an MFMA operand.
template <int FMT>
__device__ inline half8 operand(const BRaw<FMT> &b, int cs, int kh) {
    half8 r;
    if constexpr (FMT == Q_INT4) {
        const u32 w = kh == 0 ? b.q[cs].x : kh == 1 ? b.q[cs].y : kh == 2 ? b.q[cs].z : b.q[cs].w;
        const f16 s = __builtin_bit_cast(f16, (unsigned short)(b.s[cs] & 0xFFFFu));
        const h2 ss = {s, s};
        const h2 bias = {(f16)1032.0f, (f16)1032.0f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // codes m and m+4 of the dword into fp16 1024 + q, minus 1032, times s (one rounding)
            const h2 q = as_h2(bfi(0x000F000Fu, w >> (4 * m), 0x64006400u));
            const h2 v = (q - bias) * ss;
            r[2 * m] = v.x;
            r[2 * m + 1] = v.y;
        }
    } else if constexpr (FMT == Q_E2M1) {
        const u32 w = kh == 0 ? b.q[cs].x : kh == 1 ? b.q[cs].y : kh == 2 ? b.q[cs].z : b.q[cs].w;
        // elements 0..15 of the 32 use scale byte 0, 16..31 byte 1
        const float sf = __builtin_amdgcn_cvt_f32_fp8((int)(b.s[cs] >> (kh < 2 ? 0 : 8)), 0);
        const f16 s = (f16)sf;
        const h2 ss = {s, s};
        const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
        const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
        const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
        const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
        r[0] = p0.x;
        r[1] = p0.y;
        r[2] = p1.x;
        r[3] = p1.y;
        r[4] = p2.x;
        r[5] = p2.y;
        r[6] = p3.x;
        r[7] = p3.y;
    } else {
        const float4 lo = __builtin_bit_cast(float4, b.f[cs][2 * kh]);
        const float4 hi = __builtin_bit_cast(float4, b.f[cs][2 * kh + 1]);
        r[0] = (f16)lo.x;
        r[1] = (f16)lo.y;
        r[2] = (f16)lo.z;
        r[3] = (f16)lo.w;
        r[4] = (f16)hi.x;
        r[5] = (f16)hi.y;
        r[6] = (f16)hi.z;
        r[7] = (f16)hi.w;
    }
    return r;
}

// One item (up to 128 rows of one expert) against one column tile, for items of
// NRT row tiles of 32: rows past the item cost neither loads nor MFMAs.
template <int FMT, int NMAT, int NRT>
__device__ __forceinline__ void gemm_item(const PrefillGemmArgs &a, const PrefillItem &it, int tile,
                                          uint4 (*As)[BM * 8], uint4 (*Bs)[kBRows * 4], const int *s_pair) {
    constexpr int WCOLS = NMAT == 2 ? 32 : 64;  // output columns per wave (per matrix)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_steps = a.K / KS;
    const int n0 = tile * (kWavesP * WCOLS) + wave * WCOLS;

    // activations: thread -> chunk ac of rows tid/8 + 32i (i < NRT); rows past the item repeat
    // row 0 of the item (never stored)
    const __amdgpu_buffer_rsrc_t ars = make_rsrc(a.a, a.a_bytes);
    const int ac = tid & 7;
    int a_voff[NRT];
#pragma unroll
    for (int i = 0; i < NRT; ++i) {
        const int p = s_pair[(tid >> 3) + 32 * i];
        const int row = a.a_by_token ? (p < a.nk ? p / a.top_k : p - a.nk) : p;
        a_voff[i] = row * a.K * 2 + ac * 16;
    }
    // LDS slot of those chunks: rows tid/8 + 32i share the swizzle
    const int a_lds = (tid >> 3) * 8 + (ac ^ swz(tid >> 3));

    // weights: lane -> column n0 + (lane & 31) (+32 for the second slot of the down kernel),
    // elements 32j .. 32j+31 of each step.  fp32 weights are loaded by the lane itself (b_voff);
    // 4-bit scales too (s_voff: the 4 steps of 256 elements of a row are 16 bytes of scales,
    // int4 8 fp16, e2m1 16 E4M3); 4-bit codes come through LDS, below
    const int j = lane >> 5;
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(reinterpret_cast<const void *>(it.block), a.block_bytes);
    int b_voff[2], s_voff[2];
    bool col_ok[2];
#pragma unroll
    for (int cs = 0; cs < 2; ++cs) {
        const int col = n0 + (lane & 31) + (NMAT == 2 ? 0 : 32 * cs);
        col_ok[cs] = col < a.N;
        const int row = col_ok[cs] ? col : a.N - 1;
        const int moff = (int)((NMAT == 2 && cs == 1) ? a.mat_off1 : a.mat_off0);
        const int nib = a.N * (a.K / 2);
        b_voff[cs] = moff + row * a.K * 4 + j * 128;
        s_voff[cs] = FMT == Q_INT4 ? moff + nib + row * (a.K / 32) * 2 : moff + nib + row * (a.K / 16);
    }

    // 4-bit codes go through LDS: the workgroup's kBRows weight rows (row 64w + 32cs + n is
    // the column n of wave w, slot cs) hold 2 steps (64 bytes) per buffer, loaded 4 lanes to a
    // row (16 rows per instruction) and read back 16 bytes per MFMA lane; chunks swizzled
    // (rows of columns past N read whatever follows, or zeros past the block; never stored)
    const int bl_c = tid & 3;
    const int bl_voff = [&] {
        const int brow = tid >> 2, csv = (brow >> 5) & 1;
        const int col = tile * (kWavesP * WCOLS) + (NMAT == 2 ? 0 : 32 * csv) + (brow & 31);
        const int moff = (int)((NMAT == 2 && csv == 1) ? a.mat_off1 : a.mat_off0);
        return moff + col * (a.K / 2) + 16 * bl_c;
    }();
    const int bl_step = WCOLS * (a.K / 2);   // the rows loaded 64 apart belong to the next wave
    const int bl_lds = (tid >> 2) * 4 + (bl_c ^ bswz(tid >> 2));
    const int b_rd = (64 * wave + (lane & 31)) * 4;
    const int b_sw = bswz(lane & 31);
    uint4 bst[4];
    auto load_bs = [&](int s2) {
        if constexpr (FMT != Q_F32) {
#pragma unroll
            for (int i = 0; i < 4; ++i) bst[i] = ld16(brs, bl_voff, s2 * 64 + i * bl_step);
        }
    };
    auto store_bs = [&](int buf) {
        if constexpr (FMT != Q_F32) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Bs[buf][bl_lds + 256 * i] = bst[i];
        }
    };

    uint4 ar[2][NRT];
    BRaw<FMT> br;   // this step's weights of the lane (codes and scales, or fp32 values)
    // scales of a group of 4 steps (4-bit formats; the reduction length is a multiple of 256
    // there): dword u holds step u's, half j lane group j's.  The next group's are loaded
    // after step 2; step 3 uses the dword kept aside
    uint4 sc[2];
    u32 sc3[2];
    auto load_sc = [&](int g4) {
        if constexpr (FMT != Q_F32) {
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) sc[cs] = ld16(brs, s_voff[cs], g4 * 16);
        }
    };
    auto load_a = [&](int set, int g) {
#pragma unroll
        for (int i = 0; i < NRT; ++i) ar[set][i] = ld16(ars, a_voff[i], g * KS * 2);
    };
    auto store_a = [&](int set, int buf) {
#pragma unroll
        for (int i = 0; i < NRT; ++i) As[buf][a_lds + 256 * i] = ar[set][i];
    };
    auto load_b = [&](int g) {   // fp32 weights: per lane, one step ahead
        if constexpr (FMT == Q_F32) {
#pragma unroll
            for (int cs = 0; cs < 2; ++cs)
#pragma unroll
                for (int q = 0; q < 8; ++q) br.f[cs][q] = ld16(brs, b_voff[cs], g * KS * 4 + 16 * q);
        }
    };

    float16v acc[NRT][2];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int cs = 0; cs < 2; ++cs)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[rt][cs][i] = 0.f;

    // MFMA operand rows: lane -> row 32rt + (lane & 31), logical chunk 4j + kh
    const int m = lane & 31;
    const int a_rd = m * 8;
    const int a_sw = swz(m);

    // prologue: activations of steps 0 and 1 in flight, step 0 in LDS; weight codes of steps
    // 0, 1 in LDS and of 2, 3 in flight; scales of steps 0 .. 3
    load_a(0, 0);
    load_a(1, min(1, n_steps - 1));
    load_b(0);
    load_bs(0);
    store_bs(0);
    load_bs(min(1, n_steps / 2 - 1));
    load_sc(0);
    store_a(0, 0);
    load_a(0, min(2, n_steps - 1));
    __syncthreads();

    // step g: MFMAs on activation buffer g&1 and weight buffer (g/2)&1; after an odd step the
    // codes of steps g+1, g+2 go into the other weight buffer and those of g+3, g+4 are
    // loaded; step g+1's activations into the other buffer; step g+3's loads out
    auto step = [&](auto uc, int g) {
        constexpr int u = decltype(uc)::value;
        constexpr int buf = u & 1;
        constexpr int wbuf = (u >> 1) & 1;
        if constexpr (FMT != Q_F32) {
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
                const u32 d = u == 0 ? sc[cs].x : u == 1 ? sc[cs].y : u == 2 ? sc[cs].z : sc3[cs];
                br.s[cs] = d >> (16 * j);
                br.q[cs] = Bs[wbuf][b_rd + 128 * cs + ((2 * (u & 1) + j) ^ b_sw)];
            }
        }
#pragma unroll
        for (int kh = 0; kh < 4; ++kh) {
            const int chunk = (4 * j + kh) ^ a_sw;
            half8 av[NRT];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
                av[rt] = __builtin_bit_cast(half8, As[buf][a_rd + 256 * rt + chunk]);
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
                const half8 bv = operand<FMT>(br, cs, kh);
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    acc[rt][cs] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[rt], bv, acc[rt][cs], 0, 0, 0);
            }
        }
        // past the last step the loads repeat it and the store fills the idle buffer: no
        // branches, so the accumulators keep their registers through the loop
        load_b(min(g + 1, n_steps - 1));
        if constexpr ((u & 1) == 1) {
            store_bs(wbuf ^ 1);
            load_bs(min(g / 2 + 2, n_steps / 2 - 1));
        }
        if constexpr (u == 2 && FMT != Q_F32) {
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) sc3[cs] = sc[cs].w;
            load_sc(min(g / 4 + 1, n_steps / 4 - 1));
        }
        store_a(buf ^ 1, buf ^ 1);
        load_a(buf ^ 1, min(g + 3, n_steps - 1));
        __syncthreads();
    };
    int g0 = 0;
    for (; g0 + 4 <= n_steps; g0 += 4) {
        step(std::integral_constant<int, 0>{}, g0);
        step(std::integral_constant<int, 1>{}, g0 + 1);
        step(std::integral_constant<int, 2>{}, g0 + 2);
        step(std::integral_constant<int, 3>{}, g0 + 3);
    }
    if (g0 < n_steps) step(std::integral_constant<int, 0>{}, g0);
    if (g0 + 1 < n_steps) step(std::integral_constant<int, 1>{}, g0 + 1);
    if (g0 + 2 < n_steps) step(std::integral_constant<int, 2>{}, g0 + 2);

    // epilogue: register i of lane l is row (i/4)*8 + (l/32)*4 + i%4, column l%32 of a 32x32 tile
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 32 * rt + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
            if (r >= it.rows) continue;
            const int p = s_pair[r];
            if constexpr (NMAT == 2) {
                if (!col_ok[0]) continue;
                const int col = n0 + (lane & 31);
                const float gv = acc[rt][0][i];
                const float h = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * acc[rt][1][i];
                const int pos = FMT == Q_INT4 ? pair_pos(col) : col;
                static_cast<f16 *>(a.out)[(size_t)p * a.N + pos] = (f16)h;
            } else {
#pragma unroll
                for (int cs = 0; cs < 2; ++cs)
                    if (col_ok[cs])
                        static_cast<float *>(a.out)[(size_t)p * a.N + n0 + 32 * cs + (lane & 31)] = acc[rt][cs][i];
            }
        }
    }
}

template <int FMT, int NMAT>
__global__ __launch_bounds__(kWavesP * 64) __attribute__((amdgpu_waves_per_eu(FMT == Q_F32 ? 1 : 2, 2))) void k_prefill_gemm(
    PrefillGemmArgs a) {
    __shared__ __align__(16) uint4 As[2][BM * 8];       // [row][8 chunks of 8 fp16], chunks swizzled
    __shared__ __align__(16) uint4 Bs[2][kBRows * 4];   // [weight row][4 chunks of 32 codes], swizzled
    __shared__ int s_pair[BM];

    // Workgroups are dispatched to the 8 XCDs round-robin by index, and each XCD has
    // its own L2 and starts its workgroups in index order.  With a schedule the host
    // has placed every item on one XCD, longest items first; without one, every XCD
    // takes one contiguous run of (item, tile) pairs.  Either way the column tiles of
    // an item, which all read the same gathered activation rows, share one L2.
    int wg;
    if (a.sched) {
        wg = a.sched[blockIdx.x];
        if (wg < 0) return;
    } else {
        const int n_wg = gridDim.x, xcd = blockIdx.x & 7, per = n_wg >> 3;
        wg = xcd * per + min(xcd, n_wg & 7) + (blockIdx.x >> 3);
    }
    const int item = wg / a.n_tiles;
    const int tile = wg - item * a.n_tiles;
    const PrefillItem it = a.items[item];
    const int tid = threadIdx.x;

    if (tid < BM) s_pair[tid] = a.pairs[it.pair_off + (tid < it.rows ? tid : 0)];   // rows past the item: row 0
    __syncthreads();

    switch ((it.rows + 31) >> 5) {
    case 1: gemm_item<FMT, NMAT, 1>(a, it, tile, As, Bs, s_pair); break;
    case 2: gemm_item<FMT, NMAT, 2>(a, it, tile, As, Bs, s_pair); break;
    case 3: gemm_item<FMT, NMAT, 3>(a, it, tile, As, Bs, s_pair); break;
    default: gemm_item<FMT, NMAT, 4>(a, it, tile, As, Bs, s_pair); break;
    }
}

}  // namespace

int prefill_tiles(int n_mats, int N) {
    const int wg_cols = kWavesP * (n_mats == 2 ? 32 : 64);
    return (N + wg_cols - 1) / wg_cols;
}

hipError_t launch_prefill_gemm(int quant, int n_mats, const PrefillGemmArgs &a, hipStream_t stream, hipEvent_t e0,
                               hipEvent_t e1) {
    if (a.n_items <= 0) return hipSuccess;
    if (a.K % KS != 0 || a.N % 32 != 0 || a.a_bytes > 0x7FFFFFFFu || a.block_bytes > 0x7FFFFFFFu ||
        (quant != Q_F32 && a.K % (4 * KS) != 0))   // 4-bit scales are read 4 steps at a time
        return hipErrorInvalidValue;
    PrefillGemmArgs g = a;
    g.n_tiles = prefill_tiles(n_mats, a.N);
    const dim3 grid(g.sched ? g.n_sched : g.n_items * g.n_tiles), block(kWavesP * 64);
    if (grid.x == 0) return hipSuccess;
    if (quant == Q_INT4) return n_mats == 2 ? launch(k_prefill_gemm<Q_INT4, 2>, grid, block, stream, e0, e1, g)
                                            : launch(k_prefill_gemm<Q_INT4, 1>, grid, block, stream, e0, e1, g);
    if (quant == Q_E2M1) return n_mats == 2 ? launch(k_prefill_gemm<Q_E2M1, 2>, grid, block, stream, e0, e1, g)
                                            : launch(k_prefill_gemm<Q_E2M1, 1>, grid, block, stream, e0, e1, g);
    return n_mats == 2 ? launch(k_prefill_gemm<Q_F32, 2>, grid, block, stream, e0, e1, g)
                       : launch(k_prefill_gemm<Q_F32, 1>, grid, block, stream, e0, e1, g);
}

}  // namespace moe
