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
// Tiles: a workgroup of 4 waves computes up to 128 pairs of one expert against
// 128 output columns of both gate and up (gate/up kernel) or 256 output columns
// (down kernel); each wave takes all the item's rows and 32 columns of each of
// its two column slots, so every weight a lane dequantises feeds up to four
// MFMAs.  The reduction steps 64 elements at a time.
//   weights: the 4-bit codes of the workgroup's 256 weight rows go from memory
//     straight into LDS (16-byte loads that write LDS without passing through
//     registers), two steps per buffer, double-buffered, chunks XOR-swizzled;
//     each MFMA lane reads back its own 16 bytes (32 codes, one int4 scale group
//     or two e2m1 groups) and dequantises them in registers just before use.
//     For int4 the 8 codes of a dword come out as the pairs (k, k+4), so the
//     reduction index inside each group of 8 runs in that pair order on both
//     operands: the activations are stored in the same order (the router
//     writes x that way, this kernel writes h that way), and a contraction does
//     not depend on the order of its terms.  Scales are read into registers, 16
//     bytes per lane per 4 steps.
//   activations: rows gathered by pair id, loaded straight into a double-
//     buffered LDS tile whose 16-byte chunks are XOR-swizzled by row (conflict-
//     free reads of 32 rows at one chunk).
//   one barrier per step: every wave has read the step's buffers and its loads
//     for the next step have landed; the loads into the buffers just read are
//     issued right after it, a whole step ahead of the wait that needs them.
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
        // codes (k, k+4) at bits 0-3 / 16-19 (and 8-11 / 24-27) become fp16 1024 + q, minus
        // 1032; at bits 4-7 / 20-23 (and 12-15 / 28-31) they become 1024 + 16 q, times 1/16
        // minus 72: q - 8 exactly either way, then times s (one rounding)
        const h2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
        const h2 m72 = {(f16)-72.0f, (f16)-72.0f};
        const u32 w8 = w >> 8;
        const h2 v0 = (as_h2(bfi(0x000F000Fu, w, 0x64006400u)) - bias) * ss;
        const h2 v1 = __builtin_elementwise_fma(as_h2(bfi(0x00F000F0u, w, 0x64006400u)), sixteenth, m72) * ss;
        const h2 v2 = (as_h2(bfi(0x000F000Fu, w8, 0x64006400u)) - bias) * ss;
        const h2 v3 = __builtin_elementwise_fma(as_h2(bfi(0x00F000F0u, w8, 0x64006400u)), sixteenth, m72) * ss;
        r[0] = v0.x;
        r[1] = v0.y;
        r[2] = v1.x;
        r[3] = v1.y;
        r[4] = v2.x;
        r[5] = v2.y;
        r[6] = v3.x;
        r[7] = v3.y;
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

typedef __attribute__((address_space(3))) void lds_void;
// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at lds + 16 l
// (lds is the wave's base, uniform); past the buffer's range the lane reads zeros
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, uint4 *lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, 0);
}
// this wave's loads, LDS ones included, have completed
__device__ inline void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One item (up to 128 rows of one expert) against one column tile, for items of
// NRT row tiles of 32: rows past the item cost neither loads nor MFMAs.  The two
// buffers of each operand are separate LDS arrays, so the compiler's own waits for
// the loads into one do not hold back reads of the other.
template <int FMT, int NMAT, int NRT>
__device__ __forceinline__ void gemm_item(const PrefillGemmArgs &a, const PrefillItem &it, int tile, uint4 *As0,
                                          uint4 *As1, uint4 *Bs0, uint4 *Bs1, const int *s_pair) {
    constexpr int WCOLS = NMAT == 2 ? 32 : 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int n_steps = a.K / KS;
    const int n0 = tile * (kWavesP * WCOLS) + wave * WCOLS;

    // activations: the lane at LDS position tid of row tile i (row tid/8 + 32i, physical chunk
    // tid&7) loads the logical chunk that the swizzle puts there
    const __amdgpu_buffer_rsrc_t ars = make_rsrc(a.a, a.a_bytes);
    int a_voff[NRT];
#pragma unroll
    for (int i = 0; i < NRT; ++i) {
        const int p = s_pair[(tid >> 3) + 32 * i];
        const int row = a.a_by_token ? (p < a.nk ? p / a.top_k : p - a.nk) : p;
        a_voff[i] = row * a.K * 2 + ((tid & 7) ^ swz(tid >> 3)) * 16;
    }

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
    // 4-bit codes: LDS weight row tid/4 + 64i, physical chunk tid&3, holds the logical chunk
    // the swizzle puts there
    const int bl_voff = [&] {
        const int brow = tid >> 2, csv = (brow >> 5) & 1;
        const int col = tile * (kWavesP * WCOLS) + (NMAT == 2 ? 0 : 32 * csv) + (brow & 31);
        const int moff = (int)((NMAT == 2 && csv == 1) ? a.mat_off1 : a.mat_off0);
        return moff + col * (a.K / 2) + 16 * ((tid & 3) ^ bswz(brow));
    }();
    const int bl_step = WCOLS * (a.K / 2);
    const int b_rd = (64 * wave + (lane & 31)) * 4;
    const int b_sw = bswz(lane & 31);

    auto dma_a = [&](uint4 *buf, int g) {
#pragma unroll
        for (int i = 0; i < NRT; ++i) dma16(ars, buf + 256 * i + 64 * wv, a_voff[i], g * KS * 2);
    };
    auto dma_b = [&](uint4 *buf, int s2) {
        if constexpr (FMT != Q_F32) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dma16(brs, buf + 256 * i + 64 * wv, bl_voff, s2 * 64 + i * bl_step);
        }
    };
    BRaw<FMT> br;
    uint4 sc[2];
    u32 sc3[2];
    auto load_sc = [&](int g4) {
        if constexpr (FMT != Q_F32) {
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) sc[cs] = ld16(brs, s_voff[cs], g4 * 16);
        }
    };
    auto load_b = [&](int g) {
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

    const int m = lane & 31;
    const int a_rd = m * 8;
    const int a_sw = swz(m);

    // prologue: activations of steps 0 and 1, codes of steps 0 .. 3, scales of steps 0 .. 3
    dma_a(As0, 0);
    dma_a(As1, min(1, n_steps - 1));
    dma_b(Bs0, 0);
    dma_b(Bs1, min(1, n_steps / 2 - 1));
    load_sc(0);
    load_b(0);
    wait_loads();
    __syncthreads();

    // step g reads activation buffer g&1 and code buffer (g/2)&1; at its end, once every wave
    // has read them and every wave's loads for step g+1 have landed, step g+2's activations go
    // into the buffer just read, and after an odd step the codes of steps g+3, g+4 into the
    // code buffer just read
    auto step = [&](auto uc, int g) {
        constexpr int u = decltype(uc)::value;
        uint4 *const Ab = (u & 1) ? As1 : As0;
        uint4 *const Bb = ((u >> 1) & 1) ? Bs1 : Bs0;
        if constexpr (FMT != Q_F32) {
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
                const u32 d = u == 0 ? sc[cs].x : u == 1 ? sc[cs].y : u == 2 ? sc[cs].z : sc3[cs];
                br.s[cs] = d >> (16 * j);
                br.q[cs] = Bb[b_rd + 128 * cs + ((2 * (u & 1) + j) ^ b_sw)];
            }
        }
#pragma unroll
        for (int kh = 0; kh < 4; ++kh) {
            const int chunk = (4 * j + kh) ^ a_sw;
            half8 av[NRT];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) av[rt] = __builtin_bit_cast(half8, Ab[a_rd + 256 * rt + chunk]);
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
                const half8 bv = operand<FMT>(br, cs, kh);
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    acc[rt][cs] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[rt], bv, acc[rt][cs], 0, 0, 0);
            }
        }
        load_b(min(g + 1, n_steps - 1));
        wait_loads();
        __syncthreads();
        dma_a(Ab, min(g + 2, n_steps - 1));
        if constexpr ((u & 1) == 1) dma_b(Bb, min(g / 2 + 2, n_steps / 2 - 1));
        if constexpr (u == 2 && FMT != Q_F32) {
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) sc3[cs] = sc[cs].w;
            load_sc(min(g / 4 + 1, n_steps / 4 - 1));
        }
        // keep the loads here, a whole step ahead of the wait that needs them
        __builtin_amdgcn_sched_barrier(0);
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
    // the last steps' loads into LDS must land before the workgroup's LDS is handed on
    wait_loads();

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
    __shared__ __align__(16) uint4 As0[BM * 8];       // [row][8 chunks of 8 fp16], chunks swizzled
    __shared__ __align__(16) uint4 As1[BM * 8];
    __shared__ __align__(16) uint4 Bs0[kBRows * 4];   // [weight row][4 chunks of 32 codes], swizzled
    __shared__ __align__(16) uint4 Bs1[kBRows * 4];
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
    case 1: gemm_item<FMT, NMAT, 1>(a, it, tile, As0, As1, Bs0, Bs1, s_pair); break;
    case 2: gemm_item<FMT, NMAT, 2>(a, it, tile, As0, As1, Bs0, Bs1, s_pair); break;
    case 3: gemm_item<FMT, NMAT, 3>(a, it, tile, As0, As1, Bs0, Bs1, s_pair); break;
    default: gemm_item<FMT, NMAT, 4>(a, it, tile, As0, As1, Bs0, Bs1, s_pair); break;
    }
}

// 16 bytes per thread, then the last 4-byte words.
__global__ __launch_bounds__(256) void k_copy_from_host(const uint4 *src, uint4 *dst, int n16, int n4) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n16) dst[i] = src[i];
    if (i < n4 - 4 * n16)
        reinterpret_cast<uint32_t *>(dst)[4 * n16 + i] = reinterpret_cast<const uint32_t *>(src)[4 * n16 + i];
}

}  // namespace

hipError_t launch_copy_from_host(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    if (bytes % 4 || bytes > 0x7FFFFFF0u || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
        return hipErrorInvalidValue;
    const int n16 = (int)(bytes / 16), n4 = (int)(bytes / 4);
    const int n = std::max(n16, n4 - 4 * n16);
    return launch(k_copy_from_host, dim3((n + 255) / 256), dim3(256), stream, nullptr, nullptr,
                  static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n16, n4);
}

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
