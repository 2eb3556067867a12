// Internal interface between the host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace moe {

enum Quant { Q_F32 = 0, Q_INT4 = 1, Q_E2M1 = 2 };

// Work list of one expert-GEMV launch, passed by value as a kernel argument.
// A unit is one distinct expert of a wave: its weights (a pool slot, or the
// shared expert) and the (token, pick) pairs routed to it.  A pair id is
// t*top_k + j for routed picks and n_tok*top_k + t for the shared expert.
constexpr int kMaxUnits = 128;
constexpr int kMaxPairs = 128;
constexpr int kTokChunk = 8;    // token vectors a GEMV workgroup stages in LDS at a time

struct UnitList {
    int32_t n_units;
    int32_t slot[kMaxUnits];          // >= 0: block at bank + slot*S; -1: shared expert block
    uint16_t pbeg[kMaxUnits + 1];     // pairs of unit u: pair[pbeg[u] .. pbeg[u+1])
    uint16_t pair[kMaxPairs];
};

// One expert-GEMV launch: out[p][r] = sum_c W[r][c] * v[p][c] for the rows
// of each unit's matrix, or, for the gate/up kernel,
// out[p][r] = silu(Wg[r].v) * (Wu[r].v).
struct GemvArgs {
    const uint8_t *bank;       // slot bank base of the pool
    const uint8_t *shared_w;   // block of the shared expert (or null)
    size_t block_bytes;        // S
    size_t mat_off0;           // byte offset of the (first) matrix inside a block
    size_t mat_off1;           // byte offset of the second matrix (gate/up kernel)
    int rows;                  // R
    int cols;                  // C (reduction)
    const float *vec;          // fp32 input vectors
    int vec_by_token;          // 1: row of vec = token of the pair; 0: row = pair id
    int nk;                    // n_tok * top_k (first shared-expert pair id)
    int top_k;
    float *out;                // fp32 [pairs x R]
    int tiles_per_unit;
};

struct GemvShape {             // launch shape chosen for (quant, cols, n_mats)
    int lpr, cpl, u;           // lanes per row, 16-byte chunks per lane, rows in flight per lane
    int rows_per_wg;
    size_t lds_per_token;
    bool ok;
};

GemvShape gemv_shape(int quant, int cols, int n_mats);

// Launch one expert GEMV over `ul` (n_mats = 2: gate/up + SwiGLU, 1: down).
hipError_t launch_expert_gemv(int quant, int n_mats, const GemvArgs &a, const UnitList &ul, int max_pairs_per_unit,
                              hipStream_t stream);

// Router: logits in float64 from float32 operands, softmax, top-k in rank
// order (descending logit, ties to the lower index), for one or two router
// matrices (the second is the next layer's, for speculative prefetch).
struct RouterArgs {
    const float *x;            // [n_tok x H]
    const float *w0;           // [E x H]
    const float *w1;           // [E x H] or null
    int n_tok, E, H, top_k;
    double *z;                 // scratch [n_mats x n_tok x E]
    unsigned *counters;        // one per 32-token block, zero between launches
    int32_t *ids;              // [n_tok x top_k] device
    float *gate;               // [n_tok x top_k] device
    int32_t *ids_host;         // device-visible pinned copies (may be null)
    float *gate_host;
    int32_t *spec_ids_host;    // next-layer picks (w1) or null
};
hipError_t launch_router(const RouterArgs &a, hipStream_t stream);

// out[t] = (residual ? x[t] : 0) + sum_j gate[t,j] * Y[t*k+j] (+ Y[nk+t] with a shared expert)
hipError_t launch_combine(const float *x, const float *y, const float *gate, float *out, int n_tok, int H, int top_k,
                          int has_shared, int residual, hipStream_t stream);

hipError_t launch_debug_decode(int quant, int what, const uint8_t *codes, int n, float *out, hipStream_t stream);

}  // namespace moe
