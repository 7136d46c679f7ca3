// kernels.h -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Quantization group: weights per fp32 scale.
constexpr int kGroup = 128;

// Largest expert count the router/top-k and dispatch kernels support.
constexpr int kMaxExperts = 256;

// Tile height (token rows) of the prefill grouped GEMMs; the dispatch step
// lays out its tile table for this height.
constexpr int kPrefillBM = 128;

// K1
hipError_t launch_quantize_int4(const float* w, int64_t rows, int64_t K, uint8_t* q,
                                float* scales, hipStream_t stream);

// K2: logits [T, E] = x @ router_w^T (+ b), fp32
hipError_t launch_router_logits(const uint16_t* x, const float* wr, const float* b, int64_t T,
                                int64_t d, int64_t E, float* logits, hipStream_t stream);
// K2: top-k per token (ties to the lower id) and sigmoid gates
hipError_t launch_topk(const float* logits, int64_t T, int64_t E, int top_k, int32_t* ids,
                       float* gates, int32_t* ids_copy, float* gates_copy, hipStream_t stream);

// K3: counts, offsets, GEMM tile table, stable permutation and its inverse
hipError_t launch_dispatch(const int32_t* ids, int64_t T, int top_k, int64_t E, int tile_rows,
                           int32_t* counts, int32_t* offsets, int32_t* tile_base, int32_t* perm,
                           int32_t* inv, hipStream_t stream);

struct GroupedGemmArgs {
    const uint16_t* a;       // up: x [T, d]; down: H [P + T, h]
    int64_t T;
    int64_t P;
    int top_k;
    int E;
    int64_t K;               // reduction dim (up: d, down: h)
    int64_t N;               // output features (up: h, down: d)
    const int32_t* perm;
    const int32_t* offsets;
    const int32_t* counts;
    const int32_t* tile_base;
    const uint8_t* wq0;      // up: W1, down: W2 (int4, [E, N, K/2])
    const float* ws0;        //   scales [E, N, K/128]
    const uint8_t* wq1;      // up: W3
    const float* ws1;
    const uint16_t* sh0;     // up: S1, down: S2 (bf16 [N, K])
    const uint16_t* sh1;     // up: S3
    uint16_t* h_out;         // up: H [P + T, h] bf16
    float* o_out;            // down: O [P + T, d] fp32
};

// K4 (routed) + K6a (shared): H = silu(A W1^T) * (A W3^T), one launch
hipError_t launch_grouped_up(const GroupedGemmArgs& args, hipStream_t stream);
// K5 (routed) + K6b (shared): O = H W2^T, one launch
hipError_t launch_grouped_down(const GroupedGemmArgs& args, hipStream_t stream);

// K6c: y[t] = O[P + t] + sum_j gate[t, j] * O[inv[t, j]]  -> bf16
hipError_t launch_combine(const float* O, const float* gates, const int32_t* inv, int64_t T,
                          int64_t P, int top_k, int64_t d, uint16_t* y, hipStream_t stream);

}  // namespace moe
