// kernels.h -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Per-stage kernel timing (moe_profile_*). While the host has set `stop`, each
// launch of this thread goes through hipExtLaunchKernelGGL, which records the
// events at the kernel's own start and end: the stage's first launch takes
// `start` (then cleared), every launch records `stop`. Otherwise launches are
// plain hipLaunchKernelGGL.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
LaunchTiming& launch_timing();

#define MOE_LAUNCH(kernel, grid, block, lds, stream, ...)                                     \
    do {                                                                                      \
        ::moe::LaunchTiming& lt_ = ::moe::launch_timing();                                    \
        if (lt_.stop) {                                                                       \
            hipEvent_t st_ = lt_.start;                                                       \
            lt_.start = nullptr;                                                              \
            hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), stream, st_, \
                                  lt_.stop, 0, __VA_ARGS__);                                  \
        } else {                                                                              \
            hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                \
        }                                                                                     \
    } while (0)

// Tile width of the tiled weight layouts (columns per 16-row tile), and the
// default quantization group. Int4 groups of 64 or 32 weights keep the same
// code tiles and store 128 / group scales per tile row.
constexpr int kGroup = 128;

// Largest expert count the router/top-k and dispatch kernels support.
constexpr int kMaxExperts = 256;

// Tile heights (token rows) of the prefill grouped GEMMs; the dispatch step
// lays out its tile table for the one the forward uses.
constexpr int kPrefillBM = 128;
constexpr int kPrefillBM2 = 256;  // 256 x 256 tiles (gemm256.hip) for large experts

// Rows per decode chunk (the M of one MFMA tile).
constexpr int kDecodeRows = 16;
// Largest T * E the one-block small-batch routing keeps in LDS.
constexpr int kSmallRouteLogits = 8192;
// Largest T * top_k the one-block small-batch routing handles.
constexpr int kSmallRoutePairs = 1024;

// K1 (row-major groups, or the 16-row tiles the forward pass reads)
// group: 128, 64 or 32 weights per scale; K % 128 == 0
hipError_t launch_quantize_int4(const float* w, int64_t rows, int64_t K, int group, uint8_t* q,
                                float* scales, bool tiled, hipStream_t stream);
// row-major int4 codes [rows, K/2] + scales [rows, K/group] -> the tiled order
// (rows % 16 == 0)
hipError_t launch_tile_int4(const uint8_t* q_rm, const float* s_rm, int64_t rows, int64_t K, int group,
                            uint8_t* q_t, float* s_t, hipStream_t stream);
// fp8 (E4M3) row-wise quantization: weights fp32 [rows, K] -> tiled codes
// (16 x 128 tiles of 4 steps x 16 rows x 32 bytes) + per-row scales;
// activations bf16 [rows, K] -> row-major codes + per-row scales (ub > 0
// bounds a row's maximum)
hipError_t launch_quantize_fp8_weights(const float* w, int64_t rows, int64_t K, uint8_t* q,
                                       float* scales, hipStream_t stream);
hipError_t launch_quantize_fp8_activations(const uint16_t* x, int64_t rows, int64_t K, float ub,
                                           uint8_t* q, float* scales, hipStream_t stream);
// bf16 [rows, K] -> 16 x 128 tiles in MFMA step order (shared expert weights)
hipError_t launch_pack_bf16(const uint16_t* src, int64_t rows, int64_t K, uint16_t* dst,
                            hipStream_t stream);

// K2: router tiling and reduction split for a batch shape
struct RouterPlan {
    int kind;    // tile variant
    int tt, ee;  // tokens x experts per block
    int slices;  // reduction slices (split-K); partial sums [slices, T, E]
};
RouterPlan router_plan(int64_t T, int64_t d, int64_t E);
// Most reduction slices of the MFMA router plan
constexpr int kMaxRouterSlices = 16;
// Batches of at least this many tokens compute the router logits on MFMA
constexpr int64_t kRouterMfmaTokens = 256;
// K2: partials[s][t][e] = sum over slice s of x[t, :] router_w[e, :]   (fp32)
// (optional) x_perm: x with 8-element blocks in the order 0,4,1,5,2,6,3,7
hipError_t launch_router_partials(const uint16_t* x, const float* wr, int64_t T, int64_t d,
                                  int64_t E, const RouterPlan& plan, float* partials,
                                  uint16_t* x_perm, hipStream_t stream);
// K2: logits = sum of slices (+ bias), top-k per token (ties to the lower id), sigmoid gates
hipError_t launch_topk(const float* partials, int slices, const float* bias, int64_t T, int64_t E,
                       int top_k, float* logits, int32_t* ids, float* gates, int32_t* ids_copy,
                       float* gates_copy, hipStream_t stream);
// K2 + K3 for small batches in one block: logits, top-k, gates, counts, offsets,
// GEMM tile table, perm, inv and the decode row chunks (int4: group, first row, rows, 0)
hipError_t launch_route_small(const float* partials, int slices, const float* bias, int64_t T,
                              int64_t E, int top_k, int tile_rows, int small_rows, float* logits,
                              int32_t* ids,
                              float* gates, int32_t* ids_copy, float* gates_copy, int32_t* counts,
                              int32_t* offsets, int32_t* tile_base, int32_t* perm, int32_t* inv,
                              int4* chunks, int32_t* nchunks, hipStream_t stream);

// K3: counts, offsets, GEMM tile table, stable permutation and its inverse, decode chunks
hipError_t launch_dispatch(const int32_t* ids, int64_t T, int top_k, int64_t E, int tile_rows,
                           int small_rows, int32_t* counts, int32_t* offsets, int32_t* tile_base, int32_t* perm,
                           int32_t* inv, int4* chunks, int32_t* nchunks, hipStream_t stream);

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
    const float* ws0;        //   scales [E, N, K/group]
    int spt;                 //   int4 scales per tile row: 128 / group (1, 2 or 4)
    const uint8_t* wq1;      // up: W3
    const float* ws1;
    const uint16_t* sh0;     // up: S1, down: S2 (bf16 [N, K])
    const uint16_t* sh1;     // up: S3
    const uint16_t* wb0;     // bf16 routed experts instead of int4 (null: int4):
    const uint16_t* wb1;     //   up: W1 / W3, down: W2 (tiled bf16 [E, N, K])
    const uint8_t* wf0;      // fp8 routed experts instead of int4 (null: int4):
    const uint8_t* wf1;      //   up: W1 / W3, down: W2 (tiled fp8 [E, N, K])
    const float* wfs0;       //   their row scales [E, N]
    const float* wfs1;
    const uint8_t* a8;       // fp8 routed rows of A (up: x_q [T, d] by token;
    const float* a8s;        //   down: H_q [P, h] by slot) and their row scales
    uint16_t* h_out;         // up: H [P + T, h] bf16
    float* o_out;            // down: O [P + T, d] fp32
    int routed_weight;       // time of a routed tile in eighths of a shared one (xcd_tile)
    int tile_mode;           // kTilesAll, kTilesRouted or kTilesShared
};

// Which row tiles a grouped GEMM launch takes: every tile of the table; the
// table's routed tiles only; or the shared expert alone, in tiles of the
// launch's own height built from T (the table is not read).
constexpr int kTilesAll = 0;
constexpr int kTilesRouted = 1;
constexpr int kTilesShared = 2;

// K4 (routed) + K6a (shared): H = silu(A W1^T) * (A W3^T), one launch
hipError_t launch_grouped_up(const GroupedGemmArgs& args, hipStream_t stream);
// K5 (routed) + K6b (shared): O = H W2^T, one launch
hipError_t launch_grouped_down(const GroupedGemmArgs& args, hipStream_t stream);
// the same two launches with 256 x 256 tiles (tile table of kPrefillBM2 rows;
// int4, bf16 or fp8 routed experts; with kTilesShared, the shared expert alone)
hipError_t launch_grouped_up256(const GroupedGemmArgs& args, hipStream_t stream);
hipError_t launch_grouped_down256(const GroupedGemmArgs& args, hipStream_t stream);

struct DecodeArgs {
    const uint16_t* a;       // up: x [T, d]; down: H [P + T, h]
    const uint16_t* a_perm;  // routed-expert A rows, 8-blocks interleaved (up: x_perm; down: H)
    int64_t T;
    int64_t P;
    int top_k;
    int E;
    int64_t K;               // reduction dim
    int64_t N;               // output features
    int spt;                 // int4 scales per tile row: 128 / group (1, 2 or 4)
    const int32_t* perm;
    const int4* chunks;      // (group, first row, rows, 0); rows index H / O
    const int32_t* nchunks;
    const uint8_t* wq0;
    const float* ws0;
    const uint8_t* wq1;
    const float* ws1;
    const uint16_t* sh0;
    const uint16_t* sh1;
    const uint16_t* wb0;     // bf16 routed experts instead of int4 (null: int4)
    const uint16_t* wb1;
    const uint8_t* wf0;      // fp8 routed experts instead of int4 (null: int4)
    const uint8_t* wf1;
    const float* wfs0;
    const float* wfs1;
    const uint8_t* a8;       // fp8 routed A rows (up: x_q by token, down: H_q by slot)
    const float* a8s;
    uint16_t* h_out;
    float* o_out;
    float* o_out2;           // down: second half of the reduction's partial sums (null: no split)
    int sliced;              // int4 groups of 128: larger chunks stage A in LDS slices
    int lds_rows;            // set by the launcher: routed chunks this small stage A in LDS
    int max_chunks;          // set by the launcher: grid rows of the chunk list
};

// K7: decode up / down projections over the row chunks
hipError_t launch_decode_up(const DecodeArgs& a, int max_chunks, int shared_chunks,
                            hipStream_t stream);
hipError_t launch_decode_down(const DecodeArgs& a, int max_chunks, int shared_chunks,
                              hipStream_t stream);

// Measurement kernels (stream.hip): read every 16-byte word of buf (bytes % 16
// == 0) and write one XOR per block to sink[block] (kStreamBlocks words at most),
// or copy bytes from src to dst
constexpr int kStreamBlocks = 32768;  // best of 1024-32768 in a sweep of the read
unsigned stream_blocks(int64_t n16);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);

// K6c: y[t] = O[P + t] + sum_j gate[t, j] * O[inv[t, j]]  -> bf16
// (O2 non-null: the down projection's second partial sums, added to O first)
hipError_t launch_combine(const float* O, const float* O2, const float* gates, const int32_t* inv,
                          int64_t T, int64_t P, int top_k, int64_t d, uint16_t* y, hipStream_t stream);

}  // namespace moe
