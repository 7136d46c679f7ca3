// dispatch.hip -- K3: token -> expert dispatch for the grouped GEMMs (gfx950).
//
// The discosf.com page "1 卡跑通 Llama 4" (section "混合专家路由") has each
// chosen expert compute only on its own tokens and scatter its output back.
// The pages leave the index structure open; this kernel builds a counting
// sort of the (token, slot) pairs by expert:
//   counts[e]    pairs routed to expert e
//   offsets[e]   exclusive prefix sum of counts (offsets[E] = P)
//   perm[slot]   pair p = t * top_k + j, slots of expert e contiguous and the
//                pairs inside them ascending (stable: deterministic order)
//   inv[p]       slot of pair p (perm o inv = identity)
//   tile_base[g] first GEMM row-tile of group g for tiles of `tile_rows`
//                rows: routed experts are groups 0..E-1, the shared expert
//                (all T tokens) is group E; tile_base[E+1] = total tiles.
// One block per expert. Each block histograms all P ids in LDS, scans, and
// compacts the pairs of its own expert with wave ballots, so the result does
// not depend on the order atomics land in. Integer work, a few microseconds.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void dispatch_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                       int top_k, int E, int tile_rows,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ tile_base,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv) {
    __shared__ int hist[kMaxExperts];
    __shared__ int offs[kMaxExperts + 1];
    __shared__ int wave_tot[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int64_t P = T * top_k;
    const int e = blockIdx.x;

    for (int i = tid; i < E; i += 256) hist[i] = 0;
    __syncthreads();
    for (int64_t p = tid; p < P; p += 256) atomicAdd(&hist[ids[p]], 1);
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < E; ++i) {
            offs[i] = run;
            run += hist[i];
        }
        offs[E] = run;
        if (e == 0) {
            int tiles = 0;
            for (int i = 0; i < E; ++i) {
                tile_base[i] = tiles;
                tiles += (hist[i] + tile_rows - 1) / tile_rows;
            }
            tile_base[E] = tiles;
            tile_base[E + 1] = tiles + static_cast<int>((T + tile_rows - 1) / tile_rows);
        }
    }
    __syncthreads();
    if (e == 0) {
        for (int i = tid; i < E; i += 256) {
            counts[i] = hist[i];
            offsets[i] = offs[i];
        }
        if (tid == 0) offsets[E] = offs[E];
    }
    if (hist[e] == 0) return;

    // stable compaction of the pairs routed to expert e
    int running = offs[e];
    for (int64_t c0 = 0; c0 < P; c0 += 256) {
        const int64_t p = c0 + tid;
        const bool flag = p < P && ids[p] == e;
        const unsigned long long mask = __ballot(flag);
        const int rank_in_wave = __popcll(mask & ((1ull << lane) - 1ull));
        if (lane == 0) wave_tot[wid] = __popcll(mask);
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wid; ++w) before += wave_tot[w];
        const int total = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
        if (flag) {
            const int slot = running + before + rank_in_wave;
            perm[slot] = static_cast<int32_t>(p);
            inv[p] = slot;
        }
        running += total;
        __syncthreads();
        if (running == offs[e] + hist[e]) break;  // block-uniform
    }
}

hipError_t launch_dispatch(const int32_t* ids, int64_t T, int top_k, int64_t E, int tile_rows,
                           int32_t* counts, int32_t* offsets, int32_t* tile_base, int32_t* perm,
                           int32_t* inv, hipStream_t stream) {
    hipLaunchKernelGGL(dispatch_kernel, dim3(static_cast<unsigned>(E)), dim3(256), 0, stream, ids,
                       T, top_k, static_cast<int>(E), tile_rows, counts, offsets, tile_base, perm,
                       inv);
    return hipGetLastError();
}

}  // namespace moe
