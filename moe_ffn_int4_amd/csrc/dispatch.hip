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
//   chunks       row chunks (group, first row, rows) of at most kDecodeRows
//                rows for the streaming kernel, and their number in *nchunks
//                (which groups are chunked and which tiled: build_work_lists)
// One block per expert. Each block histograms all P ids in LDS, scans, and
// compacts the pairs of its own expert: every thread owns a contiguous segment
// of pairs, counts its matches, takes its base from a block-wide exclusive
// scan and writes its matches in order. The result is the stable counting sort
// whatever order the atomics land in. Integer work, a few microseconds.
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

// 32 consecutive ids of [p0, hi) (-1 past hi), loaded 16 bytes at a time so
// the loads are in flight together
__device__ __forceinline__ void load32(const int32_t* __restrict__ ids, int64_t p0, int64_t hi,
                                       int* v) {
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
        if (p0 + j + 4 <= hi) {
            const int4 q = *reinterpret_cast<const int4*>(ids + p0 + j);
            v[j] = q.x;
            v[j + 1] = q.y;
            v[j + 2] = q.z;
            v[j + 3] = q.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[j + i] = (p0 + j + i < hi) ? ids[p0 + j + i] : -1;
        }
    }
}

__global__ __launch_bounds__(256) void dispatch_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                       int top_k, int E, int tile_rows,
                                                       int small_rows,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ tile_base,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ inv,
                                                       int4* __restrict__ chunks,
                                                       int32_t* __restrict__ nchunks) {
    __shared__ int hist[kMaxExperts];
    __shared__ int offs[kMaxExperts + 1];
    __shared__ int wave_tot[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int64_t P = T * top_k;
    const int e = blockIdx.x;
    // each thread owns a contiguous segment of pairs (a multiple of 4 long)
    const int64_t seg = ((P + 255) / 256 + 3) & ~static_cast<int64_t>(3);
    const int64_t lo = min(P, tid * seg);
    const int64_t hi = min(P, lo + seg);

    for (int i = tid; i < E; i += 256) hist[i] = 0;
    __syncthreads();
    int mine = 0;  // pairs of expert e in this thread's segment
    for (int64_t p0 = lo; p0 < hi; p0 += 32) {
        int v[32];
        load32(ids, p0, hi, v);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            if (v[j] >= 0) {
                atomicAdd(&hist[v[j]], 1);
                mine += v[j] == e;
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < E; ++i) {
            offs[i] = run;
            run += hist[i];
        }
        offs[E] = run;
        if (e == 0) build_work_lists(hist, offs, E, T, P, tile_rows, small_rows, tile_base, chunks, nchunks);
    }
    __syncthreads();
    if (e == 0) {
        for (int i = tid; i < E; i += 256) {
            counts[i] = hist[i];
            offsets[i] = offs[i];
        }
        if (tid == 0) offsets[E] = offs[E];
    }
    if (hist[e] == 0) return;  // block-uniform

    // stable compaction of the pairs routed to expert e: exclusive scan of the
    // per-thread match counts gives each segment its first slot
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    int slot = offs[e] + incl - mine;
    for (int w = 0; w < wid; ++w) slot += wave_tot[w];
    if (mine == 0) return;
    for (int64_t p0 = lo; p0 < hi; p0 += 32) {
        int v[32];
        load32(ids, p0, hi, v);
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            if (v[j] == e) {
                perm[slot] = static_cast<int32_t>(p0 + j);
                inv[p0 + j] = slot;
                ++slot;
            }
        }
    }
}

hipError_t launch_dispatch(const int32_t* ids, int64_t T, int top_k, int64_t E, int tile_rows,
                           int small_rows, int32_t* counts, int32_t* offsets, int32_t* tile_base, int32_t* perm,
                           int32_t* inv, int4* chunks, int32_t* nchunks, hipStream_t stream) {
    MOE_LAUNCH(dispatch_kernel, dim3(static_cast<unsigned>(E)), dim3(256), 0, stream, ids,
                       T, top_k, static_cast<int>(E), tile_rows, small_rows, counts, offsets, tile_base, perm,
                       inv, chunks, nchunks);
    return hipGetLastError();
}

}  // namespace moe
