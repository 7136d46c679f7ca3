// plan.h -- the work lists of the expert projections, built from the expert
// pair counts by one thread of the routing step (E <= 256 entries: a few
// microseconds at most).
#pragma once
#include "kernels.h"

namespace moe {

// hist[e]: pairs routed to expert e; offs[e]: first slot of expert e.
// tile_base[g]: first GEMM row tile (tile_rows rows) of group g; routed experts
//   are groups 0..E-1, the shared expert (all T tokens) is group E;
//   tile_base[E+1] = total tiles.
// chunks / *nchunks: decode row chunks (group, first H/O row, rows, 0) of at
//   most kDecodeRows rows.
// small_rows < 0 (streaming decode path): every group is chunked, the shared
//   expert first; the tile table is unused.
// small_rows >= 0: routed experts with 1..small_rows pairs are chunked and get
//   no GEMM tiles; every other group is tiled (small_rows = 0: GEMMs only).
__device__ inline void build_work_lists(const int* hist, const int* offs, int E, int64_t T,
                                        int64_t P, int tile_rows, int small_rows,
                                        int32_t* tile_base, int4* chunks, int32_t* nchunks) {
    int tiles = 0, n = 0;
    if (small_rows < 0) {
        for (int64_t r = 0; r < T; r += kDecodeRows)
            chunks[n++] = make_int4(E, static_cast<int>(P + r),
                                    static_cast<int>(T - r < kDecodeRows ? T - r : kDecodeRows), 0);
    }
    for (int e = 0; e < E; ++e) {
        tile_base[e] = tiles;
        const int c = hist[e];
        const bool chunked = small_rows < 0 || (c > 0 && c <= small_rows);
        if (chunked) {
            for (int r = 0; r < c; r += kDecodeRows)
                chunks[n++] = make_int4(e, offs[e] + r, c - r < kDecodeRows ? c - r : kDecodeRows, 0);
        }
        if (small_rows < 0 || !chunked) tiles += (c + tile_rows - 1) / tile_rows;
    }
    tile_base[E] = tiles;
    tile_base[E + 1] = tiles + static_cast<int>((T + tile_rows - 1) / tile_rows);
    *nchunks = n;
}

}  // namespace moe
