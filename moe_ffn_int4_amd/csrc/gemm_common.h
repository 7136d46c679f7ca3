// gemm_common.h -- pieces shared by the grouped GEMM kernels (gemm.hip, gemm256.hip).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// Row tile `mt` of the dispatch step's tile table (tile_base, BM rows per
// tile): its group (routed experts 0..E-1, the shared expert E), first row and
// row count. False past the last tile.
struct Tile {
    int group;
    int64_t row0;
    int nrows;
};

template <int BM>
__device__ __forceinline__ bool find_tile(const GroupedGemmArgs& a, int mt, Tile& t) {
    const int G = a.E + 1;
    if (mt >= a.tile_base[G]) return false;
    int lo = 0, hi = G;  // tile_base[lo] <= mt < tile_base[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.tile_base[mid] <= mt) lo = mid;
        else hi = mid;
    }
    const int local = mt - a.tile_base[lo];
    int64_t start, count;
    if (lo < a.E) {
        start = a.offsets[lo];
        count = a.counts[lo];
    } else {
        start = a.P;
        count = a.T;
    }
    t.group = lo;
    t.row0 = start + static_cast<int64_t>(local) * BM;
    const int64_t left = count - static_cast<int64_t>(local) * BM;
    t.nrows = static_cast<int>(left < BM ? left : BM);
    return true;
}

// Block -> tile position for the grouped GEMMs. Blocks are dealt to the 8
// XCDs round robin (block L runs on XCD L % 8), and each XCD takes a
// contiguous range of tile positions, so the tiles it runs at once share A and
// B panels in its L2. The tile table lists the routed experts' tiles first and
// the shared expert's after them, and the two kinds differ in cost (int4
// routed tiles dequantize their weights; fp8 ones run the fp8 instruction), so
// the ranges are cut by estimated time, not by count: a routed tile weighs
// `wr`, a shared one kSharedTileWeight. Blocks past their XCD's range return
// false; the grid has slots for the largest range (xcd_grid).
constexpr int kSharedTileWeight = 8;
__host__ __device__ inline int64_t tile_weight(const GroupedGemmArgs& a) {
    return a.routed_weight > 0 ? a.routed_weight : kSharedTileWeight;
}

__device__ __forceinline__ bool xcd_tile(int L, int64_t routed, int64_t total, int64_t wr, int& lin) {
    constexpr int kXcd = 8;
    const int xcd = L % kXcd, slot = L / kXcd;
    const int64_t cr = routed * wr;
    const int64_t cost = cr + (total - routed) * kSharedTileWeight;
    // first tile of the XCD whose share of the cost starts at c
    auto tile_at = [&](int64_t c) {
        return c <= cr ? (c + wr - 1) / wr : routed + (c - cr + kSharedTileWeight - 1) / kSharedTileWeight;
    };
    const int64_t first = tile_at(cost * xcd / kXcd);
    if (first + slot >= tile_at(cost * (xcd + 1) / kXcd)) return false;
    lin = static_cast<int>(first + slot);
    return true;
}

// blocks for at most max_tiles tiles: an XCD's share of the cost is at most
// max_tiles * max weight / 8, in tiles of the lighter kind, plus one for rounding
inline unsigned xcd_grid(int64_t max_tiles, int64_t wr) {
    const int64_t wmax = wr > kSharedTileWeight ? wr : kSharedTileWeight;
    const int64_t wmin = wr < kSharedTileWeight ? wr : kSharedTileWeight;
    return static_cast<unsigned>(8 * ((max_tiles * wmax + 8 * wmin - 1) / (8 * wmin) + 1));
}

// A 128-column group spans four 32-wide reduction steps, so step k of a
// 16-row tile column starts k * 256 bytes (int4: 1 KB tiles) or k * 512 bf16
// elements (4 KB tiles) after its first tile, and its int4 scale (128 / group
// per tile row: spt) step_scale(k, spt) floats after the row's first.
static_assert(kGroup == 128, "four 32-wide steps per group");
__device__ __forceinline__ int step_scale(int k, int spt) {
    return (k >> 2) * 16 * spt + (((k & 3) * spt) >> 2);
}

// 8 int4 codes (one 32-bit word) times scale -> 4 packed bf16 pairs (RNE)
__device__ __forceinline__ u32x4 dequant8(uint32_t w, float s) {
    // The sign bit of every nibble flipped gives u = code + 8 in 0..15; the
    // even nibbles go to bytes 0..3 of lo, the odd ones to those of hi. The
    // fma forms u * s - 8 s with one rounding: the exact value is code * s
    // (8 s is exact), so each result is the fp32 product code * s (for the
    // quantizer's positive scales bit for bit; a zero or negative scale can
    // turn a -0 product into +0).
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const uint32_t x = w ^ 0x88888888u;
    uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
    // opaque to the optimizer, so each byte converts with v_cvt_f32_ubyte0..3
    // instead of a 4-bit field extract and a conversion
    asm("" : "+v"(lo), "+v"(hi));
    const float off = -8.0f * s;
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float a = static_cast<float>((lo >> (8 * j)) & 0xFFu);
        const float b = static_cast<float>((hi >> (8 * j)) & 0xFFu);
        const bf16x2 v = {static_cast<__bf16>(__builtin_fmaf(a, s, off)),
                          static_cast<__bf16>(__builtin_fmaf(b, s, off))};
        o[j] = __builtin_bit_cast(uint32_t, v);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

// MFMA fragment order of a 16-row x 32-column bf16 sub-tile (1 KB): the
// 16-byte piece (row n, columns 8q .. 8q+7) sits at slot 16 q + (n ^ 2q).
// Bank groups on gfx950, fitted to SQ_LDS_BANK_CONFLICT counts of probe
// kernels: a 16-byte write is served 8 consecutive lanes at a time, a 16-byte
// read 16 lanes at a time, the 16 sharing lane bit 5 and the parity of lane
// bits 2..4. With c[q] = 2q the staging write (lane -> n = lane / 4, q =
// lane % 4) sees c[q] distinct in bits 1..2, and the fragment read (lane ->
// n = lane % 16, q = lane / 16) sees the parity of bits 2..3 of c[q] equal
// for q = 0, 1 and for q = 2, 3: each group touches distinct banks. (The
// former c = {0, 4, 10, 14} cost every fragment read 4 extra cycles.) The
// dequantization write (lane -> n = lane % 16, q fixed) permutes 16 slots
// for any c.
__device__ __forceinline__ int frag_slot(int n, int q) {
    return (q * 16 + (n ^ (q * 2))) * 16;  // bytes in a sub-tile
}

}  // namespace moe
