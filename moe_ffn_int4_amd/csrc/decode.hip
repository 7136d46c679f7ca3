// decode.hip -- K7: HBM-streaming expert FFN for small batches (gfx950).
//
// In generation each step brings one new token per sequence (lshu.cn page,
// section "数据流"), so a decode batch is a handful of tokens: every touched
// expert's weights are streamed from HBM once and used for only its few
// tokens. This path reads each weight byte exactly once and is bound by HBM
// bandwidth.
//
// Work: row chunks (<= 16 token rows of one group: the shared expert first,
// the largest work item, then routed experts in id order) from the routing
// step, times blocks of 64 output features. A 256-thread block is 4 waves.
// For int4 and fp8 experts each wave owns 16 output features and streams them
// over the whole reduction dimension on its own, keeping the next tiles'
// loads in flight in a register ring; chunks of a few rows first stage their
// A rows in LDS once per block, and larger int4 chunks stage them in LDS
// slices along the reduction (the SL instantiation, chosen by the host for
// batches averaging 4+ pairs per expert). bf16 chunks (the shared expert, bf16 experts)
// carry four times the bytes of int4: four blocks share a 64-feature range,
// each wave of a block streams a quarter of the reduction, and the four
// partial sums are added in LDS in wave order. v_mfma_f32_16x16x32_bf16 takes
// the chunk's tokens as its 16 rows (rows past the chunk repeat its last row;
// their outputs are not stored) and the features as its 16 columns.
//
// Weights come in the tiled layouts of moe_quantize_int4_tiled /
// moe_pack_bf16_tiled / moe_quantize_fp8_tiled, so every weight access of a
// wave is one contiguous 1 KB block of a tile (int4 scales: 64 B per 16 rows
// and scale column), read with non-temporal loads.
// Int4 weights (routed experts): per 128-wide tile a lane streams one 16-byte
// piece (32 codes) of its feature's row. Codes become bf16 (128 + u),
// u = code + 8, by placing offset-binary nibbles into the bit pattern of 128.0
// (about one VALU op per code; gfx950 has no packed bf16 add to remove the
// offset). The offset is removed exactly by one extra MFMA per 32-wide step
// against a constant B of -136 (shared by W1 and W3): a group's accumulator
// starts at -136 * sum(a) and gains sum a * (128 + u) = sum a * code
// + 136 * sum a. The group's fp32 scale multiplies the fp32 group accumulator,
// so the weights reach the matrix cores exact.
// The nibble trick emits pairs in the order (0,4) (1,5) (2,6) (3,7) of each
// 8 codes, so the A rows of routed experts are stored with their 8-element
// blocks in that order: x by the router kernel (x_perm), H by this kernel's
// up-projection epilogue. bf16 weights (the shared expert) use natural order.
// Groups of 64 or 32 weights (S = 2 or 4 scales per 128-column tile row): one
// MFMA step must then stay inside one group, but a lane's 16 bytes hold 32
// consecutive codes, and the four kq lanes of a step would span four groups.
// A 4 x 4 transpose of the lanes' words across the four 16-lane rows
// (v_permlane32_swap, then v_permlane16_swap) gives lane kq the words
// kq, 4 + kq, 8 + kq, 12 + kq of its feature's row instead: step i then covers
// columns 32 i .. 32 i + 31 of the tile (one group of 32, or half of one of 64),
// the A row is read at 32 i + 8 kq, and each group's accumulator takes its
// own scale.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int NT = 256;
constexpr int kStagePieces = 4;  // A pieces per thread requested together when staging
constexpr uint32_t kMagic = 0x43004300u;   // bf16 128.0 in both halves
constexpr uint32_t kNeg136 = 0xC308C308u;  // bf16 -136.0 in both halves
}  // namespace

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Weights are read exactly once: non-temporal loads keep them from displacing
// the reused activations in the vector L1.
__device__ __forceinline__ uint4 ld_stream(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ld_stream_f(const float* p) { return __builtin_nontemporal_load(p); }

// 8 two's-complement nibbles -> bf16 pairs (128 + u) in the order 0,4 | 1,5 | 2,6 | 3,7.
// u = code ^ 8 and the OR of 128.0 are one XOR with kMagic | 0x00080008 on the
// masked nibbles (the magic's bits and the nibbles' do not overlap), so each
// pair is a shift and one three-input bit operation.
__device__ __forceinline__ uint4 offset_bf16(uint32_t w) {
    constexpr uint32_t kFlip = kMagic | 0x00080008u;
    uint4 r;
    r.x = (w & 0x000F000Fu) ^ kFlip;
    r.y = ((w >> 4) & 0x000F000Fu) ^ kFlip;
    r.z = ((w >> 8) & 0x000F000Fu) ^ kFlip;
    r.w = ((w >> 12) & 0x000F000Fu) ^ kFlip;
    return r;
}

// S scales per 128-column tile row of an int4 weight: 128 / group
template <int S>
struct RoutedSlot {
    uint4 w0, w1;
    float s0[S], s1[S];
    uint4 a[4];
};

template <int S>
struct WeightSlot {
    uint4 w0, w1;
    float s0[S], s1[S];
};

// this lane's S scales of tile g: one float, or an aligned float2 / float4
template <int S>
__device__ __forceinline__ void load_scales(float (&d)[S], const float* s, int g) {
    if constexpr (S == 1) {
        d[0] = ld_stream_f(s + g * 16);
    } else {
        typedef float fv __attribute__((ext_vector_type(S)));
        const fv v = __builtin_nontemporal_load(reinterpret_cast<const fv*>(s + g * 16 * S));
#pragma unroll
        for (int j = 0; j < S; ++j) d[j] = v[j];
    }
}

// word j of lane (n, row r) -> word r of lane (n, row j), rows of 16 lanes
__device__ __forceinline__ uint4 transpose_rows(uint4 v) {
    // rows 0-1 x words 2-3 <-> rows 2-3 x words 0-1
    const auto p = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
    const auto q = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
    // odd rows x even words <-> even rows x odd words
    const auto r = __builtin_amdgcn_permlane16_swap(p[0], q[0], false, false);
    const auto t = __builtin_amdgcn_permlane16_swap(p[1], q[1], false, false);
    return make_uint4(r[0], r[1], t[0], t[1]);
}

struct SharedSlot {
    uint4 b0[4], b1[4];
    uint4 a[4];
};

// A column step of MFMA step i: this lane's 8 columns sit at 8 i (S = 1: the
// lane's 32 columns are contiguous) or at 32 i (S > 1: after the transpose)
template <int S>
constexpr int a_step() { return S == 1 ? 8 : 32; }

// tile g of this lane's piece of a 16-row int4 tile (1 KB per tile) and its scales
template <bool UP, int S>
__device__ __forceinline__ void load_routed(RoutedSlot<S>& sl, const uint8_t* q0, const uint8_t* q1,
                                            const float* s0, const float* s1, const uint16_t* arow,
                                            int g) {
    sl.w0 = ld_stream(q0 + g * 1024);
    load_scales<S>(sl.s0, s0, g);
    if (UP) {
        sl.w1 = ld_stream(q1 + g * 1024);
        load_scales<S>(sl.s1, s1, g);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sl.a[i] = *reinterpret_cast<const uint4*>(arow + g * kGroup + i * a_step<S>());
}

// S > 1: group j of the tile covers MFMA steps 4j/S .. 4(j+1)/S - 1 and has
// its own -136 correction, accumulator and scale
template <bool UP, int S>
__device__ __forceinline__ void compute_groups(const RoutedSlot<S>& sl, f32x4& acc0, f32x4& acc1) {
    constexpr int SPG = 4 / S;  // MFMA steps per group
    const bf16x8 neg136 = as_bf16x8(make_uint4(kNeg136, kNeg136, kNeg136, kNeg136));
    const uint4 t0 = transpose_rows(sl.w0);
    const uint32_t w0[4] = {t0.x, t0.y, t0.z, t0.w};
    uint32_t w1[4] = {0u, 0u, 0u, 0u};
    if (UP) {
        const uint4 t1 = transpose_rows(sl.w1);
        w1[0] = t1.x;
        w1[1] = t1.y;
        w1[2] = t1.z;
        w1[3] = t1.w;
    }
#pragma unroll
    for (int j = 0; j < S; ++j) {
        f32x4 corr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = j * SPG; i < (j + 1) * SPG; ++i)
            corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sl.a[i]), neg136, corr, 0, 0, 0);
        f32x4 g0 = corr;
#pragma unroll
        for (int i = j * SPG; i < (j + 1) * SPG; ++i)
            g0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sl.a[i]),
                                                         as_bf16x8(offset_bf16(w0[i])), g0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc0[r] = fmaf(sl.s0[j], g0[r], acc0[r]);
        if (UP) {
            f32x4 g1 = corr;
#pragma unroll
            for (int i = j * SPG; i < (j + 1) * SPG; ++i)
                g1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sl.a[i]),
                                                             as_bf16x8(offset_bf16(w1[i])), g1, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc1[r] = fmaf(sl.s1[j], g1[r], acc1[r]);
        }
    }
}

template <bool UP, int S>
__device__ __forceinline__ void compute_routed(const RoutedSlot<S>& sl, f32x4& acc0, f32x4& acc1) {
    if constexpr (S > 1) {
        compute_groups<UP, S>(sl, acc0, acc1);
        return;
    }
    const bf16x8 neg136 = as_bf16x8(make_uint4(kNeg136, kNeg136, kNeg136, kNeg136));
    f32x4 corr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sl.a[i]), neg136, corr, 0, 0, 0);
    const uint32_t w0[4] = {sl.w0.x, sl.w0.y, sl.w0.z, sl.w0.w};
    f32x4 g0 = corr;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        g0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sl.a[i]), as_bf16x8(offset_bf16(w0[i])),
                                                     g0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc0[r] = fmaf(sl.s0[0], g0[r], acc0[r]);
    if (UP) {
        const uint32_t w1[4] = {sl.w1.x, sl.w1.y, sl.w1.z, sl.w1.w};
        f32x4 g1 = corr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            g1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sl.a[i]),
                                                         as_bf16x8(offset_bf16(w1[i])), g1, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc1[r] = fmaf(sl.s1[0], g1[r], acc1[r]);
    }
}

// group g of a step-major bf16 tile (4 steps x 16 rows x 32 columns, 4 KB):
// step i is 1 KB, this lane's piece is row l16, columns 8*kq .. 8*kq+7
template <bool UP, int S>
__device__ __forceinline__ void load_weights(WeightSlot<S>& sl, const uint8_t* q0, const uint8_t* q1,
                                             const float* s0, const float* s1, int g) {
    sl.w0 = ld_stream(q0 + g * 1024);
    load_scales<S>(sl.s0, s0, g);
    if (UP) {
        sl.w1 = ld_stream(q1 + g * 1024);
        load_scales<S>(sl.s1, s1, g);
    }
}

// one int4 tile with A fragments from LDS (row `lrow` of the staged chunk)
template <bool UP, int S>
__device__ __forceinline__ void compute_lds(const WeightSlot<S>& w, const uint16_t* lrow, int g,
                                            f32x4& acc0, f32x4& acc1) {
    RoutedSlot<S> sl;
    sl.w0 = w.w0;
    sl.w1 = w.w1;
#pragma unroll
    for (int j = 0; j < S; ++j) {
        sl.s0[j] = w.s0[j];
        sl.s1[j] = w.s1[j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sl.a[i] = *reinterpret_cast<const uint4*>(lrow + g * kGroup + i * a_step<S>());
    compute_routed<UP, S>(sl, acc0, acc1);
}

template <bool UP>
__device__ __forceinline__ void load_shared(SharedSlot& sl, const uint16_t* h0, const uint16_t* h1,
                                            const uint16_t* arow, int g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sl.b0[i] = ld_stream(h0 + g * 2048 + i * 512);
        if (UP) sl.b1[i] = ld_stream(h1 + g * 2048 + i * 512);
        sl.a[i] = *reinterpret_cast<const uint4*>(arow + g * kGroup + i * 32);
    }
}

template <bool UP>
__device__ __forceinline__ void compute_shared(const SharedSlot& sl, f32x4& acc0, f32x4& acc1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sl.a[i]), as_bf16x8(sl.b0[i]), acc0,
                                                       0, 0, 0);
        if (UP)
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(sl.a[i]), as_bf16x8(sl.b1[i]),
                                                           acc1, 0, 0, 0);
    }
}

// fp8 routed experts: per 128-wide group a lane holds 32 weight bytes of its
// feature's row and the same 32 columns of its A row. Load j (j = 0, 1) of a
// wave reads 1 KB of the 2 KB tile (steps 2j, 2j + 1): lane (l16, kq) takes
// step 2j + kq / 2, bytes 16 (kq % 2) .. + 15, i.e. columns
// 32 (2j + kq / 2) + 16 (kq % 2) .. + 15 of the group. MFMA step i pairs byte
// 8i .. 8i + 7 of both operands; the four kq lanes of a feature together cover
// the group's 128 columns once, so the sum is the same dot product.
struct Fp8Slot {
    uint4 w0[2], w1[2];
    uint4 a[2];
};

template <bool UP>
__device__ __forceinline__ void load_fp8(Fp8Slot& sl, const uint8_t* q0, const uint8_t* q1,
                                         const uint8_t* arow, int g, int boff0, int aoff0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        sl.w0[j] = ld_stream(q0 + g * 2048 + boff0 + j * 1024);
        if (UP) sl.w1[j] = ld_stream(q1 + g * 2048 + boff0 + j * 1024);
        sl.a[j] = *reinterpret_cast<const uint4*>(arow + g * kGroup + aoff0 + j * 64);
    }
}

template <bool UP>
__device__ __forceinline__ void compute_fp8(const Fp8Slot& sl, f32x4& acc0, f32x4& acc1) {
    typedef long long2v __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const long2v av = __builtin_bit_cast(long2v, sl.a[j]);
        const long2v b0 = __builtin_bit_cast(long2v, sl.w0[j]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av[h], b0[h], acc0, 0, 0, 0);
        if (UP) {
            const long2v b1 = __builtin_bit_cast(long2v, sl.w1[j]);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av[h], b1[h], acc1, 0, 0, 0);
        }
    }
}

// Sliced A staging for routed chunks of more rows than fit whole in LDS: a
// slice is half a round of the LDS path's weight ring ((DL + 1) / 2 groups;
// a whole round when DL + 1 is odd). Two slices of 16 rows then fit the LDS
// the kernel already takes (25 KB up, 33.3 KB down at groups of 128), and the
// staging registers stay within the up projection's three waves per SIMD.
constexpr int slice_groups(bool up, int dl) { return (dl + 1) % 2 == 0 ? (dl + 1) / 2 : dl + 1; }
constexpr size_t slice_lds_bytes(int sg) { return 2 * size_t(kDecodeRows) * (sg * kGroup + 8) * 2; }

// slice j of the chunk's A rows into registers: this thread's PP 16-byte pieces
// (source row start, column in the slice); past the last slice, the last
// slice again; columns past K (a partial last slice) re-read column K - 8
template <int PP, int SG>
__device__ __forceinline__ void slice_load(uint4 (&pv)[PP], const uint16_t* const (&psrc)[PP],
                                           const int (&pcol)[PP], int j, int nsl, int64_t K) {
    j = j < nsl ? j : nsl - 1;
    const int64_t c0 = static_cast<int64_t>(j) * SG * kGroup;
#pragma unroll
    for (int p = 0; p < PP; ++p) {
        const int64_t col = c0 + pcol[p] < K ? c0 + pcol[p] : K - 8;
        pv[p] = *reinterpret_cast<const uint4*>(psrc[p] + col);
    }
}

template <int PP>
__device__ __forceinline__ void slice_store(const uint4 (&pv)[PP], const int (&pdst)[PP], uint16_t* buf) {
#pragma unroll
    for (int p = 0; p < PP; ++p) *reinterpret_cast<uint4*>(buf + pdst[p]) = pv[p];
}

// DR / DS: groups kept in flight ahead of the one being computed, for int4
// (routed) and bf16 (shared) weights
// F8: the routed experts are fp8 (a separate instantiation, so the int4 one
// keeps its register budget); S: int4 scales per 128-column tile row
// SL: int4 chunks of more rows than fit whole in LDS stage A in slices (groups
// of 128; chosen by the host for batches averaging 4+ pairs per expert)
template <bool UP, int DR, int DS, int DL, bool F8, int S, bool SL>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeArgs a) {
    // routed chunks of at most a.lds_rows rows keep their A rows in LDS
    extern __shared__ __attribute__((aligned(16))) uint16_t a_lds[];
    // Rows 0 .. max_chunks-1 of the grid take the chunks; chunks of bf16 weights
    // at the head of the list (the shared expert's, or all of them when the
    // routed experts are bf16) get three more rows each (max_chunks + 3 c + s - 1):
    // sub-block s = 0..3 of a 64-feature range covers its 16 features
    // s*16 .. s*16+15 with all four waves, each wave a quarter of the reduction.
    // bf16 chunks stream 4x the bytes of an int4 chunk; split this way they
    // spread over four times as many blocks and CUs.
    int c = blockIdx.y, sub = 0;
    if (c >= a.max_chunks) {
        const int e = c - a.max_chunks;
        c = e / 3;
        sub = 1 + e % 3;
    }
    if (c >= *a.nchunks) return;
    const int4 ch = a.chunks[c];
    const int group = ch.x, row0 = ch.y, nrows = ch.z;
    const bool routed = group < a.E;
    const bool fp8 = F8 && routed;
    const bool int4 = !F8 && routed && !a.wb0;  // otherwise bf16 weights (shared, or bf16 routed)
    const bool narrow = int4 || fp8;              // one wave per 16 features, whole reduction
    if (narrow && blockIdx.y >= a.max_chunks) return;
    const int64_t K = a.K, N = a.N;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kq = lane >> 4;
    // Reduction split (the host's second output, down projection, int4 weights
    // of any group size; the same condition as the launcher): the two halves of a
    // feature range are adjacent blocks in x, so the blocks dispatched
    // together read both halves of the same row blocks of the weights
    // (measured on the Scout decode layer: down 54.7 -> 52.8 us against
    // halves in grid z).
    const int nkz = (!UP && !F8 && !SL && a.o_out2) ? 2 : 1;
    const int kz = static_cast<int>(blockIdx.x) % nkz;
    const int64_t n = static_cast<int64_t>(blockIdx.x / nkz) * 64 + (narrow ? wave : sub) * 16 + l16;  // B column
    const int ng = static_cast<int>(K / kGroup);
    // This block of the reduction split sums groups glo .. ghi - 1 and stores
    // its partial sums to o_out (kz = 0) or o_out2 (kz = 1), which the
    // combine adds.
    const int glo = (kz * ng) / nkz, ghi = ((kz + 1) * ng) / nkz, ngl = ghi - glo;  // ngl may be 0

    // A row of MFMA row l16: int4 routed experts read the interleaved copy, bf16
    // weights the natural one. Rows past the chunk repeat its last row: their
    // outputs are never stored, and every lane then loads unconditionally, which
    // keeps the load counter of the prefetch ring exact. Step i of group g uses
    // columns 128g + 32kq + 8i.. (int4: this lane's 32 codes) or 128g + 32i + 8kq..
    // (bf16 step-major tiles).
    const int m = l16 < nrows ? l16 : nrows - 1;
    int64_t src;
    if (UP) src = routed ? a.perm[row0 + m] / a.top_k : row0 + m - a.P;
    else src = row0 + m;
    const uint16_t* arow = (int4 ? a.a_perm : a.a) + src * K + ((int4 && S == 1) ? kq * 32 : kq * 8);

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    if (fp8) {
        constexpr int D = DR;
        constexpr int U = D + 1;
        const int64_t mat = static_cast<int64_t>(group) * N * K;
        const int64_t tb = (n >> 4) * ng * 2048 + l16 * 32;  // this feature's row in its tiles
        const uint8_t* q0 = a.wf0 + mat + tb;
        const uint8_t* q1 = UP ? a.wf1 + mat + tb : nullptr;
        const int boff0 = (kq >> 1) * 512 + (kq & 1) * 16;
        const int aoff0 = (kq >> 1) * 32 + (kq & 1) * 16;
        const uint8_t* a8row = a.a8 + src * K;
        Fp8Slot sl[U];
#pragma unroll
        for (int p = 0; p < D; ++p) load_fp8<UP>(sl[p], q0, q1, a8row, min(p, ng - 1), boff0, aoff0);
        const int full = ng - ng % U;
        for (int g0 = 0; g0 < full; g0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                load_fp8<UP>(sl[(u + D) % U], q0, q1, a8row, min(g0 + u + D, ng - 1), boff0, aoff0);
                compute_fp8<UP>(sl[u], acc0, acc1);
            }
        }
#pragma unroll
        for (int u = 0; u < D; ++u)
            if (u < ng - full) compute_fp8<UP>(sl[u], acc0, acc1);
        // scale by both row scales; bf16 where the fp8 products return bf16
        const float w0s = a.wfs0[static_cast<int64_t>(group) * N + n];
        const float w1s = UP ? a.wfs1[static_cast<int64_t>(group) * N + n] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int mr = kq * 4 + r;
            if (mr >= nrows) continue;
            const int64_t orow = row0 + mr;
            const float sa = a.a8s[UP ? a.perm[orow] / a.top_k : orow];
            if (UP) {
                const float g = bf16_to_f32(f32_to_bf16(acc0[r] * sa * w0s));
                const float u = bf16_to_f32(f32_to_bf16(acc1[r] * sa * w1s));
                a.h_out[orow * N + n] = f32_to_bf16(siluf_(g) * u);
            } else {
                a.o_out[orow * N + n] = bf16_to_f32(f32_to_bf16(acc0[r] * sa * w0s));
            }
        }
        return;
    } else if (int4 && nrows <= a.lds_rows) {
        // Stage the chunk's A rows (interleaved copies) in LDS once; the weight
        // ring then carries only weights and scales, and A comes from LDS.
        constexpr int D = DL;
        constexpr int U = D + 1;
        const int64_t rb = static_cast<int64_t>(group) * (N / 16) + (n >> 4);
        const uint8_t* q0 = a.wq0 + rb * ng * 1024 + kq * 256 + l16 * 16;
        const uint8_t* q1 = UP ? a.wq1 + rb * ng * 1024 + kq * 256 + l16 * 16 : nullptr;
        const float* s0 = a.ws0 + (rb * ng * 16 + l16) * S;
        const float* s1 = UP ? a.ws1 + (rb * ng * 16 + l16) * S : nullptr;
        q0 += static_cast<int64_t>(glo) * 1024;  // this block's groups (z split)
        if (UP) q1 += static_cast<int64_t>(glo) * 1024;
        s0 += static_cast<int64_t>(glo) * 16 * S;
        if (UP) s1 += static_cast<int64_t>(glo) * 16 * S;
        WeightSlot<S> sl[U];
#pragma unroll
        for (int p = 0; p < D; ++p) load_weights<UP, S>(sl[p], q0, q1, s0, s1, min(p, ngl > 0 ? ngl - 1 : 0));
        // Only this block's columns (its groups glo .. ghi - 1 of the z split)
        // are staged, at their own positions; each thread requests
        // kStagePieces 16-byte pieces before storing any, so the staging takes
        // one or two memory round trips instead of one per piece.
        const int64_t pitch = K + 8;  // 16-byte pad between rows
        const int per_row = ngl * (kGroup / 8);
        const int pieces = nrows * per_row;  // at most 16 rows of K / 8 pieces
        for (int i0 = tid; i0 < pieces; i0 += kStagePieces * NT) {
            uint4 v[kStagePieces];
#pragma unroll
            for (int u = 0; u < kStagePieces; ++u) {
                // pieces past the end re-read the last one (not stored)
                const int idx = min(i0 + u * NT, pieces - 1);
                const int r = idx / per_row;
                const int col = glo * kGroup + (idx - r * per_row) * 8;
                const int64_t srow = UP ? a.perm[row0 + r] / a.top_k : row0 + r;
                v[u] = *reinterpret_cast<const uint4*>(a.a_perm + srow * K + col);
            }
#pragma unroll
            for (int u = 0; u < kStagePieces; ++u) {
                const int idx = i0 + u * NT;
                if (idx >= pieces) break;
                const int r = idx / per_row;
                const int col = glo * kGroup + (idx - r * per_row) * 8;
                *reinterpret_cast<uint4*>(a_lds + r * pitch + col) = v[u];
            }
        }
        __syncthreads();
        const uint16_t* lrow = a_lds + m * pitch + (S == 1 ? kq * 32 : kq * 8) + glo * kGroup;
        const int full = ngl - ngl % U;
        for (int g0 = 0; g0 < full; g0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                load_weights<UP, S>(sl[(u + D) % U], q0, q1, s0, s1, min(g0 + u + D, ngl - 1));
                compute_lds<UP, S>(sl[u], lrow, g0 + u, acc0, acc1);
            }
        }
#pragma unroll
        for (int u = 0; u < D; ++u)
            if (u < ngl - full) compute_lds<UP, S>(sl[u], lrow, full + u, acc0, acc1);
    } else if (int4 && SL) {
        // Chunks of more than lds_rows rows: the block stages A in slices of SG
        // groups (SG * 128 columns of the chunk's rows). Two slices sit in LDS:
        // slice j+1 goes from registers into the other buffer at the end of
        // slice j, one barrier per slice, and slice j+2 is then requested. The
        // weight ring is the LDS path's, and slices end at fixed ring
        // positions. (Each wave reading its A rows from L2 for its own 16
        // features moved rows / 4 times the weight bytes per wave.)
        constexpr int D = DL;
        constexpr int U = D + 1;
        constexpr int SG = slice_groups(UP, DL);
        static_assert(U % SG == 0, "slices end at fixed ring positions");
        constexpr int SW = SG * kGroup + 8;                // row pitch of a slice (16-byte pad)
        constexpr int PP = kDecodeRows * SG * 16 / NT;    // 16-byte pieces per thread per slice
        static_assert(PP * NT == kDecodeRows * SG * 16, "whole pieces per thread");
        const int64_t rb = static_cast<int64_t>(group) * (N / 16) + (n >> 4);
        const uint8_t* q0 = a.wq0 + rb * ng * 1024 + kq * 256 + l16 * 16;
        const uint8_t* q1 = UP ? a.wq1 + rb * ng * 1024 + kq * 256 + l16 * 16 : nullptr;
        const float* s0 = a.ws0 + (rb * ng * 16 + l16) * S;
        const float* s1 = UP ? a.ws1 + (rb * ng * 16 + l16) * S : nullptr;
        WeightSlot<S> sl[U];
#pragma unroll
        for (int p = 0; p < D; ++p) load_weights<UP, S>(sl[p], q0, q1, s0, s1, min(p, ng - 1));
        // piece tid + NT p of a slice: row pc / (16 SG), columns 8 (pc % (16 SG)) ..;
        // rows past the chunk repeat its last row (never read)
        const uint16_t* psrc[PP];
        int pcol[PP], pdst[PP];
#pragma unroll
        for (int p = 0; p < PP; ++p) {
            const int pc = tid + NT * p;
            const int r = pc / (SG * 16);
            pcol[p] = (pc % (SG * 16)) * 8;
            const int rr = r < nrows ? r : nrows - 1;
            const int64_t srow = UP ? a.perm[row0 + rr] / a.top_k : row0 + rr;
            psrc[p] = a.a_perm + srow * K;
            pdst[p] = r * SW + pcol[p];
        }
        const int nsl = (ng + SG - 1) / SG;
        uint4 pv[PP];
        uint16_t* const buf0 = a_lds;
        uint16_t* const buf1 = a_lds + kDecodeRows * SW;
        slice_load<PP, SG>(pv, psrc, pcol, 0, nsl, K);
        slice_store<PP>(pv, pdst, buf0);
        __syncthreads();
        const uint16_t* lbase = a_lds + m * SW + (S == 1 ? kq * 32 : kq * 8);
        // Slice s sits in buffer s % 2. A slice's first group requests the next
        // slice into registers; its last group stores it into the other buffer
        // (whose previous slice was last read before the previous barrier), then
        // a barrier. Rounds of U groups hold whole slices, so nothing is carried
        // in registers from one round to the next.
        const int full = ng - ng % U;
        for (int g0 = 0; g0 < full; g0 += U) {
            const int j0 = g0 / SG;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = j0 + u / SG;
                if (u % SG == 0) slice_load<PP, SG>(pv, psrc, pcol, j + 1, nsl, K);
                load_weights<UP, S>(sl[(u + D) % U], q0, q1, s0, s1, min(g0 + u + D, ng - 1));
                compute_lds<UP, S>(sl[u], lbase + (j & 1) * (kDecodeRows * SW), u % SG, acc0, acc1);
                if ((u + 1) % SG == 0) {
                    slice_store<PP>(pv, pdst, (j & 1) ? buf0 : buf1);
                    __syncthreads();
                }
            }
        }
        // the last ng % U groups (already in the ring): their first slice is in
        // LDS; a later one (only when a slice is shorter than a round) is staged
        // on the spot
#pragma unroll
        for (int u = 0; u < D; ++u) {
            if (u < ng - full) {
                const int g = full + u;
                const int j = g / SG;
                if (u > 0 && g % SG == 0) {
                    slice_load<PP, SG>(pv, psrc, pcol, j, nsl, K);
                    slice_store<PP>(pv, pdst, (j & 1) ? buf1 : buf0);
                    __syncthreads();
                }
                compute_lds<UP, S>(sl[u], lbase + (j & 1) * (kDecodeRows * SW), g % SG, acc0, acc1);
            }
        }
    } else if (int4) {
        // each wave reads its A rows from L2 with its weights (few rows per chunk,
        // or groups of 64 / 32, where the sliced staging's registers would cost
        // a wave per SIMD)
        constexpr int D = DR;
        constexpr int U = D + 1;
        // tile row block of this lane's feature; tiles of a row block are consecutive
        const int64_t rb = static_cast<int64_t>(group) * (N / 16) + (n >> 4);
        const uint8_t* q0 = a.wq0 + rb * ng * 1024 + kq * 256 + l16 * 16;
        const uint8_t* q1 = UP ? a.wq1 + rb * ng * 1024 + kq * 256 + l16 * 16 : nullptr;
        const float* s0 = a.ws0 + (rb * ng * 16 + l16) * S;
        const float* s1 = UP ? a.ws1 + (rb * ng * 16 + l16) * S : nullptr;
        // Ring of U slots, group g in slot g % U. Loads past the last group re-read
        // it (cache hits), so every loop iteration issues the same loads and the
        // compiler can wait on exact load counts; full rounds of U groups run
        // without guards, the last ng % U groups are already in their slots.
        q0 += static_cast<int64_t>(glo) * 1024;  // this block's groups (z split)
        if (UP) q1 += static_cast<int64_t>(glo) * 1024;
        s0 += static_cast<int64_t>(glo) * 16 * S;
        if (UP) s1 += static_cast<int64_t>(glo) * 16 * S;
        const uint16_t* arow_k = arow + glo * kGroup;
        RoutedSlot<S> sl[U];
#pragma unroll
        for (int p = 0; p < D; ++p) load_routed<UP, S>(sl[p], q0, q1, s0, s1, arow_k, min(p, ngl > 0 ? ngl - 1 : 0));
        const int full = ngl - ngl % U;
        for (int g0 = 0; g0 < full; g0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                load_routed<UP, S>(sl[(u + D) % U], q0, q1, s0, s1, arow_k, min(g0 + u + D, ngl - 1));
                compute_routed<UP, S>(sl[u], acc0, acc1);
            }
        }
#pragma unroll
        for (int u = 0; u < D; ++u)
            if (u < ngl - full) compute_routed<UP, S>(sl[u], acc0, acc1);
    } else {
        // this wave's quarter of the groups: gb .. gb + cnt - 1 (cnt may be 0)
        constexpr int D = DS;
        constexpr int U = D + 1;
        const int gb = glo + (wave * ngl) / 4;
        const int cnt = glo + ((wave + 1) * ngl) / 4 - gb;
        const int last = cnt > 0 ? cnt - 1 : 0;
        const int64_t rb = n >> 4;
        const int64_t mat = routed ? static_cast<int64_t>(group) * N * K : 0;  // expert's matrix
        const uint16_t* w0 = routed ? a.wb0 + mat : a.sh0;
        const uint16_t* w1 = routed ? (UP ? a.wb1 + mat : nullptr) : a.sh1;
        const uint16_t* h0 = w0 + rb * ng * 2048 + l16 * 32 + kq * 8 + gb * 2048;
        const uint16_t* h1 = UP ? w1 + rb * ng * 2048 + l16 * 32 + kq * 8 + gb * 2048 : nullptr;
        const uint16_t* ar = arow + gb * kGroup;
        SharedSlot sl[U];
#pragma unroll
        for (int p = 0; p < D; ++p) load_shared<UP>(sl[p], h0, h1, ar, min(p, last));
        const int full = cnt - cnt % U;
        for (int g0 = 0; g0 < full; g0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                load_shared<UP>(sl[(u + D) % U], h0, h1, ar, min(g0 + u + D, last));
                compute_shared<UP>(sl[u], acc0, acc1);
            }
        }
#pragma unroll
        for (int u = 0; u < D; ++u)
            if (u < cnt - full) compute_shared<UP>(sl[u], acc0, acc1);
        // sum the four waves' partial accumulators in wave order (8 KB of LDS)
        float* red = reinterpret_cast<float*>(a_lds);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            red[(wave * 64 + lane) * 8 + r] = acc0[r];
            red[(wave * 64 + lane) * 8 + 4 + r] = acc1[r];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc0[r] = red[lane * 8 + r];
            acc1[r] = red[lane * 8 + 4 + r];
        }
#pragma unroll
        for (int w = 1; w < 4; ++w)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc0[r] += red[(w * 64 + lane) * 8 + r];
                acc1[r] += red[(w * 64 + lane) * 8 + 4 + r];
            }
    }

    // D[m][n]: m = 4 * kq + r (token row of the chunk), n = l16 (this lane's feature)
    // up: routed rows of H are stored with 8-blocks interleaved for the down projection
    const int64_t hcol = int4 ? ((n & ~7LL) | (((n & 3) << 1) | ((n >> 2) & 1))) : n;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int mr = kq * 4 + r;
        if (mr >= nrows) continue;
        const int64_t orow = row0 + mr;
        if (UP) a.h_out[orow * N + hcol] = f32_to_bf16(siluf_(acc0[r]) * acc1[r]);
        else (kz ? a.o_out2 : a.o_out)[orow * N + n] = acc0[r];
    }
}

// LDS budget for staged A rows: 48 KB keeps three blocks (12 waves) per CU
constexpr int64_t kDecodeLdsBytes = 48 * 1024;
constexpr size_t kReduceLdsBytes = 4 * 64 * 8 * sizeof(float);  // shared-chunk wave sums

static int lds_rows(int64_t K) {
    const int64_t r = kDecodeLdsBytes / ((K + 8) * 2);
    return static_cast<int>(r < kDecodeRows ? r : kDecodeRows);
}

// grid: N / 64 feature ranges (twice as many blocks with the reduction split,
// the halves of a range adjacent) x (chunks + 3 extra rows per shared-expert chunk);
// max_chunks bounds the chunk list, shared_chunks is the number of shared-expert
// chunks at its head (0 when the shared expert runs on the GEMMs)
// F8 / S pick the kernel instantiation (fp8 experts, int4 scales per tile row)
template <bool UP, int DR, int DS, int DL, bool F8, int S, bool SL = false>
static hipError_t launch_decode(const DecodeArgs& args, int max_chunks, int shared_chunks,
                                hipStream_t stream) {
    DecodeArgs a = args;
    a.lds_rows = lds_rows(a.K);
    a.max_chunks = max_chunks;
    size_t lds = a.lds_rows > 0 ? static_cast<size_t>(a.lds_rows) * (a.K + 8) * 2 : 0;
    lds = lds > kReduceLdsBytes ? lds : kReduceLdsBytes;
    // int4 chunks past lds_rows rows stage A in slices (SL)
    static_assert(!SL || (S == 1 && !F8), "sliced staging: int4 groups of 128");
    constexpr size_t sliced = SL ? slice_lds_bytes(slice_groups(UP, DL)) : 0;
    if (a.lds_rows < kDecodeRows && lds < sliced) lds = sliced;
    // two blocks per chunk and feature range, each half the reduction, when the
    // host gives a second output (down projection, int4 weights); the
    // kernel takes the half from blockIdx.x under the same condition
    const unsigned zs = (!UP && !F8 && !SL && a.o_out2) ? 2u : 1u;
    dim3 grid(static_cast<unsigned>(a.N / 64 * zs), static_cast<unsigned>(max_chunks + 3 * shared_chunks), 1);
    MOE_LAUNCH((decode_kernel<UP, DR, DS, DL, F8, S, SL>), grid, dim3(NT), lds, stream, a);
    return hipGetLastError();
}

// ring depths (tiles in flight): DR routed chunks reading A from global
// memory, DS bf16 chunks, DL routed chunks with A staged in LDS; smaller
// int4 groups hold more scales per slot and take shallower rings (measured on
// the Scout decode layer: groups of 64 up 119 -> 108 us, groups of 32 up
// 126 -> 118 us and down 86 -> 79 us against the depths of groups of 128).
// Groups of 64, up: DR 3 needs 154 VGPRs, two waves per SIMD; DR 2 fits in
// 128, three waves: 104.8 -> 98.2 us.
hipError_t launch_decode_up(const DecodeArgs& args, int max_chunks, int shared_chunks,
                            hipStream_t stream) {
    if (args.wf0) return launch_decode<true, 3, 1, 7, true, 1>(args, max_chunks, shared_chunks, stream);
    if (args.spt == 2) return launch_decode<true, 2, 1, 5, false, 2>(args, max_chunks, shared_chunks, stream);
    if (args.spt == 4) return launch_decode<true, 2, 1, 4, false, 4>(args, max_chunks, shared_chunks, stream);
    if (args.sliced) return launch_decode<true, 3, 1, 5, false, 1, true>(args, max_chunks, shared_chunks, stream);
    return launch_decode<true, 3, 1, 5, false, 1>(args, max_chunks, shared_chunks, stream);
}

hipError_t launch_decode_down(const DecodeArgs& args, int max_chunks, int shared_chunks,
                              hipStream_t stream) {
    if (args.wf0) return launch_decode<false, 3, 2, 7, true, 1>(args, max_chunks, shared_chunks, stream);
    if (args.spt == 2) return launch_decode<false, 2, 2, 5, false, 2>(args, max_chunks, shared_chunks, stream);
    if (args.spt == 4) return launch_decode<false, 2, 2, 2, false, 4>(args, max_chunks, shared_chunks, stream);
    if (args.sliced) return launch_decode<false, 3, 2, 7, false, 1, true>(args, max_chunks, shared_chunks, stream);
    // Groups of 64 and 32 with the reduction split (Scout decode layer, three
    // alternating rounds): down 63.2 -> 58.1 us and 68.8 -> 60.2 us against
    // the unsplit launch at rings (3, 7) and (2, 5); LDS rings of 4 (groups of
    // 64) and 3 (groups of 32), or a global ring of 3 at groups of 32 (68.8 us),
    // measured slower.
    // LDS ring 5 (7 before the reduction split halved each block's groups: 53.0
    // against 54.2 us on the Scout decode layer)
    return launch_decode<false, 3, 2, 5, false, 1>(args, max_chunks, shared_chunks, stream);
}

}  // namespace moe
