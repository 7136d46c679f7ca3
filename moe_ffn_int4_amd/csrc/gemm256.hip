// gemm256.hip -- grouped expert GEMMs with 256 x 256 tiles, for prefill layers
// whose experts each hold hundreds of token rows.
//
// Same computation, operands, tile table and LDS fragment order as gemm.hip
// (the expert FFN of the discosf.com page "1 卡跑通 Llama 4", section
// "混合专家路由", with the SwiGLU of the docs.ifdog.com page "Llama 开源模型系列",
// section "SwiGLU：门控激活的数学"; int4 weights dequantized as code * scale).
// What changes is the work per wave and how its latencies are hidden:
//
//  * one block per CU, 4 waves in a 2 x 2 grid, each 128 x 128 from 8 x 8
//    v_mfma_f32_16x16x32_bf16 tiles: 256 fp32 accumulators per lane (AGPRs),
//    so a wave issues 64 MFMAs per 32-wide reduction step against 16 fragment
//    reads (a 64 x 128 wave tile issues 32 against 12);
//  * three LDS stages of 32 KB: step k+1 is complete in LDS while step k's
//    MFMAs run, so its 16 fragments are read in between those MFMAs and the
//    next step starts with its operands in registers; step k+2 goes from
//    registers (int4 dequantized on the way) into the third stage meanwhile;
//  * global data is requested two steps ahead of its LDS store in two register
//    sets; one barrier per step.
//
// Stage ownership at step k: stage (k+1)%3 is read (fragments of step k+1),
// stage (k+2)%3 is written (step k+2); stage k%3 is idle (its fragments are in
// registers). The barrier at the end of step k publishes step k+2 and
// retires the reads of step k+1's stage before step k+2 (the next writer of
// that stage is step k+3's data, stored in iteration k+1... after that barrier).
//
// Partial row tiles run all MFMAs on clamped rows (results dropped). Tiles
// with fp8 weights are not handled here (the host uses the 128-row kernel).
#include <type_traits>

#include "gemm_common.h"

namespace moe {

namespace {
constexpr int BM2 = kPrefillBM2;     // 256 token rows
constexpr int BN2 = 256;             // B rows per block
constexpr int BK2 = 32;              // reduction step
constexpr int NT2 = 256;             // 4 waves
constexpr int SUB2 = 1024;           // bytes per 16 x 32 bf16 sub-tile
constexpr int ASUB2 = BM2 / 16;      // 16 A sub-tiles
constexpr int STAGE2 = (ASUB2 + 16) * SUB2;  // 32 KB
constexpr int NSTAGE2 = 3;
static_assert(BM2 == 256, "tile table row height");
}  // namespace

template <bool UP, bool ROUTED>
__device__ __forceinline__ void gemm256_tile(const GroupedGemmArgs& a, const Tile& tile, int nt,
                                             uint8_t* lds) {
    const bool routed_rows = tile.group < a.E;
    const int64_t K = a.K, N = a.N;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int64_t n0 = static_cast<int64_t>(nt) * (UP ? BN2 / 2 : BN2);
    const int64_t ng = K / kGroup;
    const int steps = static_cast<int>(K / BK2);

    // ---- A staging: thread -> rows (tid/4) + 64 i (i = 0..3), piece q = tid % 4
    constexpr int AP = BM2 * BK2 / 8 / NT2;  // 4 pieces per thread
    const uint16_t* arow[AP];
#pragma unroll
    for (int i = 0; i < AP; ++i) {
        int r = (tid >> 2) + 64 * i;
        r = r < tile.nrows ? r : tile.nrows - 1;
        const int64_t s = tile.row0 + r;
        int64_t src;
        if (UP) src = routed_rows ? a.perm[s] / a.top_k : s - a.P;
        else src = s;
        arow[i] = a.a + src * K + (tid & 3) * 8;
    }
    const int a_st = (tid >> 6) * SUB2 + frag_slot((tid >> 2) & 15, tid & 3);  // + 4 i sub-tiles

    // ---- B staging as in gemm.hip: int4 B row tid; bf16 load c of a thread
    // takes B tile 4 wave + c, lane -> row lane / 4, piece lane % 4
    int64_t bn = UP ? n0 + (tid & 127) : n0 + tid;
    bn = bn < N ? bn : N - 1;
    const uint8_t* bq = nullptr;
    const float* bs = nullptr;
    const uint16_t* bh[4] = {nullptr, nullptr, nullptr, nullptr};
    const int wv = __builtin_amdgcn_readfirstlane(wid);
    if (ROUTED) {
        const int64_t rb = static_cast<int64_t>(tile.group) * (N / 16) + (bn >> 4);
        const uint8_t* q = (UP && tid >= 128) ? a.wq1 : a.wq0;
        const float* sc = (UP && tid >= 128) ? a.ws1 : a.ws0;
        bq = q + rb * ng * 1024 + (bn & 15) * 16;
        bs = sc + (rb * ng * 16 + (bn & 15)) * a.spt;
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int bt = wv * 4 + c;
            int64_t r0 = UP ? n0 + 16 * (bt & 7) : n0 + 16 * bt;
            r0 = r0 < N ? r0 : N - 16;
            const bool w3 = UP && bt >= 8;
            const uint16_t* src;
            if (routed_rows)
                src = (w3 ? a.wb1 : a.wb0) + static_cast<int64_t>(tile.group) * N * K;
            else
                src = w3 ? a.sh1 : a.sh0;
            bh[c] = src + (r0 >> 4) * ng * 2048 + lane * 8;
        }
    }
    const int b_st = ASUB2 * SUB2 + (tid >> 4) * SUB2;
    const int b_st_h = ASUB2 * SUB2 + wv * 4 * SUB2 + frag_slot(lane >> 2, lane & 3);

    constexpr int BV = ROUTED ? 1 : 4;
    u32x4 ra0[AP], rb0[BV], ra1[AP], rb1[BV];
    float rs0 = 0.f, rs1 = 0.f;
    auto load_step = [&](u32x4 (&ra)[AP], u32x4 (&rb)[BV], float& rs, int k)
                         __attribute__((always_inline)) {
        k = k < steps ? k : steps - 1;  // past the end: reload the last step (unused)
        const int64_t k0 = static_cast<int64_t>(k) * BK2;
#pragma unroll
        for (int i = 0; i < AP; ++i) ra[i] = *reinterpret_cast<const u32x4*>(arow[i] + k0);
        const int64_t g = k0 / kGroup;
        const int quarter = k & 3;
        if (ROUTED) {
            rb[0] = *reinterpret_cast<const u32x4*>(bq + g * 1024 + quarter * 256);
            rs = bs[g * 16 * a.spt + ((quarter * a.spt) >> 2)];
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                rb[c] = *reinterpret_cast<const u32x4*>(bh[c] + g * 2048 + quarter * 512);
        }
    };
    auto store_step = [&](const u32x4 (&ra)[AP], const u32x4 (&rb)[BV], float rs, int stage)
                          __attribute__((always_inline)) {
        uint8_t* st = lds + stage * STAGE2;
#pragma unroll
        for (int i = 0; i < AP; ++i) *reinterpret_cast<u32x4*>(st + a_st + 4 * i * SUB2) = ra[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (ROUTED)
                *reinterpret_cast<u32x4*>(st + b_st + frag_slot(tid & 15, q)) = dequant8(rb[0][q], rs);
            else
                *reinterpret_cast<u32x4*>(st + b_st_h + q * SUB2) = rb[ROUTED ? 0 : q];
        }
    };

    // ---- fragments: this wave's 8 A sub-tiles (rows wm*128 ..) and 8 B sub-tiles
    const int lslot = frag_slot(lane & 15, lane >> 4);
    int a_off[8], b_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a_off[i] = (wm * 8 + i) * SUB2 + lslot;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        b_off[j] = ASUB2 * SUB2 + lslot +
                   SUB2 * (UP ? ((j < 4) ? wn * 4 + j : 8 + wn * 4 + (j - 4)) : wn * 8 + j);

    bf16x8 fa0[8], fb0[8], fa1[8], fb1[8];
    auto read_frags = [&](bf16x8 (&fa)[8], bf16x8 (&fb)[8], int stage) __attribute__((always_inline)) {
        const uint8_t* st = lds + stage * STAGE2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            fb[i] = *reinterpret_cast<const bf16x8*>(st + b_off[i]);
            fa[i] = *reinterpret_cast<const bf16x8*>(st + a_off[i]);
        }
    };

    f32x4 acc[8][8];
    auto mfma_step = [&](const bf16x8 (&fa)[8], const bf16x8 (&fb)[8], auto first)
                         __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first)::value;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    fa[i], fb[j], FIRST ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][j], 0, 0, 0);
    };

    // One step: MFMAs of step k on (fa, fb); fragments of step k+1 from stage
    // `rd`; step k+2 (in ra/rb) into stage `wr`; step k+4 requested into ra/rb.
    // With one wave per SIMD nothing else covers a stretch of VALU or LDS work,
    // so the step runs as 8 chunks, one per A sub-tile i: its 8 MFMAs, two of
    // the next step's fragment reads and one staging piece (A piece, or one
    // dequantized 8-code word of B), alternating A and B pieces so that the
    // dequantization spreads over the chunks; each register of the staging set
    // is requested again as soon as it has been stored.
    auto step = [&](const bf16x8 (&fa)[8], const bf16x8 (&fb)[8], bf16x8 (&na)[8], bf16x8 (&nb)[8],
                    u32x4 (&ra)[AP], u32x4 (&rb)[BV], float& rs, int k, int rd, int wr, auto first)
                    __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first)::value;
        const uint8_t* rs_st = lds + rd * STAGE2;
        uint8_t* ws_st = lds + wr * STAGE2;
        const int kn = (k + 4) < steps ? k + 4 : steps - 1;  // the step requested next
        const int64_t kn0 = static_cast<int64_t>(kn) * BK2;
        const int64_t gn = kn0 / kGroup;
        const int qn = kn & 3;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    fa[i], fb[j], FIRST ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][j], 0, 0, 0);
            nb[i] = *reinterpret_cast<const bf16x8*>(rs_st + b_off[i]);
            na[i] = *reinterpret_cast<const bf16x8*>(rs_st + a_off[i]);
            const int piece = i >> 1;
            if ((i & 1) == 0) {
                *reinterpret_cast<u32x4*>(ws_st + a_st + 4 * piece * SUB2) = ra[piece];
                ra[piece] = *reinterpret_cast<const u32x4*>(arow[piece] + kn0);
            } else {
                if (ROUTED) {
                    *reinterpret_cast<u32x4*>(ws_st + b_st + frag_slot(tid & 15, piece)) =
                        dequant8(rb[0][piece], rs);
                } else {
                    *reinterpret_cast<u32x4*>(ws_st + b_st_h + piece * SUB2) = rb[ROUTED ? 0 : piece];
                    rb[ROUTED ? 0 : piece] =
                        *reinterpret_cast<const u32x4*>(bh[piece] + gn * 2048 + qn * 512);
                }
            }
            if (ROUTED && i == 7) {
                rb[0] = *reinterpret_cast<const u32x4*>(bq + gn * 1024 + qn * 256);
                rs = bs[gn * 16 * a.spt + ((qn * a.spt) >> 2)];
            }
            // MFMAs paced with the chunk's other work
            if (ROUTED && (i & 1)) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };

    // prologue: steps 0 and 1 into stages 0 and 1, step 0's fragments into
    // registers, steps 2 and 3 requested
    load_step(ra0, rb0, rs0, 0);
    load_step(ra1, rb1, rs1, 1);
    store_step(ra0, rb0, rs0, 0);
    store_step(ra1, rb1, rs1, 1);
    __syncthreads();
    read_frags(fa0, fb0, 0);
    load_step(ra0, rb0, rs0, 2);
    load_step(ra1, rb1, rs1, 3);
    __builtin_amdgcn_sched_barrier(0);

    // step k: reads stage (k+1)%3, writes stage (k+2)%3; register sets
    // alternate (fragments and staging), so the loop runs two steps per pass
    step(fa0, fb0, fa1, fb1, ra0, rb0, rs0, 0, 1, 2, std::true_type{});
    int rd = 2, wr = 0;  // stages of step 1
    int k = 1;
    for (; k + 1 < steps; k += 2) {
        step(fa1, fb1, fa0, fb0, ra1, rb1, rs1, k, rd, wr, std::false_type{});
        rd = rd == 2 ? 0 : rd + 1;
        wr = wr == 2 ? 0 : wr + 1;
        step(fa0, fb0, fa1, fb1, ra0, rb0, rs0, k + 1, rd, wr, std::false_type{});
        rd = rd == 2 ? 0 : rd + 1;
        wr = wr == 2 ? 0 : wr + 1;
    }
    mfma_step(fa1, fb1, std::false_type{});  // the last step (steps is even, so it is odd)

    // ---- epilogue: D[row][col], row = 4 * lq + r inside a 16 x 16 sub-tile, col = l16
    const int l16 = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wm * 128 + i * 16 + lq * 4 + r;
            if (row >= tile.nrows) continue;
            const int64_t orow = tile.row0 + row;
            if (UP) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float g = acc[i][j][r], u = acc[i][j + 4][r];
                    const int64_t col = n0 + wn * 64 + j * 16 + l16;
                    a.h_out[orow * N + col] = f32_to_bf16(siluf_(g) * u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int64_t col = n0 + wn * 128 + j * 16 + l16;
                    if (col < N) a.o_out[orow * N + col] = acc[i][j][r];
                }
            }
        }
    }
}

// XCD-aware block order as in gemm.hip (row tiles of 256 rows)
template <bool UP>
__global__ __launch_bounds__(NT2, 1) void grouped_gemm256_kernel(GroupedGemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int ncol = UP ? static_cast<int>(a.N / (BN2 / 2)) : static_cast<int>((a.N + BN2 - 1) / BN2);
    const int nrow = a.tile_base[a.E + 1];
    const int total = nrow * ncol;
    const int L = blockIdx.x;
    if (L >= total) return;
    constexpr int kXcd = 8, kGroupRows = 4;
    const int xcd = L % kXcd, slot = L / kXcd;
    const int base = total / kXcd, extra = total % kXcd;
    const int lin = xcd * base + (xcd < extra ? xcd : extra) + slot;
    const int span = kGroupRows * ncol;
    const int first_row = (lin / span) * kGroupRows;
    const int rows_here = nrow - first_row < kGroupRows ? nrow - first_row : kGroupRows;
    const int mt = first_row + (lin % span) % rows_here;
    const int nt = (lin % span) / rows_here;

    Tile tile;
    if (!find_tile<BM2>(a, mt, tile)) return;
    if (tile.group < a.E && !a.wb0) gemm256_tile<UP, true>(a, tile, nt, lds);
    else gemm256_tile<UP, false>(a, tile, nt, lds);
}

static unsigned max_row_tiles256(const GroupedGemmArgs& a) {
    const int64_t e_bound = a.E < a.P ? a.E : a.P;
    return static_cast<unsigned>((a.P + BM2 - 1) / BM2 + e_bound + (a.T + BM2 - 1) / BM2);
}

static constexpr size_t kGemm256Lds = NSTAGE2 * STAGE2;  // 96 KB

template <bool UP>
static hipError_t allow_lds256() {
    static hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&grouped_gemm256_kernel<UP>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kGemm256Lds));
    return e;
}

hipError_t launch_grouped_up256(const GroupedGemmArgs& a, hipStream_t stream) {
    if (hipError_t e = allow_lds256<true>(); e != hipSuccess) return e;
    dim3 grid(max_row_tiles256(a) * static_cast<unsigned>(a.N / (BN2 / 2)));
    hipLaunchKernelGGL(grouped_gemm256_kernel<true>, grid, dim3(NT2), kGemm256Lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_grouped_down256(const GroupedGemmArgs& a, hipStream_t stream) {
    if (hipError_t e = allow_lds256<false>(); e != hipSuccess) return e;
    dim3 grid(max_row_tiles256(a) * static_cast<unsigned>((a.N + BN2 - 1) / BN2));
    hipLaunchKernelGGL(grouped_gemm256_kernel<false>, grid, dim3(NT2), kGemm256Lds, stream, a);
    return hipGetLastError();
}

}  // namespace moe
