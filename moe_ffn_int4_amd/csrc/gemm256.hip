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
// Partial row tiles run all MFMAs on clamped rows (results dropped); a routed
// int4 tile of at most 128 rows (an expert's tail) runs a half-height body
// (each wave 64 x 128). Tiles of fp8 experts run their own body on the 128-deep
// fp8 instruction (gemm256_tile_fp8). Blocks map to tiles by xcd_tile: each
// XCD takes a contiguous range of tiles cut by estimated time.
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

// MI: A sub-tiles (16 rows) per wave, 8 for a full 256-row tile; 4 for a half
// tile of at most 128 rows (the tail of a routed expert), each wave 64 x 128:
// half the MFMAs, the same B staging.
template <bool UP, bool ROUTED, int MI = 8>
__device__ __forceinline__ void gemm256_tile(const GroupedGemmArgs& a, const Tile& tile, int nt,
                                             uint8_t* lds) {
    static_assert(MI == 8 || MI == 4, "full or half tile");
    const bool routed_rows = tile.group < a.E;
    const int64_t K = a.K, N = a.N;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int64_t n0 = static_cast<int64_t>(nt) * (UP ? BN2 / 2 : BN2);
    const int64_t ng = K / kGroup;
    const int steps = static_cast<int>(K / BK2);

    // ---- A staging: thread -> rows (tid/4) + 64 i (i < AP), piece q = tid % 4
    constexpr int AP = MI / 2;  // 4 pieces per thread (256 rows), 2 for a half tile
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
        if (ROUTED) {
            rb[0] = *reinterpret_cast<const u32x4*>(bq + k * 256);
            rs = bs[step_scale(k, a.spt)];
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) rb[c] = *reinterpret_cast<const u32x4*>(bh[c] + k * 512);
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

    // ---- fragments: this wave's MI A sub-tiles (rows wm*16*MI ..) and 8 B sub-tiles
    const int lslot = frag_slot(lane & 15, lane >> 4);
    int a_off[MI], b_off[8];
#pragma unroll
    for (int i = 0; i < MI; ++i) a_off[i] = (wm * MI + i) * SUB2 + lslot;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        b_off[j] = ASUB2 * SUB2 + lslot +
                   SUB2 * (UP ? ((j < 4) ? wn * 4 + j : 8 + wn * 4 + (j - 4)) : wn * 8 + j);

    bf16x8 fa0[MI], fb0[8], fa1[MI], fb1[8];
    auto read_frags = [&](bf16x8 (&fa)[MI], bf16x8 (&fb)[8], int stage) __attribute__((always_inline)) {
        const uint8_t* st = lds + stage * STAGE2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            fb[i] = *reinterpret_cast<const bf16x8*>(st + b_off[i]);
            if (i < MI) fa[i] = *reinterpret_cast<const bf16x8*>(st + a_off[i]);
        }
    };

    f32x4 acc[MI][8];
    auto mfma_step = [&](const bf16x8 (&fa)[MI], const bf16x8 (&fb)[8], auto first)
                         __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first)::value;
#pragma unroll
        for (int i = 0; i < MI; ++i)
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
    auto step = [&](const bf16x8 (&fa)[MI], const bf16x8 (&fb)[8], bf16x8 (&na)[MI], bf16x8 (&nb)[8],
                    u32x4 (&ra)[AP], u32x4 (&rb)[BV], float& rs, int k, int rd, int wr, auto first)
                    __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first)::value;
        const uint8_t* rs_st = lds + rd * STAGE2;
        uint8_t* ws_st = lds + wr * STAGE2;
        const int kn = (k + 4) < steps ? k + 4 : steps - 1;  // the step requested next
        const int64_t kn0 = static_cast<int64_t>(kn) * BK2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // chunk i: A sub-tile i against all 8 B fragments (full tile), or
            // A sub-tile i / 2 against B fragments 4 (i % 2) .. + 3 (half tile)
#pragma unroll
            for (int jj = 0; jj < MI; ++jj) {
                const int ai = MI == 8 ? i : i >> 1;
                const int j = MI == 8 ? jj : 4 * (i & 1) + jj;
                acc[ai][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    fa[ai], fb[j], FIRST ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[ai][j], 0, 0, 0);
            }
            nb[i] = *reinterpret_cast<const bf16x8*>(rs_st + b_off[i]);
            if (i < MI) na[i] = *reinterpret_cast<const bf16x8*>(rs_st + a_off[i]);
            const int piece = i >> 1;
            if ((i & 1) == 0) {
                if (piece < AP) {
                    *reinterpret_cast<u32x4*>(ws_st + a_st + 4 * piece * SUB2) = ra[piece];
                    ra[piece] = *reinterpret_cast<const u32x4*>(arow[piece] + kn0);
                }
            } else {
                if (ROUTED) {
                    *reinterpret_cast<u32x4*>(ws_st + b_st + frag_slot(tid & 15, piece)) =
                        dequant8(rb[0][piece], rs);
                } else {
                    *reinterpret_cast<u32x4*>(ws_st + b_st_h + piece * SUB2) = rb[ROUTED ? 0 : piece];
                    rb[ROUTED ? 0 : piece] = *reinterpret_cast<const u32x4*>(bh[piece] + kn * 512);
                }
            }
            if (ROUTED && i == 7) {
                rb[0] = *reinterpret_cast<const u32x4*>(bq + kn * 256);
                rs = bs[step_scale(kn, a.spt)];
            }
            // MFMAs paced with the chunk's other work
            if (ROUTED && (i & 1)) {
#pragma unroll
                for (int t = 0; t < MI; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 32 / MI, 0);
                }
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, MI / 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, MI / 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, MI / 2, 0);
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
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wm * 16 * MI + i * 16 + lq * 4 + r;
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

// Routed tiles of fp8 experts (fp8 activation rows x fp8 weights): the
// gfx950 scaled fp8 matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4
// with both operands E4M3 and unit block scales (exponent 127), twice the rate
// of the 32-deep bf16 and fp8 instructions. One step is 128 deep. Lane
// (n = l % 16, q = l / 16) of a 16-row operand holds row n, bytes 32q .. 32q + 31
// of the step; A and B use the same assignment, so every product pairs equal
// k whatever order the instruction sums in. That is the contiguous 32 bytes
// at 32 l of a 16-row x 128-column tile of the fp8 weights, and the 32 bytes
// at 32q of the step in an activation row: global loads arrive in fragment
// order. A 16-row sub-tile takes 2 KB of LDS as two 1 KB halves (lane l's
// bytes 0-15 at 16 l, 16-31 at 1024 + 16 l), so staging writes and fragment
// reads are contiguous 1 KB per instruction. Two 64 KB stages: step k+1 is
// stored into the other stage while step k is multiplied, and step k+2 is
// requested into registers, paced between the products. Each wave: 128 x 128 from 8 x 8 products, 256
// accumulators. The epilogue scales by both row scales and rounds to bf16
// where the fp8 matmul of the pages returns bf16: the two up-projections, then
// the SwiGLU product (bf16 H); down: the expert output.
constexpr int FSUB2 = 2048;               // bytes per 16-row x 128-column fp8 sub-tile
constexpr int FSTAGE2 = 32 * FSUB2;       // 16 A + 16 B sub-tiles: 64 KB
constexpr int NFSTAGE2 = 2;

template <bool UP>
__device__ __forceinline__ void gemm256_tile_fp8(const GroupedGemmArgs& a, const Tile& tile, int nt,
                                                 uint8_t* lds) {
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    constexpr int FK = 128;
    const int64_t K = a.K, N = a.N;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int64_t n0 = static_cast<int64_t>(nt) * (UP ? BN2 / 2 : BN2);
    const int64_t ng = K / kGroup;
    const int steps = static_cast<int>(K / FK);

    // ---- staging: this wave takes A sub-tiles 4 wid + i (rows 64 wid + 16 i + r16)
    // and B sub-tiles 4 wid + i (B rows 16 (4 wid + i) + r16), lane l's 32 bytes of each
    const uint8_t* arow[4];
    const uint8_t* brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int r = 64 * wid + 16 * i + r16;
        r = r < tile.nrows ? r : tile.nrows - 1;
        const int64_t s = tile.row0 + r;
        const int64_t src = UP ? a.perm[s] / a.top_k : s;
        arow[i] = a.a8 + src * K + 32 * q4;
        const int br = 16 * (4 * wid + i) + r16;
        int64_t bn = UP ? n0 + (br & 127) : n0 + br;
        bn = bn < N ? bn : N - 1;
        const uint8_t* m = ((UP && br >= 128) ? a.wf1 : a.wf0) + static_cast<int64_t>(tile.group) * N * K;
        brow[i] = m + (bn >> 4) * ng * 2048 + (bn & 15) * 32 + 512 * q4;  // + step * 2048
    }
    u32x4 ra[4][2], rb[4][2];
    auto load_step = [&](int k) __attribute__((always_inline)) {
        k = k < steps ? k : steps - 1;  // past the end: reload the last step (unused)
        const int64_t ka = static_cast<int64_t>(k) * FK, kb = static_cast<int64_t>(k) * 2048;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                ra[i][h] = *reinterpret_cast<const u32x4*>(arow[i] + ka + 16 * h);
                rb[i][h] = *reinterpret_cast<const u32x4*>(brow[i] + kb + 16 * h);
            }
    };
    auto store_step = [&](int stage) __attribute__((always_inline)) {
        uint8_t* st = lds + stage * FSTAGE2 + lane * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                *reinterpret_cast<u32x4*>(st + (4 * wid + i) * FSUB2 + h * 1024) = ra[i][h];
                *reinterpret_cast<u32x4*>(st + (16 + 4 * wid + i) * FSUB2 + h * 1024) = rb[i][h];
            }
    };
    auto frag = [&](const uint8_t* st, int sub) __attribute__((always_inline)) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(st + sub * FSUB2);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(st + sub * FSUB2 + 1024);
        return i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                     static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                     static_cast<int>(hi.z), static_cast<int>(hi.w)};
    };
    int sb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sb[j] = 16 + (UP ? ((j < 4) ? wn * 4 + j : 8 + wn * 4 + (j - 4)) : wn * 8 + j);

    f32x4 acc[8][8];
    // Step k: 8 chunks, one per B fragment j: its 8 products, the read of
    // fragment j+1, and one staging piece of step k+1 (A and B sub-tile j / 2,
    // half j % 2) written into the other stage, its registers then requested
    // again for step k+2 (one step ahead of their next store). At the last step
    // the piece goes to the idle stage and the request re-reads the last step.
    // The first step starts the accumulators from zero (peeled, so that the
    // loop-carried accumulators keep one register assignment).
    auto step = [&](int k, auto first) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first)::value;
        const uint8_t* st = lds + (k & 1) * FSTAGE2 + lane * 16;
        uint8_t* wst = lds + ((k & 1) ^ 1) * FSTAGE2 + lane * 16;
        const int kn = k + 2 < steps ? k + 2 : steps - 1;
        const int64_t ka = static_cast<int64_t>(kn) * FK, kb = static_cast<int64_t>(kn) * 2048;
        i32x8 fa[8], fb[2];
        fb[0] = frag(st, sb[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) fa[i] = frag(st, wm * 8 + i);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j + 1 < 8) fb[(j + 1) & 1] = frag(st, sb[j + 1]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    fa[i], fb[j & 1], FIRST ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][j], 0, 0, 0, 127, 0, 127);
            const int p = j >> 1, h = j & 1;
            *reinterpret_cast<u32x4*>(wst + (4 * wid + p) * FSUB2 + h * 1024) = ra[p][h];
            *reinterpret_cast<u32x4*>(wst + (16 + 4 * wid + p) * FSUB2 + h * 1024) = rb[p][h];
            ra[p][h] = *reinterpret_cast<const u32x4*>(arow[p] + ka + 16 * h);
            rb[p][h] = *reinterpret_cast<const u32x4*>(brow[p] + kb + 16 * h);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // next fragment's reads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);  // staging writes
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // global loads
            __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };

    load_step(0);
    store_step(0);
    __syncthreads();
    load_step(1);
    step(0, std::true_type{});
    for (int k = 1; k < steps; ++k) step(k, std::false_type{});

    // ---- epilogue: D[row][col], row = 4 * lq + r inside a 16 x 16 sub-tile, col = l16
    const int l16 = lane & 15, lq = lane >> 4;
    const float* ws0 = a.wfs0 + static_cast<int64_t>(tile.group) * N;
    const float* ws1 = UP ? a.wfs1 + static_cast<int64_t>(tile.group) * N : nullptr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wm * 128 + i * 16 + lq * 4 + r;
            if (row >= tile.nrows) continue;
            const int64_t orow = tile.row0 + row;
            const float sa = a.a8s[UP ? a.perm[orow] / a.top_k : orow];
            if (UP) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t col = n0 + wn * 64 + j * 16 + l16;
                    const float g = bf16_to_f32(f32_to_bf16(acc[i][j][r] * sa * ws0[col]));
                    const float u = bf16_to_f32(f32_to_bf16(acc[i][j + 4][r] * sa * ws1[col]));
                    a.h_out[orow * N + col] = f32_to_bf16(siluf_(g) * u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int64_t col = n0 + wn * 128 + j * 16 + l16;
                    if (col < N) a.o_out[orow * N + col] = bf16_to_f32(f32_to_bf16(acc[i][j][r] * sa * ws0[col]));
                }
            }
        }
    }
}

// XCD-aware block order as in gemm.hip (row tiles of 256 rows; xcd_tile).
// F8: launches with fp8 routed experts, a separate instantiation so that the
// int4 / bf16 one keeps its register allocation and schedule.
template <bool UP, bool F8>
__global__ __launch_bounds__(NT2, 1) void grouped_gemm256_kernel(GroupedGemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int ncol = UP ? static_cast<int>(a.N / (BN2 / 2)) : static_cast<int>((a.N + BN2 - 1) / BN2);
    // kTilesShared: the shared expert alone, 256-row tiles of its T rows
    const bool shared_only = a.tile_mode == kTilesShared;
    const int nrow = shared_only ? static_cast<int>((a.T + BM2 - 1) / BM2) : a.tile_base[a.E + 1];
    const int64_t routed = shared_only ? 0 : static_cast<int64_t>(a.tile_base[a.E]) * ncol;
    constexpr int kGroupRows = 4;
    int lin;
    if (!xcd_tile(blockIdx.x, routed, static_cast<int64_t>(nrow) * ncol, tile_weight(a), lin))
        return;
    const int span = kGroupRows * ncol;
    const int first_row = (lin / span) * kGroupRows;
    const int rows_here = nrow - first_row < kGroupRows ? nrow - first_row : kGroupRows;
    const int mt = first_row + (lin % span) % rows_here;
    const int nt = (lin % span) / rows_here;

    Tile tile;
    if (shared_only) {
        tile.group = a.E;
        tile.row0 = a.P + static_cast<int64_t>(mt) * BM2;
        const int64_t left = a.T - static_cast<int64_t>(mt) * BM2;
        tile.nrows = static_cast<int>(left < BM2 ? left : BM2);
    } else if (!find_tile<BM2>(a, mt, tile)) {
        return;
    }
    if (F8 && tile.group < a.E) gemm256_tile_fp8<UP>(a, tile, nt, lds);
    else if (!F8 && tile.group < a.E && !a.wb0 && tile.nrows <= 128) gemm256_tile<UP, true, 4>(a, tile, nt, lds);
    else if (!F8 && tile.group < a.E && !a.wb0) gemm256_tile<UP, true>(a, tile, nt, lds);
    else gemm256_tile<UP, false>(a, tile, nt, lds);
}

static unsigned max_row_tiles256(const GroupedGemmArgs& a) {
    if (a.tile_mode == kTilesShared) return static_cast<unsigned>((a.T + BM2 - 1) / BM2);
    const int64_t e_bound = a.E < a.P ? a.E : a.P;
    return static_cast<unsigned>((a.P + BM2 - 1) / BM2 + e_bound + (a.T + BM2 - 1) / BM2);
}

// 96 KB for bf16 / int4 tiles, 128 KB when fp8 tiles are in the launch
static constexpr size_t kGemm256Lds = NSTAGE2 * STAGE2;
static constexpr size_t kGemm256LdsFp8 = NFSTAGE2 * FSTAGE2;

template <bool UP, bool F8>
static hipError_t launch256(const GroupedGemmArgs& a, unsigned ncol, hipStream_t stream) {
    constexpr size_t lds = F8 ? kGemm256LdsFp8 : kGemm256Lds;
    static hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&grouped_gemm256_kernel<UP, F8>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    dim3 grid(xcd_grid(static_cast<int64_t>(max_row_tiles256(a)) * ncol, tile_weight(a)));
    MOE_LAUNCH((grouped_gemm256_kernel<UP, F8>), grid, dim3(NT2), lds, stream, a);
    return hipGetLastError();
}

// the shared expert's tiles are bf16 whatever the routed experts are: a
// shared-only launch takes the bf16 / int4 instantiation
hipError_t launch_grouped_up256(const GroupedGemmArgs& a, hipStream_t stream) {
    const unsigned ncol = static_cast<unsigned>(a.N / (BN2 / 2));
    return a.wf0 && a.tile_mode != kTilesShared ? launch256<true, true>(a, ncol, stream)
                                                : launch256<true, false>(a, ncol, stream);
}

hipError_t launch_grouped_down256(const GroupedGemmArgs& a, hipStream_t stream) {
    const unsigned ncol = static_cast<unsigned>((a.N + BN2 - 1) / BN2);
    return a.wf0 && a.tile_mode != kTilesShared ? launch256<false, true>(a, ncol, stream)
                                                : launch256<false, false>(a, ncol, stream);
}

}  // namespace moe
