// gemm.hip -- K4/K5/K6: grouped expert GEMMs on gfx950 bf16 MFMA (prefill).
//
// Every chosen expert runs its SwiGLU FFN only on the tokens routed to it
// (discosf.com page "1 卡跑通 Llama 4", section "混合专家路由"), and the
// shared expert runs on every token. The expert FFN is
// (Swish(x W1^T) * (x W3^T)) W2^T (docs.ifdog.com page "Llama 开源模型系列",
// section "SwiGLU：门控激活的数学"). Routed weights are int4 with one fp32
// scale per group of 128 (or 64, 32) weights of a row and dequantize
// symmetrically as code * scale
// (lshu.cn page, section "量化环节": zero-points are all zero).
//
// One launch covers all groups: routed experts 0..E-1 (int4 weights, or bf16
// / fp8 for the other expert formats; rows = the expert's slots from the
// dispatch step) and the shared expert as group E (bf16 weights, rows = all T
// tokens): row tiles of all groups (tile_base from
// the dispatch step) x column tiles. Block order is XCD-aware: blocks are
// dealt round-robin to the 8 XCDs, so each XCD is given a contiguous range of
// tiles (cut by estimated time: xcd_tile), walked in groups of 8 row tiles x
// all column tiles; the 64 blocks an XCD runs at a time then share the A and
// B panels of 8 row tiles x 8 column tiles through that XCD's L2 instead of
// fetching them from HBM again.
//
//   up:   H[slot, n]  = silu(A W1^T)[n] * (A W3^T)[n]  (bf16 out)
//         A = x gathered by slot (routed) or x itself (shared); a block
//         computes 128 hidden units of W1 and the same 128 of W3, so the
//         SwiGLU product is formed in registers
//   down: O[slot, m]  = (H W2^T)[m]                    (fp32 out)
//
// Block tile 128 rows x 256 B-rows, reduction step 32 (a quarter of a
// 128-column weight tile, inside one quantization group); 256 threads = 4
// waves in a 2 x 2 grid, each wave 64 x 128 from 4 x 8
// v_mfma_f32_16x16x32_bf16 tiles (128 fp32 accumulators per lane). That leaves room for two blocks per CU (two waves per SIMD, 2 x 48 KB
// of LDS): with one wave per SIMD nothing covers a wave's wait for global or
// LDS data, with two the other block's MFMAs do. LDS holds two 24 KB stages in
// a bank-conflict-free fragment order; global data for step k+1 is in flight
// while step k's MFMAs run, and step k+2 is requested (pipeline described at
// gemm_tile). A partial row tile still runs all its MFMAs on clamped rows
// (results dropped). Layers whose experts hold hundreds of rows use the
// 256 x 256 tiles of gemm256.hip instead.
//
// Weights come in the tiled layouts (moe_quantize_int4_tiled /
// moe_pack_bf16_tiled). Int4 B rows are dequantized on the way into LDS:
// each thread takes 32 codes of one row per step, sign-extends the nibbles,
// multiplies by the group scale in fp32 and rounds to bf16 (round to nearest
// even). Accumulation is fp32 in the MFMA.
#include <type_traits>

#include "gemm_common.h"

namespace moe {

namespace {
constexpr int BM = kPrefillBM;  // 128 rows (tokens / slots)
constexpr int BN = 256;         // B rows staged per block
constexpr int BK = 32;          // reduction step: within one quantization group
constexpr int NT = 256;
static_assert(BM == 128, "tile table row height");
}  // namespace

// One block's tile: ROUTED picks the int4 or bf16 B source at compile time so
// the reduction loop has no branches (a load under a branch is waited on where
// the branch joins). Rows past the group's end and B rows past N read a valid
// clamped address; their results are dropped by the epilogue.
//
// LDS holds 2 stages of one 32-wide reduction step: 8 A sub-tiles then
// 16 B sub-tiles, each 16 rows x 32 k = 1 KB in MFMA fragment order: the
// 16-byte piece (row n, k 8q..8q+7) sits at slot 16 q + (n ^ 2q) (frag_slot),
// where fragment reads and staging writes are free of bank conflicts.
//
// Step k: the global loads of step k+2 are issued first, into the register
// set that step k+1's data is not in; each wave then reads all 12 of its
// fragments of step k from LDS before the first of its 32 MFMAs (the reads
// are forced ahead of the MFMAs, so LDS latency is paid once per step, not
// once per fragment); then step k+1 goes from registers into the other LDS
// stage (int4 dequantized on the way); one barrier per step.
// Loads are not issued under branches: a load under a branch is waited on
// where the branch joins, which would serialize it with the MFMAs.

// MI: A sub-tiles (16 rows) per wave: 4 for a full 128-row tile, 2 for a
// routed int4 tile of at most 64 rows (an expert's tail), which then issues
// half the MFMAs and stages half the A rows, with the same B staging.
template <bool UP, bool ROUTED, int MI = 4>
__device__ __forceinline__ void gemm_tile(const GroupedGemmArgs& a, const Tile& tile, int nt,
                                          uint8_t* lds) {
    static_assert(MI == 4 || MI == 2, "full or half tile");
    // ROUTED: int4 B (routed experts); otherwise bf16 B: the shared expert, or
    // routed experts held in bf16 (wb0 / wb1)
    const bool routed_rows = tile.group < a.E;
    constexpr int SUB = 1024;                 // bytes per 16 x 32 sub-tile
    constexpr int ASUB = BM / 16;             // 8 A sub-tiles
    constexpr int STAGE_BYTES = (ASUB + 16) * SUB;  // 8 A + 16 B sub-tiles
    const int64_t K = a.K, N = a.N;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int64_t n0 = static_cast<int64_t>(nt) * (UP ? BN / 2 : BN);
    const int64_t ng = K / kGroup;
    const int steps = static_cast<int>(K / BK);

    // ---- A staging: thread -> rows (tid/4) + 64 i, piece q = tid % 4
    constexpr int AP = MI / 2;  // 2 pieces per thread (128 rows), 1 for a half tile
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
    // LDS byte offset of this thread's A piece i: sub-tile (tid/64) + 4 i
    const int a_st = (tid >> 6) * SUB + frag_slot((tid >> 2) & 15, tid & 3);

    // ---- B staging. Up: B rows 0..127 are W1 rows n0 .. n0+127, rows
    // 128..255 the same rows of W3; down: W2 rows n0 .. n0+255 (the last down
    // tile may reach past N: those rows re-read valid rows, results dropped).
    // int4: thread tid takes B row tid (32 codes per step; a wave reads four
    // 256-byte step blocks); bf16: load c of a thread takes B tile (16 rows)
    // 4 wave + c, lane -> row lane / 4, piece lane % 4 (one 1 KB step block).
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
        bq = q + rb * ng * 1024 + (bn & 15) * 16;        // + tile * 1024 + quarter * 256
        bs = sc + (rb * ng * 16 + (bn & 15)) * a.spt;   // + tile * 16 * spt + the step's group
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int bt = wv * 4 + c;  // B tile 0..15
            int64_t r0 = UP ? n0 + 16 * (bt & 7) : n0 + 16 * bt;
            r0 = r0 < N ? r0 : N - 16;
            const bool w3 = UP && bt >= 8;
            const uint16_t* src;
            if (routed_rows)
                src = (w3 ? a.wb1 : a.wb0) + static_cast<int64_t>(tile.group) * N * K;
            else
                src = w3 ? a.sh1 : a.sh0;
            bh[c] = src + (r0 >> 4) * ng * 2048 + lane * 8;  // + tile*2048 + quarter*512
        }
    }
    const int b_st = ASUB * SUB + (tid >> 4) * SUB;  // int4: + frag_slot(tid & 15, q)
    const int b_st_h = ASUB * SUB + wv * 4 * SUB + frag_slot(lane >> 2, lane & 3);  // bf16: + c SUB

    constexpr int BV = ROUTED ? 1 : 4;
    // two register sets: global data two steps ahead of the MFMAs
    u32x4 ra0[AP], rb0[BV], ra1[AP], rb1[BV];
    float rs0 = 0.f, rs1 = 0.f;
    // global -> registers for reduction step k
    auto load_step = [&](u32x4 (&ra)[AP], u32x4 (&rb)[BV], float& rs, int k)
                         __attribute__((always_inline)) {
        k = k < steps ? k : steps - 1;  // past the end: reload the last step (unused)
        const int64_t k0 = static_cast<int64_t>(k) * BK;
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
    // registers -> LDS stage (int4 B dequantized on the way)
    auto store_step = [&](const u32x4 (&ra)[AP], const u32x4 (&rb)[BV], float rs, int stage)
                          __attribute__((always_inline)) {
        uint8_t* st = lds + stage * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < AP; ++i) *reinterpret_cast<u32x4*>(st + a_st + 4 * i * SUB) = ra[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (ROUTED)
                *reinterpret_cast<u32x4*>(st + b_st + frag_slot(tid & 15, q)) = dequant8(rb[0][q], rs);
            else
                *reinterpret_cast<u32x4*>(st + b_st_h + q * SUB) = rb[ROUTED ? 0 : q];
        }
    };

    f32x4 acc[MI][8];

    // fragment read offsets: lane's slot, this wave's A and B sub-tiles
    const int lslot = frag_slot(lane & 15, lane >> 4);
    int a_off[MI], b_off[8];
#pragma unroll
    for (int i = 0; i < MI; ++i) a_off[i] = (wm * MI + i) * SUB + lslot;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        b_off[j] = ASUB * SUB + lslot +
                   SUB * (UP ? ((j < 4) ? wn * 4 + j : 8 + wn * 4 + (j - 4)) : wn * 8 + j);

    // FIRST: the accumulators start from the MFMA's zero operand (no separate
    // zeroing of 256 registers, which also keeps the register allocation of the
    // loop-carried accumulators stable)
    auto mfma_step = [&](int stage, auto first) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first)::value;
        const uint8_t* st = lds + stage * STAGE_BYTES;
        bf16x8 fa[MI], fb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(st + b_off[j]);
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(st + a_off[i]);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    fa[i], fb[j], FIRST ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][j], 0, 0, 0);
        // scheduling groups: the 8 + MI LDS reads, then the 8 MI MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 8 + MI, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8 * MI, 0);
    };

    // step k computes from LDS stage k & 1; its loop iteration first requests
    // step k+2 into the register set it frees, then stores step k+1 (requested
    // one step earlier) into the other stage after the MFMAs
    load_step(ra0, rb0, rs0, 0);
    load_step(ra1, rb1, rs1, 1);
    store_step(ra0, rb0, rs0, 0);
    __syncthreads();
    load_step(ra0, rb0, rs0, 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(0, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    store_step(ra1, rb1, rs1, 1);
    __syncthreads();
    int k = 1;
    for (; k + 1 < steps; k += 2) {
        load_step(ra1, rb1, rs1, k + 2);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
        mfma_step(1, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);  // stores (which wait for the loads) after the MFMAs
        store_step(ra0, rb0, rs0, 0);
        __syncthreads();
        load_step(ra0, rb0, rs0, k + 3);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(0, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        store_step(ra1, rb1, rs1, 1);
        __syncthreads();
    }
    mfma_step(1, std::false_type{});  // the last step (steps is even, so it is odd)

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

// Routed tiles of fp8 experts: A is the tile's fp8 activation rows (x_q by
// token for up, H_q by slot for down; quantized per row beforehand), B the
// expert's fp8 weights, v_mfma_f32_16x16x32_fp8_fp8 (exact fp8 products, fp32
// sums). Same tile, waves and pipeline as gemm_tile; one 16-row x 32-column
// sub-tile of either operand is 512 B in fragment order (lane l's 8 bytes,
// row l % 16, columns 8 (l / 16).., at 8 l), so staging writes and fragment
// reads are both contiguous. The epilogue scales by both row scales and
// rounds to bf16 where the fp8 matmul of the pages returns bf16: the two
// up-projections, then the SwiGLU product (bf16 H); down: the expert output.
template <bool UP>
__device__ __forceinline__ void gemm_tile_fp8(const GroupedGemmArgs& a, const Tile& tile, int nt,
                                              uint8_t* lds) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr int SUB = 512;                  // bytes per 16 x 32 fp8 sub-tile
    constexpr int ASUB = BM / 16;             // 8 A sub-tiles
    constexpr int STAGE_BYTES = (ASUB + 16) * SUB;
    const int64_t K = a.K, N = a.N;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int64_t n0 = static_cast<int64_t>(nt) * (UP ? BN / 2 : BN);
    const int64_t ng = K / kGroup;
    const int steps = static_cast<int>(K / BK);

    // ---- A: this wave stages sub-tiles 2 wid, 2 wid + 1 (rows 32 wid + 16 i + r16)
    const uint8_t* arow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int r = 32 * wid + 16 * i + r16;
        r = r < tile.nrows ? r : tile.nrows - 1;
        const int64_t s = tile.row0 + r;
        const int64_t src = UP ? a.perm[s] / a.top_k : s;
        arow[i] = a.a8 + src * K + 8 * q4;
    }
    // ---- B: this wave stages sub-tiles 4 wid .. 4 wid + 3 (B rows 16 j + r16)
    const uint8_t* brow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int br = 16 * (4 * wid + i) + r16;
        int64_t bn = UP ? n0 + (br & 127) : n0 + br;
        bn = bn < N ? bn : N - 1;
        const uint8_t* m = ((UP && br >= 128) ? a.wf1 : a.wf0) + static_cast<int64_t>(tile.group) * N * K;
        brow[i] = m + (bn >> 4) * ng * 2048 + (bn & 15) * 32 + 8 * q4;  // + group*2048 + step*512
    }

    u32x2 ra0[2], rb0[4], ra1[2], rb1[4];
    auto load_step = [&](u32x2 (&ra)[2], u32x2 (&rb)[4], int k) __attribute__((always_inline)) {
        k = k < steps ? k : steps - 1;
        const int64_t k0 = static_cast<int64_t>(k) * BK;
#pragma unroll
        for (int i = 0; i < 2; ++i) ra[i] = *reinterpret_cast<const u32x2*>(arow[i] + k0);
        const int64_t boff = (k0 / kGroup) * 2048 + (k & 3) * 512;
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = *reinterpret_cast<const u32x2*>(brow[i] + boff);
    };
    auto store_step = [&](const u32x2 (&ra)[2], const u32x2 (&rb)[4], int stage)
                          __attribute__((always_inline)) {
        uint8_t* st = lds + stage * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *reinterpret_cast<u32x2*>(st + (2 * wid + i) * SUB + lane * 8) = ra[i];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x2*>(st + (ASUB + 4 * wid + i) * SUB + lane * 8) = rb[i];
    };

    f32x4 acc[4][8];
    int sb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sb[j] = UP ? ((j < 4) ? wn * 4 + j : 8 + wn * 4 + (j - 4)) : wn * 8 + j;
    auto mfma_step = [&](int stage, auto first) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first)::value;
        const uint8_t* st = lds + stage * STAGE_BYTES;
        long fa[4], fb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) fb[j] = *reinterpret_cast<const long*>(st + (ASUB + sb[j]) * SUB + lane * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const long*>(st + (wm * 4 + i) * SUB + lane * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                    fa[i], fb[j], FIRST ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);
    };

    load_step(ra0, rb0, 0);
    load_step(ra1, rb1, 1);
    store_step(ra0, rb0, 0);
    __syncthreads();
    load_step(ra0, rb0, 2);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(0, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    store_step(ra1, rb1, 1);
    __syncthreads();
    int k = 1;
    for (; k + 1 < steps; k += 2) {
        load_step(ra1, rb1, k + 2);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(1, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        store_step(ra0, rb0, 0);
        __syncthreads();
        load_step(ra0, rb0, k + 3);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(0, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        store_step(ra1, rb1, 1);
        __syncthreads();
    }
    mfma_step(1, std::false_type{});

    // ---- epilogue: D[row][col], row = 4 * lq + r inside a 16 x 16 sub-tile, col = l16
    const int l16 = lane & 15, lq = lane >> 4;
    const float* ws0 = a.wfs0 + static_cast<int64_t>(tile.group) * N;
    const float* ws1 = UP ? a.wfs1 + static_cast<int64_t>(tile.group) * N : nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wm * 64 + i * 16 + lq * 4 + r;
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

template <bool UP>
__global__ __launch_bounds__(NT, 2) void grouped_gemm_kernel(GroupedGemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // 3 stages of [A | B]

    // ---- block -> (row tile, column tile), XCD-aware (see the file comment)
    const int ncol = static_cast<int>(UP ? a.N / (BN / 2) : (a.N + BN - 1) / BN);
    // kTilesRouted: the routed tiles only (they lead the table)
    const int nrow = a.tile_base[a.tile_mode == kTilesRouted ? a.E : a.E + 1];
    constexpr int kGroupRows = 8;
    int lin;
    if (!xcd_tile(blockIdx.x, static_cast<int64_t>(a.tile_base[a.E]) * ncol, static_cast<int64_t>(nrow) * ncol,
                  tile_weight(a), lin))
        return;
    const int span = kGroupRows * ncol;
    const int first_row = (lin / span) * kGroupRows;
    const int rows_here = nrow - first_row < kGroupRows ? nrow - first_row : kGroupRows;
    const int mt = first_row + (lin % span) % rows_here;
    const int nt = (lin % span) / rows_here;

    Tile tile;
    if (!find_tile<BM>(a, mt, tile)) return;
    if (tile.group < a.E && a.wf0) gemm_tile_fp8<UP>(a, tile, nt, lds);
    else if (tile.group < a.E && !a.wb0 && tile.nrows <= BM / 2) gemm_tile<UP, true, 2>(a, tile, nt, lds);
    else if (tile.group < a.E && !a.wb0) gemm_tile<UP, true>(a, tile, nt, lds);
    else gemm_tile<UP, false>(a, tile, nt, lds);
}

static unsigned max_row_tiles(const GroupedGemmArgs& a) {
    // each routed expert adds at most one partial tile beyond P / BM
    const int64_t e_bound = a.E < a.P ? a.E : a.P;
    const int64_t shared = a.tile_mode == kTilesRouted ? 0 : (a.T + BM - 1) / BM;
    return static_cast<unsigned>((a.P + BM - 1) / BM + e_bound + shared);
}

static constexpr size_t kGemmLds = 2 * 24 * 1024;  // 2 stages of 8 A + 16 B sub-tiles

// more than 64 KB of dynamic LDS must be allowed per kernel once
template <bool UP>
static hipError_t allow_lds() {
    static hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_kernel<UP>),
                                              hipFuncAttributeMaxDynamicSharedMemorySize,
                                              static_cast<int>(kGemmLds));
    return e;
}

hipError_t launch_grouped_up(const GroupedGemmArgs& a, hipStream_t stream) {
    if (hipError_t e = allow_lds<true>(); e != hipSuccess) return e;
    dim3 grid(xcd_grid(static_cast<int64_t>(max_row_tiles(a)) * (a.N / (BN / 2)), tile_weight(a)));
    MOE_LAUNCH(grouped_gemm_kernel<true>, grid, dim3(NT), kGemmLds, stream, a);
    return hipGetLastError();
}

hipError_t launch_grouped_down(const GroupedGemmArgs& a, hipStream_t stream) {
    if (hipError_t e = allow_lds<false>(); e != hipSuccess) return e;
    dim3 grid(xcd_grid(static_cast<int64_t>(max_row_tiles(a)) * ((a.N + BN - 1) / BN), tile_weight(a)));
    MOE_LAUNCH(grouped_gemm_kernel<false>, grid, dim3(NT), kGemmLds, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- combine (K6c)
// y[t] = O[P + t] + sum_j gate[t, j] * O[inv[t * k + j]], j ascending, fp32, then
// bf16 (round to nearest even). One thread per 4 consecutive columns.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ O,
                                                      const float* __restrict__ O2,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ inv, int64_t T,
                                                      int64_t P, int top_k, int64_t d,
                                                      uint16_t* __restrict__ y) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t per_row = d / 4;
    if (q >= T * per_row) return;
    const int64_t t = q / per_row;
    const int64_t c = (q - t * per_row) * 4;
    // a row of O, plus its second partial sums when the down projection split
    // its reduction (added first, in this fixed order)
    auto row = [&](int64_t r) {
        float4 v = *reinterpret_cast<const float4*>(O + r * d + c);
        if (O2) {
            const float4 w = *reinterpret_cast<const float4*>(O2 + r * d + c);
            v.x += w.x;
            v.y += w.y;
            v.z += w.z;
            v.w += w.w;
        }
        return v;
    };
    float4 acc = row(P + t);
    for (int j = 0; j < top_k; ++j) {
        const float g = gates[t * top_k + j];
        const int64_t slot = inv[t * top_k + j];
        const float4 o = row(slot);
        acc.x = fmaf(g, o.x, acc.x);
        acc.y = fmaf(g, o.y, acc.y);
        acc.z = fmaf(g, o.z, acc.z);
        acc.w = fmaf(g, o.w, acc.w);
    }
    uint2 out;
    out.x = pack_bf16x2(acc.x, acc.y);
    out.y = pack_bf16x2(acc.z, acc.w);
    *reinterpret_cast<uint2*>(y + t * d + c) = out;
}

hipError_t launch_combine(const float* O, const float* O2, const float* gates, const int32_t* inv,
                          int64_t T, int64_t P, int top_k, int64_t d, uint16_t* y, hipStream_t stream) {
    const int64_t n = T * (d / 4);
    MOE_LAUNCH(combine_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       stream, O, O2, gates, inv, T, P, top_k, d, y);
    return hipGetLastError();
}

}  // namespace moe
