// gemm.hip -- K4/K5/K6: grouped expert GEMMs on gfx950 bf16 MFMA.
//
// Every chosen expert runs its SwiGLU FFN only on the tokens routed to it
// (discosf.com page "1 卡跑通 Llama 4", section "混合专家路由"), and the
// shared expert runs on every token. The expert FFN is
// (Swish(x W1^T) * (x W3^T)) W2^T (docs.ifdog.com page "Llama 开源模型系列",
// section "SwiGLU：门控激活的数学"). Routed weights are int4 with one fp32
// scale per 128 weights of a row and dequantize symmetrically as code * scale
// (lshu.cn page, section "量化环节": zero-points are all zero).
//
// One launch covers all groups: routed experts 0..E-1 (int4 weights, rows =
// the expert's slots from the dispatch step) and the shared expert as group E
// (bf16 weights, rows = all T tokens). blockIdx.x walks the row tiles of all
// groups (tile_base from the dispatch step), blockIdx.y the output columns.
//
//   up:   H[slot, n]  = silu(A W1^T)[n] * (A W3^T)[n]  (bf16 out)
//         A = x gathered by slot (routed) or x itself (shared)
//         a block computes 64 hidden units of W1 and the same 64 of W3, so
//         the SwiGLU product is formed in registers
//   down: O[slot, m]  = (H W2^T)[m]                    (fp32 out)
//
// Tiles: 128 rows x 128 columns x 128 reduction (one quantization group) per
// step, 256 threads = 4 waves in a 2 x 2 grid, each wave 64 x 64 from 4 x 4
// v_mfma_f32_16x16x32_bf16. A and B are staged through LDS (rows padded by 16
// bytes so the 16-byte fragment reads are bank-conflict free). Weights come in
// the tiled layouts (moe_quantize_int4_tiled / moe_pack_bf16_tiled): per step
// the block reads eight whole 16-row tiles, 1 KB (int4) or 4 KB (bf16) each.
// Int4 B rows are dequantized on the way into LDS: each thread takes 64 codes
// of one row (32 bytes), sign-extends the nibbles, multiplies by the group
// scale in fp32 and rounds to bf16 (round to nearest even). Accumulation is
// fp32 in the MFMA.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int BM = kPrefillBM;  // 128 rows (tokens / slots)
constexpr int BN = 128;         // B rows staged per block (output columns)
constexpr int BK = kGroup;      // reduction step: one quantization group
constexpr int LDK = BK + 8;     // LDS row pitch in bf16 elements
constexpr int NT = 256;
}  // namespace

struct Tile {
    int group;
    int64_t row0;
    int nrows;
};

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

// 8 int4 codes (one 32-bit word) times scale -> 4 packed bf16 pairs
__device__ __forceinline__ void dequant8(uint32_t w, float s, uint32_t* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        out[j] = pack_bf16x2(static_cast<float>(nib(w, 2 * j)) * s,
                             static_cast<float>(nib(w, 2 * j + 1)) * s);
}

template <bool UP>
__global__ __launch_bounds__(NT) void grouped_gemm_kernel(GroupedGemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];

    Tile tile;
    if (!find_tile(a, blockIdx.x, tile)) return;
    const bool routed = tile.group < a.E;
    const int64_t K = a.K, N = a.N;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const int wm = wid >> 1, wn = wid & 1;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * (UP ? BN / 2 : BN);

    // ---- A rows this thread stages: rows (tid + 256 i) / 16, 16-byte column piece (tid & 15)
    constexpr int AP = BM * BK / 8 / NT;  // 16-byte pieces per thread
    const uint16_t* arow[AP];
#pragma unroll
    for (int i = 0; i < AP; ++i) {
        const int r = (tid + NT * i) >> 4;
        arow[i] = nullptr;
        if (r < tile.nrows) {
            const int64_t s = tile.row0 + r;
            int64_t src;
            if (UP) src = routed ? a.perm[s] / a.top_k : s - a.P;
            else src = s;
            arow[i] = a.a + src * K + (tid & 15) * 8;
        }
    }

    // ---- B: LDS row r (0..127) is weight row n0 + (r & 63) of W1 / W3 (up) or
    // n0 + r of W2 (down). Tiles of one 16-row block are consecutive, ng per block.
    const int64_t ng = K / kGroup;
    auto row_block = [&](int r) -> int64_t {  // global 16-row block of LDS row r
        const int64_t n = UP ? n0 + (r & 63) : n0 + r;
        return n >> 4;
    };
    // int4: thread -> LDS row tid/2, 64 codes (32 bytes) at half (tid & 1)
    const int qr = tid >> 1, qh = tid & 1;
    const uint8_t* bq = nullptr;
    const float* bs = nullptr;
    // bf16: thread -> piece tid of each of the 8 row blocks' 4 KB tiles
    const uint16_t* bh[8];
    if (routed) {
        const int64_t rb = static_cast<int64_t>(tile.group) * (N / 16) + row_block(qr);
        const uint8_t* q = (UP && qr >= 64) ? a.wq1 : a.wq0;
        const float* sc = (UP && qr >= 64) ? a.ws1 : a.ws0;
        bq = q + rb * ng * 1024 + (qr & 15) * 64 + qh * 32;
        bs = sc + rb * ng * 16 + (qr & 15);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint16_t* src = (UP && i >= 4) ? a.sh1 : a.sh0;
            bh[i] = src + row_block(i * 16) * ng * 2048 + tid * 8;
        }
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // B-fragment row of sub-tile j inside Bs (up: cols 0,1 -> W1 rows, 2,3 -> W3 rows)
    int brow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        brow[j] = UP ? ((j < 2) ? wn * 32 + j * 16 : 64 + wn * 32 + (j - 2) * 16) + l16
                     : wn * 64 + j * 16 + l16;

    for (int64_t g = 0; g < ng; ++g) {
        const int64_t k0 = g * BK;
        uint4 av[AP];
#pragma unroll
        for (int i = 0; i < AP; ++i)
            av[i] = arow[i] ? *reinterpret_cast<const uint4*>(arow[i] + k0) : make_uint4(0, 0, 0, 0);
        uint4 bv[8];
        float scale = 0.f;
        if (routed) {
            bv[0] = *reinterpret_cast<const uint4*>(bq + g * 1024);
            bv[1] = *reinterpret_cast<const uint4*>(bq + g * 1024 + 16);
            scale = bs[g * 16];
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) bv[i] = *reinterpret_cast<const uint4*>(bh[i] + g * 2048);
        }
        __syncthreads();  // previous step's fragments are consumed
#pragma unroll
        for (int i = 0; i < AP; ++i) {
            const int r = (tid + NT * i) >> 4;
            *reinterpret_cast<uint4*>(&As[r * LDK + (tid & 15) * 8]) = av[i];
        }
        if (routed) {
            uint32_t d[32];
            const uint32_t w[8] = {bv[0].x, bv[0].y, bv[0].z, bv[0].w, bv[1].x, bv[1].y, bv[1].z, bv[1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) dequant8(w[i], scale, d + 4 * i);
            uint4* dst = reinterpret_cast<uint4*>(&Bs[qr * LDK + qh * 64]);
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[i] = make_uint4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]);
        } else {
            // piece tid of a step-major tile: step tid/64, row (tid/4)%16, columns 8*(tid%4)
            const int step = tid >> 6, row = (tid >> 2) & 15, col = step * 32 + (tid & 3) * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<uint4*>(&Bs[(i * 16 + row) * LDK + col]) = bv[i];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + i * 16 + l16) * LDK + kk + lq * 8]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const bf16x8*>(&Bs[brow[j] * LDK + kk + lq * 8]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }

    // ---- epilogue: D[row][col], row = 4 * lq + r inside a 16 x 16 sub-tile, col = l16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wm * 64 + i * 16 + lq * 4 + r;
            if (row >= tile.nrows) continue;
            const int64_t orow = tile.row0 + row;
            if (UP) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float g = acc[i][j][r], u = acc[i][j + 2][r];
                    const int64_t col = n0 + wn * 32 + j * 16 + l16;
                    a.h_out[orow * N + col] = f32_to_bf16(siluf_(g) * u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t col = n0 + wn * 64 + j * 16 + l16;
                    a.o_out[orow * N + col] = acc[i][j][r];
                }
            }
        }
    }
}

static unsigned max_row_tiles(const GroupedGemmArgs& a) {
    // each routed expert adds at most one partial tile beyond P / BM
    const int64_t e_bound = a.E < a.P ? a.E : a.P;
    return static_cast<unsigned>((a.P + BM - 1) / BM + e_bound + (a.T + BM - 1) / BM);
}

hipError_t launch_grouped_up(const GroupedGemmArgs& a, hipStream_t stream) {
    dim3 grid(max_row_tiles(a), static_cast<unsigned>(a.N / (BN / 2)));
    hipLaunchKernelGGL(grouped_gemm_kernel<true>, grid, dim3(NT), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_grouped_down(const GroupedGemmArgs& a, hipStream_t stream) {
    dim3 grid(max_row_tiles(a), static_cast<unsigned>(a.N / BN));
    hipLaunchKernelGGL(grouped_gemm_kernel<false>, grid, dim3(NT), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- combine (K6c)
// y[t] = O[P + t] + sum_j gate[t, j] * O[inv[t * k + j]], j ascending, fp32, then
// bf16 (round to nearest even). One thread per 4 consecutive columns.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ O,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ inv, int64_t T,
                                                      int64_t P, int top_k, int64_t d,
                                                      uint16_t* __restrict__ y) {
    const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t per_row = d / 4;
    if (q >= T * per_row) return;
    const int64_t t = q / per_row;
    const int64_t c = (q - t * per_row) * 4;
    float4 acc = *reinterpret_cast<const float4*>(O + (P + t) * d + c);
    for (int j = 0; j < top_k; ++j) {
        const float g = gates[t * top_k + j];
        const int64_t slot = inv[t * top_k + j];
        const float4 o = *reinterpret_cast<const float4*>(O + slot * d + c);
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

hipError_t launch_combine(const float* O, const float* gates, const int32_t* inv, int64_t T,
                          int64_t P, int top_k, int64_t d, uint16_t* y, hipStream_t stream) {
    const int64_t n = T * (d / 4);
    hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                       stream, O, gates, inv, T, P, top_k, d, y);
    return hipGetLastError();
}

}  // namespace moe
