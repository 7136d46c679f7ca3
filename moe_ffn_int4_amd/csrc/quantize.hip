// quantize.hip -- K1: int4 group quantizer for gfx950.
//
// Computes int4_row_quantize as printed on the discosf.com page
// "1 卡跑通 Llama 4", section "FP8 / Int4 混合量化": per group of 128
// consecutive fp32 weights (its group_size argument; 64 and 32 are the
// smaller groups the lshu.cn page expects next), scale = max(max|w|, 1e-6) / 8
// and code = clamp(round_half_even(w / scale), -8, 7).
//
// Bound by HBM: 4 bytes read and 0.5 + 4/group bytes written per weight.
// Mapping: one wave per 16-row x 128-column tile of w (8 KB of fp32), all of
// it requested at once: load i brings rows 2i and 2i+1 (two whole 512-byte
// row segments, one float4 per lane), so lane l holds columns 4(l%32) .. +3
// of rows 2i + l/32. A group's max is a reduction over its group / 4 aligned
// lanes: DPP swaps inside quads and the 8- and 16-lane mirrors, and one
// lane ^ 16 shuffle for groups of 128 (the group size is a template argument,
// so the steps unroll; a runtime loop of five LDS permutes per row cost
// 40.2 against 33.8 us on an 8192 x 5120 matrix). The codes round the
// IEEE correctly rounded quotient (the library is compiled with
// -fhip-fp32-correctly-rounded-divide-sqrt and no fast-math) half to even
// (rintf): each weight is first multiplied by the scale's approximate
// reciprocal, and only a product near a rounding boundary takes the IEEE
// division, so codes and scales are bit-identical to the fp32 definition at
// a fraction of the division's VALU cost. The tile's codes (1 KB) and scales gather in LDS, and each lane
// then stores one whole 16-byte piece, so every output line is written once,
// in full.
//
// TILED = true writes the storage order the forward pass reads: tile
// t = (row/16) * (K/128) + k/128 holds those 128 columns of 16 rows (1 KB) as
// four 32-column steps of 16 rows x 16 bytes, and their 16 x (128 / group)
// scales, scale s of row r at t*16*S + (r%16)*S + s (S = 128 / group): one
// wavefront access covers one tile, one GEMM step of 16 rows is 256
// contiguous bytes. Row-major output: row r's 128 columns of tile column g are
// bytes r*K/2 + 64 g .. + 63.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int kQuantWaves = 4;  // waves (tiles in flight) per block
// distance to a rounding boundary below which the quotient is computed
// exactly: 8 ulp of 8.0 (v_rcp_f32 is within 1 ulp, the product adds 1/2)
constexpr float kNearHalf = 8.0f * 9.5367431640625e-7f;
}

// max over the G / 4 lanes of a group (32, 16 or 8 aligned lanes), in the
// same ternary form as a sequential scan (the maximum is exact in any order):
// swaps inside quads, then the 8-lane and 16-lane mirrors, then lane ^ 16
template <int CTRL>
__device__ __forceinline__ float max_dpp(float m) {
    const float o = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, m), CTRL, 0xF, 0xF, false));
    return o > m ? o : m;
}
template <int G>
__device__ __forceinline__ float group_max(float m) {
    m = max_dpp<0xB1>(m);   // quad_perm [1,0,3,2]: lane ^ 1
    m = max_dpp<0x4E>(m);   // quad_perm [2,3,0,1]: lane ^ 2
    m = max_dpp<0x141>(m);  // row_half_mirror: the other quad of 8 lanes
    if (G >= 64) m = max_dpp<0x140>(m);  // row_mirror: the other 8 of 16 lanes
    if (G == 128) {
        const float o = __shfl_xor(m, 16, 64);
        m = o > m ? o : m;
    }
    return m;
}

template <bool TILED, int G>
__global__ __launch_bounds__(256) void quantize_int4_kernel(const float* __restrict__ w, int64_t rows,
                                                            int64_t K, uint8_t* __restrict__ q,
                                                            float* __restrict__ scales) {
    // per wave: the tile's codes in tiled order (step s, row r at s*256 + r*16)
    // and its 16 x S scales
    __shared__ __attribute__((aligned(16))) uint8_t code_lds[kQuantWaves][1024];
    __shared__ float scale_lds[kQuantWaves][64];
    constexpr int S = kGroup / G, lanes = G / 4;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int half = lane >> 5, c4 = lane & 31;
    const int64_t ng = K / kGroup;
    const int64_t ntiles = (rows + 15) / 16 * ng;
    // every wave of a block runs the same iterations (block-wide barriers)
    for (int64_t tb = static_cast<int64_t>(blockIdx.x) * kQuantWaves; tb < ntiles;
         tb += static_cast<int64_t>(gridDim.x) * kQuantWaves) {
        const int64_t t = tb + wv;
        const bool tv = t < ntiles;
        const int64_t rb = tv ? t / ng : 0, g = tv ? t - rb * ng : 0;
        f32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t row = rb * 16 + 2 * i + half;
            v[i] = (tv && row < rows)
                       ? __builtin_nontemporal_load(
                             reinterpret_cast<const f32x4*>(w + row * K + g * kGroup + c4 * 4))
                       : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 2 * i + half;
            const float m = group_max<G>(
                fmaxf(fmaxf(fabsf(v[i][0]), fabsf(v[i][1])), fmaxf(fabsf(v[i][2]), fabsf(v[i][3]))));
            const float s = (m < 1e-6f ? 1e-6f : m) / 8.0f;
            const float rs = __builtin_amdgcn_rcpf(s);
            // round(w / s): the product with the approximate reciprocal is
            // within 3 ulp of w / s (|w / s| <= 8), so its rounding agrees
            // with that of the correctly rounded quotient unless it lies
            // within kNearHalf of a rounding boundary n + 1/2; there the IEEE
            // division decides (one test per row, the rare fix-up per value)
            float c[4];
            bool near = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float qa = v[i][j] * rs;
                c[j] = rintf(qa);
                near |= fabsf(fabsf(qa - c[j]) - 0.5f) < kNearHalf;
            }
            if (near) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float qa = v[i][j] * rs;
                    if (fabsf(fabsf(qa - c[j]) - 0.5f) < kNearHalf) c[j] = rintf(v[i][j] / s);
                }
            }
            uint32_t packed = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // |w| <= max|w| <= 8 s, so the code is at least -8 (also
                // through the reciprocal, whose error rounds away); only 8
                // needs clamping (a NaN weight keeps its code 0)
                const float cj = c[j] > 7.0f ? 7.0f : c[j];
                packed |= (static_cast<uint32_t>(static_cast<int>(cj)) & 0xFu) << (4 * j);
            }
            // columns 4 c4 .. 4 c4 + 3 sit in step c4 / 8, bytes 2 (c4 % 8) .. + 1
            *reinterpret_cast<uint16_t*>(&code_lds[wv][(c4 >> 3) * 256 + r * 16 + (c4 & 7) * 2]) =
                static_cast<uint16_t>(packed);
            if (c4 % lanes == 0) scale_lds[wv][r * S + c4 / lanes] = s;
        }
        __syncthreads();
        if (tv) {
            if (TILED) {
                // lane l: step l / 16, row l % 16 -- the tile's 1 KB in order
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&code_lds[wv][lane * 16]),
                                            reinterpret_cast<u32x4*>(q + t * 1024 + lane * 16));
                if (lane < 16 * S) scales[t * 16 * S + lane] = scale_lds[wv][lane];
            } else {
                // lane l: row l / 4, columns 32 (l % 4) .. + 31 of the tile
                const int r = lane >> 2, p = lane & 3;
                const int64_t row = rb * 16 + r;
                if (row < rows)
                    __builtin_nontemporal_store(
                        *reinterpret_cast<const u32x4*>(&code_lds[wv][p * 256 + r * 16]),
                        reinterpret_cast<u32x4*>(q + row * (K / 2) + g * 64 + p * 16));
                if (lane < 16 * S) {
                    const int64_t srow = rb * 16 + lane / S;
                    if (srow < rows) scales[srow * (K / G) + g * S + lane % S] = scale_lds[wv][lane];
                }
            }
        }
        __syncthreads();
    }
}

hipError_t launch_quantize_int4(const float* w, int64_t rows, int64_t K, int group, uint8_t* q,
                                float* scales, bool tiled, hipStream_t stream) {
    const int64_t ntiles = (rows + 15) / 16 * (K / kGroup);
    if (ntiles == 0) return hipSuccess;
    if (group != 128 && group != 64 && group != 32) return hipErrorInvalidValue;
    const int64_t want = (ntiles + kQuantWaves - 1) / kQuantWaves;
    const int blocks = static_cast<int>(want < 16384 ? want : 16384);
#define MOE_QUANT_LAUNCH(TL, G)                                                                 \
    MOE_LAUNCH((quantize_int4_kernel<TL, G>), dim3(blocks), dim3(256), 0, stream, w, rows, K, q, \
               scales)
    if (tiled) {
        if (group == 128) MOE_QUANT_LAUNCH(true, 128);
        else if (group == 64) MOE_QUANT_LAUNCH(true, 64);
        else MOE_QUANT_LAUNCH(true, 32);
    } else {
        if (group == 128) MOE_QUANT_LAUNCH(false, 128);
        else if (group == 64) MOE_QUANT_LAUNCH(false, 64);
        else MOE_QUANT_LAUNCH(false, 32);
    }
#undef MOE_QUANT_LAUNCH
    return hipGetLastError();
}

// Row-major int4 (the quantizer's row-major output) -> the tiled order, one
// wave per tile: lane l moves the 16-byte piece of step l / 16, row l % 16
// (bytes 64 g + 16 (l / 16) .. of the row) to byte 16 l of the tile, and
// lanes below 16 S move the tile's scales.
__global__ __launch_bounds__(256) void tile_int4_kernel(const uint8_t* __restrict__ q_rm,
                                                        const float* __restrict__ s_rm, int64_t rows,
                                                        int64_t K, int group, uint8_t* __restrict__ q_t,
                                                        float* __restrict__ s_t) {
    const int lane = threadIdx.x & 63;
    const int64_t ng = K / kGroup;
    const int64_t ntiles = rows / 16 * ng;
    const int S = kGroup / group;
    for (int64_t t = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6; t < ntiles;
         t += (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6) {
        const int64_t rb = t / ng, g = t - rb * ng;
        const int64_t row = rb * 16 + (lane & 15);
        const u32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(q_rm + row * (K / 2) + g * 64 + (lane >> 4) * 16));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(q_t + t * 1024 + lane * 16));
        if (lane < 16 * S)
            s_t[t * 16 * S + lane] = s_rm[(rb * 16 + lane / S) * (K / group) + g * S + lane % S];
    }
}

hipError_t launch_tile_int4(const uint8_t* q_rm, const float* s_rm, int64_t rows, int64_t K, int group,
                            uint8_t* q_t, float* s_t, hipStream_t stream) {
    const int64_t ntiles = rows / 16 * (K / kGroup);
    if (ntiles == 0) return hipSuccess;
    const int64_t want = (ntiles + 3) / 4;
    const int blocks = static_cast<int>(want < 16384 ? want : 16384);
    MOE_LAUNCH(tile_int4_kernel, dim3(blocks), dim3(256), 0, stream, q_rm, s_rm, rows, K, group, q_t, s_t);
    return hipGetLastError();
}

// bf16 [rows, K] -> tiles of 16 rows x 128 columns stored as 4 steps of 32
// columns (the B-operand order of one 16x16x32 MFMA step per 1 KB). One
// thread per destination 16-byte piece; reads and writes are both 16 bytes.
__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint4* __restrict__ src, int64_t K,
                                                        int64_t n16, uint4* __restrict__ dst) {
    const int64_t ng = K / kGroup;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; j < n16;
         j += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t t = j >> 8;           // 256 pieces per tile
        const int within = static_cast<int>(j & 255);
        const int step = within >> 6, row = (within >> 2) & 15, piece = within & 3;
        const int64_t rb = t / ng, g = t - rb * ng;
        const int64_t k = g * kGroup + step * 32 + piece * 8;
        dst[j] = src[((rb * 16 + row) * K + k) / 8];
    }
}

hipError_t launch_pack_bf16(const uint16_t* src, int64_t rows, int64_t K, uint16_t* dst,
                            hipStream_t stream) {
    const int64_t n16 = rows * K / 8;
    if (n16 == 0) return hipSuccess;
    const int64_t want = (n16 + 255) / 256;
    const int blocks = static_cast<int>(want < 16384 ? want : 16384);
    MOE_LAUNCH(pack_bf16_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(src), K, n16, reinterpret_cast<uint4*>(dst));
    return hipGetLastError();
}

}  // namespace moe
