// quantize.hip -- K1: int4 group quantizer for gfx950.
//
// Computes int4_row_quantize as printed on the discosf.com page
// "1 卡跑通 Llama 4", section "FP8 / Int4 混合量化": per group of 128
// consecutive fp32 weights (its group_size argument; 64 and 32 are the
// smaller groups the lshu.cn page expects next), scale = max(max|w|, 1e-6) / 8
// and code = clamp(round_half_even(w / scale), -8, 7).
//
// Bound by HBM: 4 bytes read and 0.5 + 4/128 bytes written per weight.
// Mapping: one half-wave (32 lanes) per 128 weights of a row, each lane one
// float4, so a wave reads 1 KB in one fully coalesced load and writes 2 x 64
// bytes of packed codes. A group's max is an xor-shuffle reduction over its
// group / 4 lanes (5 steps for 128, 4 for 64, 3 for 32). The division is IEEE
// correctly rounded (the library is compiled with
// -fhip-fp32-correctly-rounded-divide-sqrt and no fast-math), rintf maps to
// round-half-even, so codes and scales are bit-identical to the fp32
// definition.
//
// TILED = true writes the storage order the forward pass reads: tile
// t = (row/16) * (K/128) + k/128 holds those 128 columns of 16 rows (1 KB) as
// four 32-column steps of 16 rows x 16 bytes, and their 16 x (128 / group)
// scales, scale s of row r at t*16*S + (r%16)*S + s (S = 128 / group): one
// wavefront access covers one tile, one GEMM step of 16 rows is 256
// contiguous bytes.
#include "common.h"
#include "kernels.h"

namespace moe {

template <bool TILED>
__global__ __launch_bounds__(256) void quantize_int4_kernel(const float4* __restrict__ w,
                                                            int64_t ngroups, int64_t groups_per_row,
                                                            int group, uint16_t* __restrict__ q16,
                                                            float* __restrict__ scales) {
    // ngroups / groups_per_row count 128-weight units; a unit holds S groups
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5;
    const int hl = lane & 31;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;

    for (int64_t g0 = wave * 2; g0 < ngroups; g0 += nwaves * 2) {
        const int64_t g = g0 + half;
        const bool valid = g < ngroups;
        float4 v = valid ? w[g * 32 + hl] : make_float4(0.f, 0.f, 0.f, 0.f);
        float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        for (int off = group >> 3; off >= 1; off >>= 1) {  // lanes of one group
            float o = __shfl_xor(m, off, 64);
            m = o > m ? o : m;
        }
        const float s = (m < 1e-6f ? 1e-6f : m) / 8.0f;
        float e[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float c = rintf(e[i] / s);
            c = c < -8.0f ? -8.0f : (c > 7.0f ? 7.0f : c);
            packed |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xFu) << (4 * i);
        }
        if (valid) {
            int64_t at = g;  // row-major: unit g of the flattened [rows, K/128]
            if (TILED) {
                const int64_t r = g / groups_per_row, gg = g - r * groups_per_row;
                at = ((r >> 4) * groups_per_row + gg) * 16 + (r & 15);
            }
            // tiled: 32-column step (hl / 8) of the 16-row tile, then the row, then
            // this lane's 4 codes; row-major: the row's 64 bytes in order
            q16[TILED ? (at >> 4) * 512 + (hl >> 3) * 128 + (at & 15) * 8 + (hl & 7) : at * 32 + hl] =
                static_cast<uint16_t>(packed);
            const int lanes = group >> 2, S = kGroup / group;
            if (hl % lanes == 0) scales[at * S + hl / lanes] = s;
        }
    }
}

hipError_t launch_quantize_int4(const float* w, int64_t rows, int64_t K, int group, uint8_t* q,
                                float* scales, bool tiled, hipStream_t stream) {
    const int64_t ngroups = rows * (K / kGroup);
    if (ngroups == 0) return hipSuccess;
    const int64_t want = (ngroups + 7) / 8;  // 8 units per 256-thread block per pass
    const int blocks = static_cast<int>(want < 8192 ? want : 8192);
    if (tiled)
        MOE_LAUNCH(quantize_int4_kernel<true>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const float4*>(w), ngroups, K / kGroup, group,
                           reinterpret_cast<uint16_t*>(q), scales);
    else
        MOE_LAUNCH(quantize_int4_kernel<false>, dim3(blocks), dim3(256), 0, stream,
                           reinterpret_cast<const float4*>(w), ngroups, K / kGroup, group,
                           reinterpret_cast<uint16_t*>(q), scales);
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
