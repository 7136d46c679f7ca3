// quantize.hip -- K1: int4 group quantizer for gfx950.
//
// Computes int4_row_quantize as printed on the discosf.com page
// "1 卡跑通 Llama 4", section "FP8 / Int4 混合量化": per group of 128
// consecutive fp32 weights, scale = max(max|w|, 1e-6) / 8 and
// code = clamp(round_half_even(w / scale), -8, 7).
//
// Bound by HBM: 4 bytes read and 0.5 + 4/128 bytes written per weight.
// Mapping: one half-wave (32 lanes) per group, each lane one float4, so a
// wave reads two whole groups (1 KB) in one fully coalesced load and writes
// 2 x 64 bytes of packed codes. The group max is a 5-step xor-shuffle
// reduction inside the half-wave. The division is IEEE correctly rounded (the
// library is compiled with -fhip-fp32-correctly-rounded-divide-sqrt and no
// fast-math), rintf maps to round-half-even, so codes and scales are
// bit-identical to the fp32 definition.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void quantize_int4_kernel(const float4* __restrict__ w,
                                                            int64_t ngroups,
                                                            uint16_t* __restrict__ q16,
                                                            float* __restrict__ scales) {
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
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) {
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
            q16[g * 32 + hl] = static_cast<uint16_t>(packed);
            if (hl == 0) scales[g] = s;
        }
    }
}

hipError_t launch_quantize_int4(const float* w, int64_t rows, int64_t K, uint8_t* q,
                                float* scales, hipStream_t stream) {
    const int64_t ngroups = rows * (K / kGroup);
    if (ngroups == 0) return hipSuccess;
    const int64_t want = (ngroups + 7) / 8;  // 8 groups per 256-thread block per pass
    const int blocks = static_cast<int>(want < 8192 ? want : 8192);
    hipLaunchKernelGGL(quantize_int4_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(w), ngroups,
                       reinterpret_cast<uint16_t*>(q), scales);
    return hipGetLastError();
}

}  // namespace moe
