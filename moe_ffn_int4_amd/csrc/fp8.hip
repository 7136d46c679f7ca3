// fp8.hip -- row-wise fp8 (E4M3) quantization for the fp8 routed-expert path.
//
// The lshu.cn page "Llama 4 单卡量化推理与选型指南" (section "量化环节")
// shows the fp8 branch of bmm_nt: each activation row is quantized to fp8 on
// the fly, with its scale bounded by activation_scale_ub, and the weights are
// fp8 with one scale per row ("FP8 行级", section "三条推理路径差异").
// Both quantizers here compute, per row of K values,
//   scale = min(max(max|v|, 1e-12), ub) / 448     (no bound for weights)
//   code  = fp8(clamp(v / scale, -448, 448))
// in fp32 with a correctly rounded division (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt) and gfx950's v_cvt_pk_fp8_f32,
// which rounds to the nearest OCP E4M3 value, ties to even.
//
// One block per row: the row maximum is reduced across the block, then the
// row is converted, 4 consecutive values per thread (one 32-bit store of 4
// codes), from registers where the row fits them, else read again (from L2). HBM-bound: weights read 4 B and write 1 B
// per value (+ 4 B per row); activations read 2 B and write 1 B.
//
// Weight codes go to the tiled order the forward pass reads: tile
// t = (row/16) * (K/128) + k/128 is 2 KB, stored as 4 steps of 32 columns,
// byte t*2048 + ((k%128)/32)*512 + (row%16)*32 + k%32, so one MFMA step of 16
// rows is a contiguous 512 bytes. Activation codes stay row-major.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int NT = 256;
constexpr float kFp8Max = 448.0f;
constexpr float kTiny = 1e-12f;
constexpr int64_t kFp8WideRowsBelow = 512;  // activation rows taking 1024-thread blocks

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_to_f32(static_cast<uint16_t>(u.x & 0xFFFF)),
                       bf16_to_f32(static_cast<uint16_t>(u.x >> 16)),
                       bf16_to_f32(static_cast<uint16_t>(u.y & 0xFFFF)),
                       bf16_to_f32(static_cast<uint16_t>(u.y >> 16)));
}
}  // namespace

// SRC = float (weights, tiled codes) or uint16_t (bf16 activations, row-major
// codes); ub > 0 bounds the row maximum. NB threads per row; rows of at most
// 4 * NB * R values keep their values in registers between the two passes,
// longer rows read them again (from L2).
template <typename SRC, bool TILED, int NB, int R>
__global__ __launch_bounds__(NB) void quantize_fp8_rows_kernel(const SRC* __restrict__ src, int64_t K,
                                                               float ub, uint8_t* __restrict__ q,
                                                               float* __restrict__ scales) {
    constexpr int NW = NB / 64;
    __shared__ float red[NW];
    const int64_t row = blockIdx.x;
    const SRC* r = src + row * K;
    const int tid = threadIdx.x;
    const bool held = K <= 4 * NB * R;
    float4 hv[R];
    float m = 0.f;
    if (held) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t k = 4 * (tid + i * NB);
            hv[i] = k < K ? load4(r + k) : make_float4(0.f, 0.f, 0.f, 0.f);
            m = fmaxf(m, fmaxf(fmaxf(fabsf(hv[i].x), fabsf(hv[i].y)),
                               fmaxf(fabsf(hv[i].z), fabsf(hv[i].w))));
        }
    } else {
        for (int64_t k = 4 * tid; k < K; k += 4 * NB) {
            const float4 v = load4(r + k);
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    }
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = fmaxf(m, red[i]);
    m = fmaxf(m, kTiny);
    if (ub > 0.f) m = fminf(m, ub);
    const float s = m / kFp8Max;
    if (tid == 0) scales[row] = s;
    auto put = [&](const float4 v, int64_t k) __attribute__((always_inline)) {
        const float a = fminf(fmaxf(v.x / s, -kFp8Max), kFp8Max);
        const float b = fminf(fmaxf(v.y / s, -kFp8Max), kFp8Max);
        const float c = fminf(fmaxf(v.z / s, -kFp8Max), kFp8Max);
        const float d = fminf(fmaxf(v.w / s, -kFp8Max), kFp8Max);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
        int64_t at;
        if (TILED) {
            const int64_t t = (row >> 4) * (K / kGroup) + k / kGroup;
            at = t * 2048 + ((k % kGroup) >> 5) * 512 + (row & 15) * 32 + (k & 31);
        } else {
            at = row * K + k;
        }
        *reinterpret_cast<int*>(q + at) = w;
    };
    if (held) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t k = 4 * (tid + i * NB);
            if (k < K) put(hv[i], k);
        }
    } else {
        for (int64_t k = 4 * tid; k < K; k += 4 * NB) put(load4(r + k), k);
    }
}

hipError_t launch_quantize_fp8_weights(const float* w, int64_t rows, int64_t K, uint8_t* q,
                                       float* scales, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    MOE_LAUNCH((quantize_fp8_rows_kernel<float, true, NT, 1>), dim3(static_cast<unsigned>(rows)),
                       dim3(NT), 0, stream, w, K, 0.f, q, scales);
    return hipGetLastError();
}

// activations, the row held in registers up to K = 8192: a decode batch of a
// few rows takes 1024 threads per row; thousands of prefill rows take 256, so
// more rows are in flight per CU. Per step for x and H (three alternating
// rounds): 16 rows 8.4 us (10.2 us at 256 threads re-reading the row); 8192
// rows 69.5 us (85.3 us re-reading, 98.9 us at 1024 threads)
hipError_t launch_quantize_fp8_activations(const uint16_t* x, int64_t rows, int64_t K, float ub,
                                           uint8_t* q, float* scales, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if (rows < kFp8WideRowsBelow)
        MOE_LAUNCH((quantize_fp8_rows_kernel<uint16_t, false, 1024, 2>),
                   dim3(static_cast<unsigned>(rows)), dim3(1024), 0, stream, x, K, ub, q, scales);
    else
        MOE_LAUNCH((quantize_fp8_rows_kernel<uint16_t, false, NT, 8>),
                   dim3(static_cast<unsigned>(rows)), dim3(NT), 0, stream, x, K, ub, q, scales);
    return hipGetLastError();
}

}  // namespace moe
