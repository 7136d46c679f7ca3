// router.hip -- K2: router logits, top-k selection and sigmoid gates (gfx950).
//
// The router of the discosf.com page "1 卡跑通 Llama 4", section "混合专家路由":
// every token scores every expert, and the top-k experts are chosen
// (torch.topk there). The score is a sigmoid gate of the logit; selection is
// on the logits (same order as the sigmoid), ties go to the lower expert id.
//
// Logits stay fp32 (the bf16 x widens exactly, router weights are fp32, fp32
// FMA accumulation): the choice of experts must not move with a cheaper
// precision, so this small GEMM runs on the vector ALUs, not on bf16 MFMA.
// Tiling: 32 tokens x 64 experts per 256-thread block, reduction staged through
// LDS in chunks of 32; each thread owns 2 tokens x 4 experts. Router weights
// (E x d fp32, 2.6 MB at E = 128) stay in L2 across token tiles.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int RT = 32;   // tokens per block
constexpr int RE = 64;   // experts per block
constexpr int RK = 32;   // reduction chunk
}  // namespace

__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            int64_t T, int64_t d, int64_t E,
                                                            float* __restrict__ logits) {
    __shared__ float xs[RT][RK + 1];
    __shared__ float ws[RE][RK + 1];
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT;
    const int64_t e0 = static_cast<int64_t>(blockIdx.y) * RE;
    const int tl = tid >> 4;  // tokens 2*tl, 2*tl+1
    const int el = tid & 15;  // experts el + 16*j
    float acc[2][4] = {};

    for (int64_t k0 = 0; k0 < d; k0 += RK) {
        {   // x chunk: 32 x 32 bf16, 4 per thread
            const int r = tid >> 3, c = (tid & 7) * 4;
            const int64_t t = t0 + r;
            uint2 v = make_uint2(0u, 0u);
            if (t < T) v = *reinterpret_cast<const uint2*>(x + t * d + k0 + c);
            xs[r][c + 0] = __uint_as_float(v.x << 16);
            xs[r][c + 1] = __uint_as_float(v.x & 0xFFFF0000u);
            xs[r][c + 2] = __uint_as_float(v.y << 16);
            xs[r][c + 3] = __uint_as_float(v.y & 0xFFFF0000u);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {  // router chunk: 64 x 32 fp32, 8 per thread
            const int idx = tid + 256 * i;
            const int r = idx >> 3, c = (idx & 7) * 4;
            const int64_t e = e0 + r;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < E) v = *reinterpret_cast<const float4*>(wr + e * d + k0 + c);
            ws[r][c + 0] = v.x;
            ws[r][c + 1] = v.y;
            ws[r][c + 2] = v.z;
            ws[r][c + 3] = v.w;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < RK; ++kk) {
            const float xa = xs[2 * tl][kk], xb = xs[2 * tl + 1][kk];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float w = ws[el + 16 * j][kk];
                acc[0][j] = fmaf(xa, w, acc[0][j]);
                acc[1][j] = fmaf(xb, w, acc[1][j]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t t = t0 + 2 * tl + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t e = e0 + el + 16 * j;
            if (e < E) logits[t * E + e] = acc[i][j] + (bias ? bias[e] : 0.0f);
        }
    }
}

// One wave per token: k rounds of a wave-wide arg-max over (logit, -id).
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t T,
                                                   int64_t E, int top_k, int32_t* __restrict__ ids,
                                                   float* __restrict__ gates,
                                                   int32_t* __restrict__ ids_copy,
                                                   float* __restrict__ gates_copy) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
    if (t >= T) return;
    constexpr int PER = kMaxExperts / 64;
    float v[PER];
    bool taken[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int64_t e = lane + 64 * i;
        v[i] = e < E ? logits[t * E + e] : 0.0f;
        taken[i] = e >= E;
    }
    for (int j = 0; j < top_k; ++j) {
        float best = 0.0f;
        int bid = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + 64 * i;
            if (!taken[i] && (bid == 0x7FFFFFFF || v[i] > best)) {
                best = v[i];
                bid = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ob = __shfl_xor(best, off, 64);
            const int oid = __shfl_xor(bid, off, 64);
            const bool better = oid != 0x7FFFFFFF &&
                                (bid == 0x7FFFFFFF || ob > best || (ob == best && oid < bid));
            if (better) {
                best = ob;
                bid = oid;
            }
        }
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (lane + 64 * i == bid) taken[i] = true;
        if (lane == 0) {
            const float g = 1.0f / (1.0f + expf(-best));
            ids[t * top_k + j] = bid;
            gates[t * top_k + j] = g;
            if (ids_copy) ids_copy[t * top_k + j] = bid;
            if (gates_copy) gates_copy[t * top_k + j] = g;
        }
    }
}

hipError_t launch_router_logits(const uint16_t* x, const float* wr, const float* b, int64_t T,
                                int64_t d, int64_t E, float* logits, hipStream_t stream) {
    dim3 grid(static_cast<unsigned>((T + RT - 1) / RT), static_cast<unsigned>((E + RE - 1) / RE));
    hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, stream, x, wr, b, T, d, E, logits);
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t T, int64_t E, int top_k, int32_t* ids,
                       float* gates, int32_t* ids_copy, float* gates_copy, hipStream_t stream) {
    const unsigned blocks = static_cast<unsigned>((T + 3) / 4);  // 4 waves (tokens) per block
    hipLaunchKernelGGL(topk_kernel, dim3(blocks), dim3(256), 0, stream, logits, T, E, top_k, ids,
                       gates, ids_copy, gates_copy);
    return hipGetLastError();
}

}  // namespace moe
