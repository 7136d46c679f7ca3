// router.hip -- K2: router logits, top-k selection and sigmoid gates (gfx950).
//
// The router of the discosf.com page "1 卡跑通 Llama 4", section "混合专家路由":
// every token scores every expert, and the top-k experts are chosen
// (torch.topk there). The score is a sigmoid gate of the logit; selection is
// on the logits (same order as the sigmoid), ties go to the lower expert id.
//
// Logits stay fp32: the choice of experts must not move with a cheaper
// precision. Small batches (decode) run this small GEMM on the vector ALUs
// (the bf16 x widens exactly, fp32 FMA accumulation). Prefill batches run it
// on bf16 MFMA without losing precision: each fp32 router weight is split
// exactly into three bf16 parts (hi + mid + lo, every part the rounding of
// what the previous parts leave), so each product x * part is exact and the
// matrix cores sum x * w in fp32 (router_gemm_kernel).
//
// router_partials_kernel<TT, EE, MT, ME>: a 256-thread block computes a
// TT-token x EE-expert tile over one slice of the reduction dimension; each
// thread owns MT tokens x ME experts (experts strided so LDS reads are
// conflict-free). Slices (split-K) give small batches enough blocks; partial
// sums go to partials[s][t][e] and are added in slice order by the consumer,
// so the result does not depend on scheduling.
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

// RK: reduction chunk staged in LDS. The decode tile (16 x 16) stages its
// whole 128-column slice at once, so its loads take one memory round trip.
template <int TT, int EE, int MT, int ME, int RK = 32>
__global__ __launch_bounds__(256) void router_partials_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ wr,
                                                              int64_t T, int64_t d, int64_t E,
                                                              int64_t slice,
                                                              float* __restrict__ partials,
                                                              uint16_t* __restrict__ x_perm) {
    static_assert((TT / MT) * (EE / ME) == 256, "one output micro-tile per thread");
    __shared__ float xs[TT][RK + 1];
    __shared__ float ws[EE][RK + 1];
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TT;
    const int64_t e0 = static_cast<int64_t>(blockIdx.y) * EE;
    const int64_t kb = static_cast<int64_t>(blockIdx.z) * slice;
    constexpr int EW = EE / ME;  // threads along experts
    const int tt = tid / EW;     // tokens tt*MT + i
    const int ee = tid % EW;     // experts ee + EW*j
    float acc[MT][ME] = {};

    // every load of a chunk is issued before its LDS stores
    constexpr int XN = TT * (RK / 4), WN = EE * (RK / 4);
    constexpr int XI = (XN + 255) / 256, WI = (WN + 255) / 256;
    for (int64_t k0 = kb; k0 < kb + slice; k0 += RK) {
        uint2 xv[XI];
        float4 wv[WI];
#pragma unroll
        for (int i = 0; i < XI; ++i) {  // x: TT x RK bf16
            const int idx = tid + 256 * i;
            const int r = idx / (RK / 4), c = (idx % (RK / 4)) * 4;
            const int64_t t = t0 + r;
            xv[i] = (idx < XN && t < T) ? *reinterpret_cast<const uint2*>(x + t * d + k0 + c)
                                        : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < WI; ++i) {  // router: EE x RK fp32
            const int idx = tid + 256 * i;
            const int r = idx / (RK / 4), c = (idx % (RK / 4)) * 4;
            const int64_t e = e0 + r;
            wv[i] = (idx < WN && e < E) ? *reinterpret_cast<const float4*>(wr + e * d + k0 + c)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int idx = tid + 256 * i;
            if (idx >= XN) continue;
            const int r = idx / (RK / 4), c = (idx % (RK / 4)) * 4;
            xs[r][c + 0] = __uint_as_float(xv[i].x << 16);
            xs[r][c + 1] = __uint_as_float(xv[i].x & 0xFFFF0000u);
            xs[r][c + 2] = __uint_as_float(xv[i].y << 16);
            xs[r][c + 3] = __uint_as_float(xv[i].y & 0xFFFF0000u);
        }
#pragma unroll
        for (int i = 0; i < WI; ++i) {
            const int idx = tid + 256 * i;
            if (idx >= WN) continue;
            const int r = idx / (RK / 4), c = (idx % (RK / 4)) * 4;
            ws[r][c + 0] = wv[i].x;
            ws[r][c + 1] = wv[i].y;
            ws[r][c + 2] = wv[i].z;
            ws[r][c + 3] = wv[i].w;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < RK; ++kk) {
            float xk[MT], wk[ME];
#pragma unroll
            for (int i = 0; i < MT; ++i) xk[i] = xs[tt * MT + i][kk];
#pragma unroll
            for (int j = 0; j < ME; ++j) wk[j] = ws[ee + EW * j][kk];
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < ME; ++j) acc[i][j] = fmaf(xk[i], wk[j], acc[i][j]);
        }
        __syncthreads();
    }
    // x with 8-element blocks stored in the order 0,4,1,5,2,6,3,7: the A operand
    // layout of the decode path's int4 nibble-pair dequantization (after the
    // products, so that its loads find this slice of x in the cache)
    if (x_perm && blockIdx.y == 0) {
        for (int64_t idx = tid; idx < static_cast<int64_t>(TT) * (slice / 8); idx += 256) {
            const int64_t t = t0 + idx / (slice / 8);
            if (t >= T) break;
            const int64_t col = kb + (idx % (slice / 8)) * 8;
            const uint4 v = *reinterpret_cast<const uint4*>(x + t * d + col);
            uint4 r;
            r.x = (v.x & 0xFFFFu) | (v.z << 16);
            r.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
            r.z = (v.y & 0xFFFFu) | (v.w << 16);
            r.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
            *reinterpret_cast<uint4*>(x_perm + t * d + col) = r;
        }
    }

    float* out = partials + static_cast<int64_t>(blockIdx.z) * T * E;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t t = t0 + tt * MT + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < ME; ++j) {
            const int64_t e = e0 + ee + EW * j;
            if (e < E) out[t * E + e] = acc[i][j];
        }
    }
}

RouterPlan router_plan(int64_t T, int64_t d, int64_t E) {
    RouterPlan p{};
    if (T >= kRouterMfmaTokens) {
        // bf16 MFMA on the exactly split weights: blocks of 128 tokens x up to
        // 128 experts (ee), slices of the reduction (multiples of 32 wide)
        // until there are about 512 blocks
        p.kind = 4;
        p.tt = 128;
        p.ee = E <= 16 ? 16 : E <= 32 ? 32 : E <= 64 ? 64 : 128;
        const int64_t blocks = ((T + 127) / 128) * ((E + p.ee - 1) / p.ee);
        const int64_t want = (512 + blocks - 1) / blocks;
        int64_t s = 1;
        for (int64_t c = 1; c <= d / 32 && c <= kMaxRouterSlices; ++c)
            if ((d / 32) % c == 0 && c <= want) s = c;
        p.slices = static_cast<int>(s);
        return p;
    }
    if (T <= 16 && E <= 16) {
        p.kind = 0;
        p.tt = 16;
        p.ee = 16;
    } else if (E <= 16) {
        p.kind = 1;
        p.tt = 128;
        p.ee = 16;
    } else if (E <= 32) {
        p.kind = 2;
        p.tt = 64;
        p.ee = 32;
    } else {
        p.kind = 3;
        p.tt = 32;
        p.ee = 64;
    }
    const int64_t tiles = ((T + p.tt - 1) / p.tt) * ((E + p.ee - 1) / p.ee);
    // enough blocks to cover the chip; slices are whole multiples of 128 wide
    const int64_t want = (512 + tiles - 1) / tiles;
    int64_t s = 1;
    for (int64_t c = 1; c <= d / 128; ++c)
        if ((d / 128) % c == 0 && c <= want) s = c;
    p.slices = static_cast<int>(s);
    return p;
}

// Prefill batches: router logits on the bf16 matrix cores without losing
// the fp32 weights. Each fp32 weight w is split exactly into three bf16
// parts, hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid) (each
// difference is exact in fp32, and what is left after mid fits 8 bits), so
// hi + mid + lo == w, every product x * part is exact and the matrix cores
// sum x * w in fp32.
//
// router_gemm_kernel<EC>: a block is 4 waves over 128 tokens (32 per wave:
// two 16-row v_mfma_f32_16x16x32_bf16 tiles) and EC experts (blockIdx.y: a
// chunk of EC, EC in 16..128) for one slice of the reduction (blockIdx.z).
// Per 32-wide step the block reads its EC x 32 fp32 weights once (8 threads
// per expert row, one float4 each), splits them in registers and stores the
// three parts in LDS in B-fragment order (part p, expert tile j: lane
// (n, q) at (q * 16 + n) * 16 bytes); the waves then read them against their
// own tokens' A fragments, which come straight from x. The next step's loads
// are requested before this step's products. Blocks of expert chunk 0 also
// write x_perm for their tokens and columns. Partial sums go to
// out[slice][t][e] and are added in slice order by the top-k kernel.
namespace {
constexpr int kRouterStepBytes = 1024;  // one 16-expert x 32-column bf16 fragment tile
}

template <int EC>
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr, int64_t T,
                                                          int64_t d, int64_t E, int64_t slice,
                                                          float* __restrict__ out,
                                                          uint16_t* __restrict__ x_perm) {
    constexpr int NJ = EC / 16;                    // expert tiles
    constexpr int PART = NJ * kRouterStepBytes;    // one bf16 part of the step
    constexpr int WI = (EC * 8 + 255) / 256;       // float4 weight loads per thread
    __shared__ __attribute__((aligned(16))) uint8_t bs[3 * PART];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, kq = lane >> 4;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 128 + 32 * w;
    const int64_t e0 = static_cast<int64_t>(blockIdx.y) * EC;
    const int64_t kb = static_cast<int64_t>(blockIdx.z) * slice;
    const int steps = static_cast<int>(slice / 32);

    // A: rows t0 + 16 i + l16 (past T: the last row, not stored), columns 8 kq ..
    const uint16_t* xr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int64_t t = t0 + 16 * i + l16;
        t = t < T ? t : T - 1;
        xr[i] = x + t * d + kb + kq * 8;
    }
    // B: thread -> expert row er[u] = tid / 8 + 32 u of the chunk, columns 4 (tid % 8) ..
    const float* wrow[WI];
    int boff[WI];
    bool bval[WI];
#pragma unroll
    for (int u = 0; u < WI; ++u) {
        const int r = tid / 8 + 32 * u;
        const int c = (tid & 7) * 4;
        bval[u] = r < EC && e0 + r < E;
        wrow[u] = wr + (bval[u] ? (e0 + r) * d : 0) + kb + c;
        boff[u] = (r / 16) * kRouterStepBytes + ((c / 8) * 16 + (r % 16)) * 16 + (c % 8) * 2;
    }

    f32x4 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 ra[2];
    float4 rw[WI];
    auto load = [&](int s) __attribute__((always_inline)) {
        const int64_t k = static_cast<int64_t>(s) * 32;
#pragma unroll
        for (int i = 0; i < 2; ++i) ra[i] = *reinterpret_cast<const uint4*>(xr[i] + k);
#pragma unroll
        for (int u = 0; u < WI; ++u)
            rw[u] = bval[u] ? *reinterpret_cast<const float4*>(wrow[u] + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    };
    load(0);
    for (int s = 0; s < steps; ++s) {
        // split this step's weights into the three parts, in fragment order
#pragma unroll
        for (int u = 0; u < WI; ++u) {
            if (tid / 8 + 32 * u >= EC) continue;
            const float v[4] = {rw[u].x, rw[u].y, rw[u].z, rw[u].w};
            uint16_t hi[4], mid[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hi[e] = f32_to_bf16(v[e]);
                const float r1 = v[e] - bf16_to_f32(hi[e]);
                mid[e] = f32_to_bf16(r1);
                lo[e] = f32_to_bf16(r1 - bf16_to_f32(mid[e]));
            }
            *reinterpret_cast<uint2*>(bs + boff[u]) =
                make_uint2(hi[0] | (static_cast<uint32_t>(hi[1]) << 16), hi[2] | (static_cast<uint32_t>(hi[3]) << 16));
            *reinterpret_cast<uint2*>(bs + PART + boff[u]) =
                make_uint2(mid[0] | (static_cast<uint32_t>(mid[1]) << 16), mid[2] | (static_cast<uint32_t>(mid[3]) << 16));
            *reinterpret_cast<uint2*>(bs + 2 * PART + boff[u]) =
                make_uint2(lo[0] | (static_cast<uint32_t>(lo[1]) << 16), lo[2] | (static_cast<uint32_t>(lo[3]) << 16));
        }
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, ra[0]);
        const bf16x8 a1 = __builtin_bit_cast(bf16x8, ra[1]);
        if (x_perm && blockIdx.y == 0) {
            // this lane's 8 columns of both rows, 8-element blocks in the order 0,4,1,5,2,6,3,7
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int64_t t = t0 + 16 * i + l16;
                if (t >= T) continue;
                const uint4 v = ra[i];
                uint4 r;
                r.x = (v.x & 0xFFFFu) | (v.z << 16);
                r.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
                r.z = (v.y & 0xFFFFu) | (v.w << 16);
                r.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
                *reinterpret_cast<uint4*>(x_perm + t * d + kb + static_cast<int64_t>(s) * 32 + kq * 8) = r;
            }
        }
        __syncthreads();
        if (s + 1 < steps) load(s + 1);  // the next step's loads fly under the products
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(
                    bs + p * PART + j * kRouterStepBytes + (kq * 16 + l16) * 16);
                acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc[0][j], 0, 0, 0);
                acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc[1][j], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    float* o = out + static_cast<int64_t>(blockIdx.z) * T * E;
    // D[token][expert]: token row 4 kq + r of a 16 x 16 tile, expert column l16
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = t0 + 16 * i + 4 * kq + r;
                const int64_t e = e0 + 16 * j + l16;
                if (t < T && e < E) o[t * E + e] = acc[i][j][r];
            }
}

hipError_t launch_router_partials(const uint16_t* x, const float* wr, int64_t T, int64_t d,
                                  int64_t E, const RouterPlan& p, float* partials,
                                  uint16_t* x_perm, hipStream_t stream) {
    if (p.kind == 4) {
        const int64_t slice = d / p.slices;
        const int ec = p.ee;
        dim3 grid(static_cast<unsigned>((T + 127) / 128), static_cast<unsigned>((E + ec - 1) / ec),
                  static_cast<unsigned>(p.slices));
        switch (ec) {
            case 16:
                MOE_LAUNCH((router_gemm_kernel<16>), grid, dim3(256), 0, stream, x, wr, T, d, E, slice,
                           partials, x_perm);
                break;
            case 32:
                MOE_LAUNCH((router_gemm_kernel<32>), grid, dim3(256), 0, stream, x, wr, T, d, E, slice,
                           partials, x_perm);
                break;
            case 64:
                MOE_LAUNCH((router_gemm_kernel<64>), grid, dim3(256), 0, stream, x, wr, T, d, E, slice,
                           partials, x_perm);
                break;
            default:
                MOE_LAUNCH((router_gemm_kernel<128>), grid, dim3(256), 0, stream, x, wr, T, d, E, slice,
                           partials, x_perm);
                break;
        }
        return hipGetLastError();
    }
    dim3 grid(static_cast<unsigned>((T + p.tt - 1) / p.tt), static_cast<unsigned>((E + p.ee - 1) / p.ee),
              static_cast<unsigned>(p.slices));
    const int64_t slice = d / p.slices;
    switch (p.kind) {
        case 0:
            if (slice % 128 == 0)
                MOE_LAUNCH((router_partials_kernel<16, 16, 1, 1, 128>), grid, dim3(256), 0, stream, x,
                           wr, T, d, E, slice, partials, x_perm);
            else
                MOE_LAUNCH((router_partials_kernel<16, 16, 1, 1>), grid, dim3(256), 0, stream, x,
                           wr, T, d, E, slice, partials, x_perm);
            break;
        case 1:
            MOE_LAUNCH((router_partials_kernel<128, 16, 8, 1>), grid, dim3(256), 0, stream, x,
                               wr, T, d, E, slice, partials, x_perm);
            break;
        case 2:
            MOE_LAUNCH((router_partials_kernel<64, 32, 4, 2>), grid, dim3(256), 0, stream, x,
                               wr, T, d, E, slice, partials, x_perm);
            break;
        default:
            MOE_LAUNCH((router_partials_kernel<32, 64, 2, 4>), grid, dim3(256), 0, stream, x,
                               wr, T, d, E, slice, partials, x_perm);
            break;
    }
    return hipGetLastError();
}

// sum_{s < slices} p[s * stride] in slice order, slices <= M: all M loads are
// issued before the first add (rows past `slices` re-read the last one), so
// the sum costs one memory latency instead of one per few slices
template <int M>
__device__ __forceinline__ float sum_slices_m(const float* p, int slices, int64_t stride) {
    float v[M];
#pragma unroll
    for (int j = 0; j < M; ++j) v[j] = p[static_cast<int64_t>(j < slices ? j : slices - 1) * stride];
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < M; ++j) s = j < slices ? s + v[j] : s;
    return s;
}

// any number of slices, in rounds of 16 (still in slice order)
__device__ __forceinline__ float sum_slices(const float* p, int slices, int64_t stride) {
    if (slices <= 1) return p[0];
    if (slices <= 4) return sum_slices_m<4>(p, slices, stride);
    float s = 0.0f;
    for (int k = 0; k < slices; k += 16)
        s += sum_slices_m<16>(p + static_cast<int64_t>(k) * stride, slices - k < 16 ? slices - k : 16,
                              stride);
    return s;
}

// One wave per token: sums the slices' partial logits (slice order) plus the
// bias, then k rounds of a wave-wide arg-max over (logit, lower id first).
__device__ __forceinline__ void topk_wave(const float* v_in, int64_t E, int top_k, int lane,
                                          int32_t* ids_out, float* gates_out,
                                          int32_t* ids_copy, float* gates_copy) {
    constexpr int PER = kMaxExperts / 64;
    float v[PER];
    bool taken[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int64_t e = lane + 64 * i;
        v[i] = e < E ? v_in[e] : 0.0f;
        taken[i] = e >= E;
    }
    for (int j = 0; j < top_k; ++j) {
        float best = 0.0f;
        int bid = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (!taken[i] && (bid == 0x7FFFFFFF || v[i] > best)) {
                best = v[i];
                bid = lane + 64 * i;
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
            ids_out[j] = bid;
            gates_out[j] = g;
            if (ids_copy) ids_copy[j] = bid;
            if (gates_copy) gates_copy[j] = g;
        }
    }
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ partials, int slices,
                                                   const float* __restrict__ bias, int64_t T,
                                                   int64_t E, int top_k, float* __restrict__ logits,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ gates,
                                                   int32_t* __restrict__ ids_copy,
                                                   float* __restrict__ gates_copy) {
    __shared__ float row[4][kMaxExperts];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (t >= T) return;  // wave-uniform; no block-wide barrier below
    for (int64_t e = lane; e < E; e += 64) {
        float s = sum_slices(partials + t * E + e, slices, T * E);
        if (bias) s += bias[e];
        row[w][e] = s;
        logits[t * E + e] = s;
    }
    __builtin_amdgcn_wave_barrier();
    topk_wave(row[w], E, top_k, lane, ids + t * top_k, gates + t * top_k,
              ids_copy ? ids_copy + t * top_k : nullptr, gates_copy ? gates_copy + t * top_k : nullptr);
}

hipError_t launch_topk(const float* partials, int slices, const float* bias, int64_t T, int64_t E,
                       int top_k, float* logits, int32_t* ids, float* gates, int32_t* ids_copy,
                       float* gates_copy, hipStream_t stream) {
    const unsigned blocks = static_cast<unsigned>((T + 3) / 4);  // 4 waves (tokens) per block
    MOE_LAUNCH(topk_kernel, dim3(blocks), dim3(256), 0, stream, partials, slices, bias, T, E,
                       top_k, logits, ids, gates, ids_copy, gates_copy);
    return hipGetLastError();
}

// ------------------------------------------------------------------------
// Small-batch routing in one block: logits (slice sums + bias), top-k and
// gates, then the dispatch (counts, offsets, stable perm / inv) and the work
// lists of the projections, the same lists build_work_lists makes, with every
// thread (a pair or an expert per thread). Used when T * E <= kSmallRouteLogits
// and T * top_k <= 1024.
__global__ __launch_bounds__(1024) void route_small_kernel(
    const float* __restrict__ partials, int slices, const float* __restrict__ bias, int64_t T,
    int E, int top_k, int tile_rows, int small_rows, float* __restrict__ logits,
    int32_t* __restrict__ ids,
    float* __restrict__ gates, int32_t* __restrict__ ids_copy, float* __restrict__ gates_copy,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ tile_base,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int4* __restrict__ chunks,
    int32_t* __restrict__ nchunks) {
    __shared__ float lg[kSmallRouteLogits];
    __shared__ int sids[1024];
    __shared__ float sg[1024];
    __shared__ int off[kMaxExperts];
    __shared__ float part[4][1024];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t TE = T * E;
    const int P = static_cast<int>(T) * top_k;
    if (TE <= 1024) {
        // four threads per logit, each a quarter of the slices (in order), then
        // the quarters in order: one round of loads in flight instead of several
        const int q = tid >> 8;
        const int qs = (slices + 3) / 4;
        const int s0 = q * qs, s1 = (s0 + qs < slices) ? s0 + qs : slices;
        for (int64_t i = tid & 255; i < TE; i += 256)
            part[q][i] = s1 > s0 ? sum_slices(partials + s0 * TE + i, s1 - s0, TE) : 0.0f;
        __syncthreads();
        for (int64_t i = tid; i < TE; i += 1024) {
            float s = ((part[0][i] + part[1][i]) + part[2][i]) + part[3][i];
            if (bias) s += bias[i % E];
            lg[i] = s;
            logits[i] = s;
        }
    } else {
        for (int64_t i = tid; i < TE; i += 1024) {
            float s = sum_slices(partials + i, slices, TE);
            if (bias) s += bias[i % E];
            lg[i] = s;
            logits[i] = s;
        }
    }
    __syncthreads();
    for (int64_t t = w; t < T; t += 16)
        topk_wave(lg + t * E, E, top_k, lane, sids + t * top_k, sg + t * top_k,
                  ids_copy ? ids_copy + t * top_k : nullptr,
                  gates_copy ? gates_copy + t * top_k : nullptr);
    __syncthreads();
    for (int p = tid; p < P; p += 1024) {
        ids[p] = sids[p];
        gates[p] = sg[p];
    }

    // Dispatch with every thread, pair p = tid (P <= 1024). Inside a wave, one
    // ballot per distinct expert gives each pair its rank among the wave's
    // pairs of that expert, and the wave's count of it; the counts taken over
    // the waves in order make the slots stable (pairs ascending per expert).
    int* wcnt = reinterpret_cast<int*>(&part[0][0]);  // [16 waves][kMaxExperts]; part is dead
    for (int i = tid; i < 16 * kMaxExperts; i += 1024) wcnt[i] = 0;
    __syncthreads();
    const bool has = tid < P;
    const int my_e = has ? sids[tid] : -1;
    int rank = 0;
    for (uint64_t todo = __ballot(has); todo;) {
        const int leader = __ffsll(static_cast<unsigned long long>(todo)) - 1;
        const int e0 = __shfl(my_e, leader, 64);
        const uint64_t m = __ballot(my_e == e0);
        if (my_e == e0) rank = __popcll(m & ((1ull << lane) - 1));
        if (lane == leader) wcnt[w * kMaxExperts + e0] = __popcll(m);
        todo &= ~m;
    }
    __syncthreads();

    // Per expert (thread e < E <= 256, waves 0-3): its count, the waves' counts
    // made exclusive prefixes, and the work lists' sizes by the rule of
    // build_work_lists: streaming chunks of kDecodeRows pairs for chunked
    // experts (all of them when small_rows < 0, else those with 1..small_rows
    // pairs), GEMM tiles of tile_rows for the others (all when small_rows < 0).
    int c = 0, nch = 0, ntl = 0;
    if (tid < E) {
        for (int v = 0; v < (P + 63) / 64; ++v) {
            const int n = wcnt[v * kMaxExperts + tid];
            wcnt[v * kMaxExperts + tid] = c;
            c += n;
        }
        const bool chunked = small_rows < 0 || (c > 0 && c <= small_rows);
        nch = chunked ? (c + kDecodeRows - 1) / kDecodeRows : 0;
        ntl = (small_rows < 0 || !chunked) ? (c + tile_rows - 1) / tile_rows : 0;
    }
    // inclusive scans of (c, nch, ntl) over threads 0..255: in each wave by
    // shuffles, then the wave totals
    __shared__ int wtot[3][4];
    int ic = c, ich = nch, itl = ntl;
    if (w < 4) {
        for (int o = 1; o < 64; o <<= 1) {
            const int a = __shfl_up(ic, o, 64), b = __shfl_up(ich, o, 64), t = __shfl_up(itl, o, 64);
            if (lane >= o) {
                ic += a;
                ich += b;
                itl += t;
            }
        }
        if (lane == 63) {
            wtot[0][w] = ic;
            wtot[1][w] = ich;
            wtot[2][w] = itl;
        }
    }
    // the shared expert's chunks (every token) lead the chunk list when small_rows < 0
    const int lead = small_rows < 0 ? static_cast<int>((T + kDecodeRows - 1) / kDecodeRows) : 0;
    for (int i = tid; i < lead; i += 1024) {
        const int r = i * kDecodeRows;
        chunks[i] = make_int4(E, P + r, T - r < kDecodeRows ? static_cast<int>(T - r) : kDecodeRows, 0);
    }
    __syncthreads();
    if (tid < E) {
        for (int v = 0; v < w; ++v) {
            ic += wtot[0][v];
            ich += wtot[1][v];
            itl += wtot[2][v];
        }
        const int oc = ic - c, och = lead + ich - nch, otl = itl - ntl;
        off[tid] = oc;
        counts[tid] = c;
        offsets[tid] = oc;
        tile_base[tid] = otl;
        for (int i = 0; i < nch; ++i) {
            const int r = i * kDecodeRows;
            chunks[och + i] = make_int4(tid, oc + r, c - r < kDecodeRows ? c - r : kDecodeRows, 0);
        }
        if (tid == E - 1) {
            offsets[E] = ic;
            tile_base[E] = itl;
            tile_base[E + 1] = itl + static_cast<int>((T + tile_rows - 1) / tile_rows);
            *nchunks = lead + ich;
        }
    }
    __syncthreads();
    if (has) {
        const int slot = off[my_e] + wcnt[w * kMaxExperts + my_e] + rank;
        perm[slot] = tid;
        inv[tid] = slot;
    }
}

hipError_t launch_route_small(const float* partials, int slices, const float* bias, int64_t T,
                              int64_t E, int top_k, int tile_rows, int small_rows, float* logits,
                              int32_t* ids, float* gates, int32_t* ids_copy, float* gates_copy,
                              int32_t* counts, int32_t* offsets, int32_t* tile_base, int32_t* perm,
                              int32_t* inv, int4* chunks, int32_t* nchunks, hipStream_t stream) {
    MOE_LAUNCH(route_small_kernel, dim3(1), dim3(1024), 0, stream, partials, slices, bias, T,
                       static_cast<int>(E), top_k, tile_rows, small_rows, logits, ids, gates, ids_copy,
                       gates_copy, counts, offsets, tile_base, perm, inv, chunks, nchunks);
    return hipGetLastError();
}

}  // namespace moe
