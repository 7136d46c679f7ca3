// stream.hip -- measurement kernels (not part of the layer): the HBM rates that
// plain streaming reaches on the device, the practical ceiling beside the
// nominal peak for the streaming decode kernels.
//
//  * read: every 16-byte word of a buffer once, with the same non-temporal
//    loads as the streaming decode kernels, folded into one XOR per block (so
//    the loads cannot be dropped) and written to sink[block];
//  * copy: a plain device copy in 16-byte words.
// Grid-stride loops over blocks sized to fill the chip several times.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int NTS = 256;
constexpr int kUnroll = 4;  // independent loads in flight per thread per iteration
}  // namespace

__global__ __launch_bounds__(NTS) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n,
                                                          uint32_t* __restrict__ sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * NTS;
    int64_t i = static_cast<int64_t>(blockIdx.x) * NTS + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    for (int o = 32; o > 0; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o, 64));
    __shared__ uint32_t wsum[NTS / 64];
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = wsum[0] ^ wsum[1] ^ wsum[2] ^ wsum[3];
}

__global__ __launch_bounds__(NTS) void stream_copy_kernel(u32x4* __restrict__ dst,
                                                          const u32x4* __restrict__ src, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * NTS;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * NTS + threadIdx.x; i < n; i += stride)
        dst[i] = __builtin_nontemporal_load(src + i);
}

unsigned stream_blocks(int64_t n16) {
    const int64_t want = (n16 + NTS - 1) / NTS;
    return static_cast<unsigned>(want < kStreamBlocks ? (want > 0 ? want : 1) : kStreamBlocks);
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    const int64_t n = bytes / 16;
    MOE_LAUNCH(stream_read_kernel, dim3(stream_blocks(n)), dim3(NTS), 0, stream,
               static_cast<const u32x4*>(buf), n, sink);
    return hipGetLastError();
}

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
    const int64_t n = bytes / 16;
    MOE_LAUNCH(stream_copy_kernel, dim3(stream_blocks(n)), dim3(NTS), 0, stream,
               static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n);
    return hipGetLastError();
}

}  // namespace moe
