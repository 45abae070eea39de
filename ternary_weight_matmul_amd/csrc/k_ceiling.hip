// Measured HBM ceilings (measurement support, not part of the computation):
// streaming kernels in the access patterns of the library's bandwidth-bound
// kernels -- 16-byte loads by consecutive lanes, eight in flight per lane,
// 8192 workgroups of 256 threads (the fastest of a sweep over 1024-8192
// workgroups, 4-16 loads per lane and temporal / non-temporal accesses on
// MI355X). A GEMV streams its packed weights as a read-only stream; the scan
// reads two tensors and writes one. What these kernels move per second is the
// roof the bandwidth-bound kernels are read against next to the published
// 8 TB/s.
#include "device_common.hpp"
#include "launch.hpp"

namespace mmf {

constexpr int kCeilThreads = 256;
constexpr int kCeilUnroll = 8;  // 16-byte loads in flight per lane

__device__ __forceinline__ i32x4 ld_nt(const i32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(i32x4 v, i32x4 *p) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ int fold(i32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// Every lane XORs the words it reads; the workgroup's XOR of them goes to
// sink (one word per workgroup), so the loads cannot be dropped.
__global__ __launch_bounds__(kCeilThreads) void stream_read_kernel(const i32x4 *__restrict__ src, int64_t n16,
                                                                  uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kCeilThreads;
    int64_t i = (int64_t)blockIdx.x * kCeilThreads + threadIdx.x;
    int acc = 0;
    for (; i + (kCeilUnroll - 1) * stride < n16; i += kCeilUnroll * stride) {
        i32x4 v[kCeilUnroll];
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) v[u] = ld_nt(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) acc ^= fold(v[u]);
    }
    for (; i < n16; i += stride) acc ^= fold(src[i]);
    __shared__ int red[kCeilThreads / kWave];
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int w = 0; w < kCeilThreads / kWave; ++w) t ^= red[w];
        sink[blockIdx.x] = (uint32_t)t;
    }
}

// dst = src (a read and a write stream), or dst = src ^ src2 (two read streams and one write
// stream, the scan's pattern), non-temporal throughout.
template <bool TWO>
__global__ __launch_bounds__(kCeilThreads) void stream_copy_kernel(const i32x4 *__restrict__ src,
                                                                  const i32x4 *__restrict__ src2,
                                                                  i32x4 *__restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kCeilThreads;
    int64_t i = (int64_t)blockIdx.x * kCeilThreads + threadIdx.x;
    for (; i + (kCeilUnroll - 1) * stride < n16; i += kCeilUnroll * stride) {
        i32x4 v[kCeilUnroll];
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) v[u] = ld_nt(src + i + u * stride);
        if constexpr (TWO) {
#pragma unroll
            for (int u = 0; u < kCeilUnroll; ++u) v[u] ^= ld_nt(src2 + i + u * stride);
        }
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) st_nt(v[u], dst + i + u * stride);
    }
    for (; i < n16; i += stride) dst[i] = TWO ? src[i] ^ src2[i] : src[i];
}

int ceiling_blocks() { return 8192; }

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t st) {
    launch_k(stream_read_kernel, ceiling_blocks(), kCeilThreads, 0, st, static_cast<const i32x4 *>(src), bytes / 16,
             sink);
    return hipGetLastError();
}

hipError_t launch_stream_copy(const void *src, const void *src2, void *dst, int64_t bytes, hipStream_t st) {
    const i32x4 *a = static_cast<const i32x4 *>(src), *b = static_cast<const i32x4 *>(src2);
    i32x4 *d = static_cast<i32x4 *>(dst);
    if (src2) launch_k(stream_copy_kernel<true>, ceiling_blocks(), kCeilThreads, 0, st, a, b, d, bytes / 16);
    else launch_k(stream_copy_kernel<false>, ceiling_blocks(), kCeilThreads, 0, st, a, b, d, bytes / 16);
    return hipGetLastError();
}

}  // namespace mmf
