// Measured HBM ceilings (measurement support, not part of the computation):
// a streaming read of a buffer and a streaming copy, in the access pattern of
// the library's bandwidth-bound kernels (16-byte loads by consecutive lanes,
// several loads in flight per lane). A GEMV streams its packed weights as a
// read-only stream; the scan reads two tensors and writes one. What these
// kernels move per second is the roof the bandwidth-bound kernels are read
// against next to the published 8 TB/s.
#include "device_common.hpp"
#include "launch.hpp"

namespace mmf {

constexpr int kCeilThreads = 256;
constexpr int kCeilUnroll = 4;  // 16-byte loads in flight per lane

// Every lane XORs the words it reads; one word per workgroup goes to sink so
// that the loads cannot be dropped.
// Plain (cached) loads, as the GEMV reads its weights.
__global__ __launch_bounds__(kCeilThreads) void stream_read_kernel(const i32x4 *__restrict__ src, int64_t n16,
                                                                  uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kCeilThreads;
    int64_t i = (int64_t)blockIdx.x * kCeilThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kCeilUnroll - 1) * stride < n16; i += kCeilUnroll * stride) {
        i32x4 v[kCeilUnroll];
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) acc ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    }
    for (; i < n16; i += stride) {
        const i32x4 v = src[i];
        acc ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
    }
    __shared__ uint32_t red[kCeilThreads / kWave];
    acc = (uint32_t)wave_sum_int((int)acc);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kCeilThreads / kWave; ++w) t ^= red[w];
        sink[blockIdx.x] = t;
    }
}

// Streaming (non-temporal) loads and stores, as the scan moves tensors larger than the caches.
__global__ __launch_bounds__(kCeilThreads) void stream_copy_kernel(const i32x4 *__restrict__ src,
                                                                  i32x4 *__restrict__ dst, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * kCeilThreads;
    int64_t i = (int64_t)blockIdx.x * kCeilThreads + threadIdx.x;
    for (; i + (kCeilUnroll - 1) * stride < n16; i += kCeilUnroll * stride) {
        i32x4 v[kCeilUnroll];
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

int ceiling_blocks() { return 256 * 8; }  // 8 workgroups of 256 threads per CU

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t st) {
    launch_k(stream_read_kernel, ceiling_blocks(), kCeilThreads, 0, st, static_cast<const i32x4 *>(src), bytes / 16,
             sink);
    return hipGetLastError();
}

hipError_t launch_stream_copy(const void *src, void *dst, int64_t bytes, hipStream_t st) {
    launch_k(stream_copy_kernel, ceiling_blocks(), kCeilThreads, 0, st, static_cast<const i32x4 *>(src),
             static_cast<i32x4 *>(dst), bytes / 16);
    return hipGetLastError();
}

}  // namespace mmf
