// Measured HBM ceilings (measurement support, not part of the computation):
// streaming kernels in the access patterns of the library's bandwidth-bound
// kernels -- 16-byte loads by consecutive lanes, eight in flight per lane,
// each workgroup streaming its own contiguous range. The shapes are the
// fastest of sweeps on MI355X over 1024-32768 workgroups, 2-16 loads per lane,
// temporal / non-temporal accesses and grid-strided or contiguous ranges: the
// read stream with cached loads and 8192 workgroups, the copy and the
// two-reads-one-write stream with non-temporal loads and stores and 16384. A
// GEMV streams its packed weights as a read-only stream; the scan reads two
// tensors and writes one. What these kernels move per second is the roof the
// bandwidth-bound kernels are read against next to the published 8 TB/s.
#include "device_common.hpp"
#include "launch.hpp"
#include "ceiling.hpp"

namespace mmf {

constexpr int kCeilThreads = 256;
constexpr int kCeilUnroll = 8;  // 16-byte loads in flight per lane and stream

__device__ __forceinline__ int fold(i32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// [begin, end) of workgroup blockIdx.x's contiguous range of n16 16-byte pieces
__device__ __forceinline__ void wg_range(int64_t n16, int64_t &b, int64_t &e) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    b = (int64_t)blockIdx.x * per;
    e = b + per < n16 ? b + per : n16;
}

// Every lane XORs the words it reads; the workgroup's XOR of them goes to
// sink (one word per workgroup), so the loads cannot be dropped.
__global__ __launch_bounds__(kCeilThreads) void stream_read_kernel(const i32x4 *__restrict__ src, int64_t n16,
                                                                  uint32_t *__restrict__ sink) {
    int64_t b, e;
    wg_range(n16, b, e);
    int64_t i = b + threadIdx.x;
    int acc = 0;
    for (; i + (kCeilUnroll - 1) * kCeilThreads < e; i += kCeilUnroll * kCeilThreads) {
        i32x4 v[kCeilUnroll];
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) v[u] = src[i + u * kCeilThreads];
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) acc ^= fold(v[u]);
    }
    for (; i < e; i += kCeilThreads) acc ^= fold(src[i]);
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
    int64_t b, e;
    wg_range(n16, b, e);
    int64_t i = b + threadIdx.x;
    for (; i + (kCeilUnroll - 1) * kCeilThreads < e; i += kCeilUnroll * kCeilThreads) {
        i32x4 v[kCeilUnroll];
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kCeilThreads);
        if constexpr (TWO) {
#pragma unroll
            for (int u = 0; u < kCeilUnroll; ++u) v[u] ^= __builtin_nontemporal_load(src2 + i + u * kCeilThreads);
        }
#pragma unroll
        for (int u = 0; u < kCeilUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * kCeilThreads);
    }
    for (; i < e; i += kCeilThreads) dst[i] = TWO ? src[i] ^ src2[i] : src[i];
}

int ceiling_blocks() { return 8192; }  // the read stream's workgroups (one sink word each)
constexpr int kCopyBlocks = 16384;

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t st) {
    launch_k(stream_read_kernel, ceiling_blocks(), kCeilThreads, 0, st, static_cast<const i32x4 *>(src), bytes / 16,
             sink);
    return hipGetLastError();
}

hipError_t launch_stream_copy(const void *src, const void *src2, void *dst, int64_t bytes, hipStream_t st) {
    const i32x4 *a = static_cast<const i32x4 *>(src), *b = static_cast<const i32x4 *>(src2);
    i32x4 *d = static_cast<i32x4 *>(dst);
    if (src2) launch_k(stream_copy_kernel<true>, kCopyBlocks, kCeilThreads, 0, st, a, b, d, bytes / 16);
    else launch_k(stream_copy_kernel<false>, kCopyBlocks, kCeilThreads, 0, st, a, b, d, bytes / 16);
    return hipGetLastError();
}

// Measured int8 MFMA ceiling: every wave runs `iters` rounds of kChains
// independent v_mfma_i32_32x32x32_i8 on register operands (no memory traffic
// inside the loop), kMfmaWaves waves per CU, so the matrix pipes stay busy and
// the clock settles where it does under a contraction's load. One word per
// workgroup goes to sink (the accumulators must be formed).
constexpr int kChains = 4;
constexpr int kMfmaThreads = 256;

__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(int64_t iters, uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const i32x4 a = {lane * 0x01010101, 0x02020202, lane, 0x7f7f7f7f};
    const i32x4 b = {0x01010101, lane * 0x00010001, 0x03030303, lane};
    i32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = i32x16{};
    for (int64_t i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    int x = 0;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) x ^= acc[c][r];
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    if (threadIdx.x == 0) sink[blockIdx.x] = (uint32_t)x;
}

int mfma_ceiling_blocks(int cus) { return 4 * cus; }  // 4 workgroups of 4 waves per CU: 4 waves per SIMD

hipError_t launch_mfma_loop(int64_t iters, int blocks, uint32_t *sink, hipStream_t st) {
    launch_k(mfma_loop_kernel, blocks, kMfmaThreads, 0, st, iters, sink);
    return hipGetLastError();
}

int64_t mfma_loop_ops(int64_t iters, int blocks) {
    return (int64_t)blocks * (kMfmaThreads / kWave) * iters * kChains * (2LL * 32 * 32 * 32);
}

}  // namespace mmf
