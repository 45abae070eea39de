// The token-to-token loop of generation (gfx950): embedding rows and the greedy
// choice of the next token.
//
// "MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，剩下什麼", section
// "安裝與初始化：三行指令與一個 config 物件": the default model has a 32000-token
// vocabulary, width 2048 and 24 blocks, and the project ships a generation
// example. The head is read as one more FusedBitLinear (every projection of the
// model is ternary); its logits are acc * dq with one dq > 0 per row, so the
// greedy token is the smallest index of the largest exact int32 sum acc, and
// the choice is made on the integers, never on rounded logits.
#include "device_common.hpp"
#include "launch.hpp"

namespace mmf {

// out[i][:] = table[ids[i]][:], a zero row for an id outside [0, vocab). One
// thread copies 16 bytes; grid.y covers the row's 16-byte pieces.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t *__restrict__ ids, const uint4 *__restrict__ table,
                                                    int64_t vocab, int64_t pieces, uint4 *__restrict__ out) {
    const int64_t row = blockIdx.x;
    const int64_t p = (int64_t)blockIdx.y * 256 + threadIdx.x;
    if (p >= pieces) return;
    const int64_t id = ids[row];
    const bool ok = id >= 0 && id < vocab;
    out[row * pieces + p] = ok ? table[id * pieces + p] : make_uint4(0u, 0u, 0u, 0u);
}

// Per row of acc [m][n] (n % 4 == 0): the smallest index of the largest value.
// Thread t scans the 4-element groups t, t + 256, ... in increasing order and
// keeps the first maximum it meets; the 256 candidates meet in LDS, larger
// value first, smaller index on a tie.
__global__ __launch_bounds__(256) void argmax_rows_kernel(const int32_t *__restrict__ acc, int64_t n,
                                                          int32_t *__restrict__ tokens) {
    __shared__ int32_t bv[256];
    __shared__ int32_t bi[256];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int4 *src = reinterpret_cast<const int4 *>(acc + row * n);
    int32_t best = INT32_MIN, arg = INT32_MAX;
    for (int64_t g = tid; g < n / 4; g += 256) {
        const int4 v = src[g];
        const int32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e[j] > best) {
                best = e[j];
                arg = (int32_t)(4 * g + j);
            }
    }
    bv[tid] = best;
    bi[tid] = arg;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) {
            const int32_t ov = bv[tid + w], oi = bi[tid + w];
            if (ov > bv[tid] || (ov == bv[tid] && oi < bi[tid])) {
                bv[tid] = ov;
                bi[tid] = oi;
            }
        }
        __syncthreads();
    }
    if (tid == 0) tokens[row] = bi[0];
}

hipError_t launch_embed(const int32_t *ids, int64_t count, const void *table, int64_t vocab, int64_t row_bytes,
                        void *out, hipStream_t st) {
    if (count <= 0) return hipSuccess;
    const int64_t pieces = row_bytes / 16;
    const dim3 grid((unsigned)count, (unsigned)((pieces + 255) / 256));
    launch_k(embed_kernel, grid, 256, 0, st, ids, static_cast<const uint4 *>(table), vocab, pieces, static_cast<uint4 *>(out));
    return hipGetLastError();
}

hipError_t launch_argmax_rows(const int32_t *acc, int64_t m, int64_t n, int32_t *tokens, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    launch_k(argmax_rows_kernel, (unsigned)m, 256, 0, st, acc, n, tokens);
    return hipGetLastError();
}

}  // namespace mmf
