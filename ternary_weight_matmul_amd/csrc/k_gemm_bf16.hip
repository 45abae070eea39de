// bf16 products of the FusedBitLinear derivative (gfx950), hand-written.
//
// The straight-through derivative of FusedBitLinear ("MatMul-Free LLM 深度分析报告",
// list "可复用的模式与技巧": weight_quant passes the gradient through unchanged)
// has two plain products once the quantised operands are expanded:
//   du = dy W^   (contract over the n outputs)    and    dW = dy^T u^   (over the m rows).
// Both run here as C[M][N] = A[M][K] B[N][K]^T in fp32 from bf16 operands whose
// contraction dimension K is contiguous ("NT"): the ternary values, the int8
// codes and integer-valued scaled inputs are exact in bf16, and the fp32
// accumulation of v_mfma_f32_32x32x16_bf16 keeps the sums to fp32 rounding.
// The operands reach that layout through the expansion and transposes at the
// end of this file: t^T [k][n] from the packed words for du; (dy / s)^T [n][m]
// and q^T [k][m] for dW (zero-padded along m to the K step).
//
// Two kernels share the MFMA tiling and the LDS row layout: where K is a whole
// number of K steps and rows are 16-byte aligned (both products at the layer
// shapes), an LDS-DMA kernel with three stages (gemm_bf16_nt_dma_kernel, below);
// otherwise the register-staged kernel described here.
//
// Tiling of the staged kernel: a workgroup of four waves owns a 128 x 128 block of C; each wave a
// 64 x 64 block (2 x 2 tiles of 32 x 32, 64 accumulators per lane), two
// workgroups per CU. K moves 64 bf16 (128 bytes) per step through two LDS
// stages; the next step's tiles are loaded into registers while the current
// one is multiplied. Rows are 128 bytes in LDS with their 16-byte chunks
// XOR-swizzled by the row, so the 32 rows a fragment read touches fall in
// different banks. Tiles are dealt XCD-major (workgroups are dispatched
// round-robin over the 8 XCDs), eight row strips at a time, so the tiles one
// XCD has in flight share operand strips in its L2. A product with few tiles
// and a long K (dW contracts over every row of the batch) is split along K
// over grid.y: each split writes its own partial block, and a second kernel
// sums the splits in a fixed order (the result does not depend on scheduling).
#include "device_common.hpp"
#include "launch.hpp"

namespace mmf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGM = 128, kGN = 128, kGK = 64;  // workgroup tile, K step (elements)
constexpr int kGRowBytes = kGK * 2;           // 128 bytes of a row per K step
constexpr int kGA = kGM * kGRowBytes;         // 16 KB
constexpr int kGB = kGN * kGRowBytes;         // 16 KB
constexpr int kGStage = kGA + kGB;
constexpr int kGGroupM = 8;

__device__ __forceinline__ int swz(int row, int c16) { return (c16 ^ ((row >> 1) & 7)) << 4; }

// C (+ split * split_stride) = A[m0.., kb..ke) B[n0.., kb..ke)^T for the tile of this workgroup;
// split y of grid.y covers K steps [y * steps_per_split, (y + 1) * steps_per_split).
__global__ __launch_bounds__(256, 2) void gemm_bf16_nt_kernel(const uint16_t *__restrict__ A,
                                                              const uint16_t *__restrict__ B, float *__restrict__ C,
                                                              int M, int N, int K, int64_t lda, int64_t ldb,
                                                              int64_t ldc, int tiles_n, int steps_per_split,
                                                              int64_t split_stride) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kGStage];
    const int G = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int tile = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int tiles_m = G / tiles_n;
    const int group = tile / (kGGroupM * tiles_n);
    const int first_m = group * kGGroupM;
    const int gsz = tiles_m - first_m < kGGroupM ? tiles_m - first_m : kGGroupM;
    const int in_group = tile - group * kGGroupM * tiles_n;
    const int tm = first_m + in_group % gsz, tn = in_group / gsz;
    const int m0 = tm * kGM, n0 = tn * kGN;
    C += (int64_t)blockIdx.y * split_stride;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // wave block: rows wm*64 + [0,64), columns wn*64 + [0,64)
    const int lr = lane & 31, lg = lane >> 5;
    const int all_steps = (K + kGK - 1) / kGK;
    const int s0 = blockIdx.y * steps_per_split;
    const int s1 = s0 + steps_per_split < all_steps ? s0 + steps_per_split : all_steps;

    // staging: A and B 128 rows x 8 chunks each (4 + 4 per thread); rows past M / N and
    // columns past K load zeros
    uint4 ra[4], rb[4];
    auto gload = [&](int ks) {
        const int k0 = ks * kGK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ci = tid + 256 * i, row = ci >> 3, c16 = ci & 7;
            const int kk = k0 + 8 * c16;
            const int ga = m0 + row, gb = n0 + row;
            ra[i] = (ga < M && kk < K) ? *reinterpret_cast<const uint4 *>(A + (int64_t)ga * lda + kk)
                                       : make_uint4(0, 0, 0, 0);
            rb[i] = (gb < N && kk < K) ? *reinterpret_cast<const uint4 *>(B + (int64_t)gb * ldb + kk)
                                       : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
        uint8_t *sa = smem + buf * kGStage;
        uint8_t *sb = sa + kGA;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ci = tid + 256 * i, row = ci >> 3, c16 = ci & 7;
            *reinterpret_cast<uint4 *>(sa + row * kGRowBytes + swz(row, c16)) = ra[i];
            *reinterpret_cast<uint4 *>(sb + row * kGRowBytes + swz(row, c16)) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    auto compute = [&](int buf) {
        const uint8_t *sa = smem + buf * kGStage;
        const uint8_t *sb = sa + kGA;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {  // 16 of K per MFMA: chunk 2 kk + lg of the row
            const int c16 = 2 * kk + lg;
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + lr;
                af[i] = *reinterpret_cast<const bf16x8 *>(sa + row * kGRowBytes + swz(row, c16));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = wn * 64 + j * 32 + lr;
                bfr[j] = *reinterpret_cast<const bf16x8 *>(sb + row * kGRowBytes + swz(row, c16));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };

    if (s0 < s1) {
        gload(s0);
        sstore(0);
        __syncthreads();
        for (int ks = s0; ks < s1; ++ks) {
            const int buf = (ks - s0) & 1;
            if (ks + 1 < s1) gload(ks + 1);
            compute(buf);
            if (ks + 1 < s1) sstore(buf ^ 1);
            __syncthreads();
        }
    }

    // register r of lane l holds row (r / 4) * 8 + (l / 32) * 4 + r % 4, column l % 32 of its tile
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + lr;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
                if (row < M) C[(int64_t)row * ldc + col] = acc[i][j][r];
            }
        }
}

// ----------------------------------------------------------------------------
// K a multiple of 64, 16-byte aligned rows: LDS stages filled by LDS-DMA
// ----------------------------------------------------------------------------
// A BM x BN block of C per workgroup of eight waves, each wave a block of TI x TJ
// tiles of 32 x 32; NS LDS stages are filled straight from memory by 16-byte
// LDS-DMA loads (global_load_lds_dwordx4) NS - 1 K steps ahead of the MFMAs, with
// no staging registers and one barrier per step. Each lane picks the source chunk
// of the LDS slot it fills, which is how the rows get the same XOR swizzle as
// above; rows past M or N read a clamped valid row (their outputs are never
// stored).
template <int BM, int BN, int NS, int TI, int TJ, int BK>
struct DmaGemm {
    static constexpr int WN = BN / (32 * TJ);                  // waves along N
    static constexpr int NW = (BM / (32 * TI)) * WN;           // waves
    static constexpr int NT = NW * 64;
    static constexpr int RB = BK * 2;                          // bytes of a row per K step
    static constexpr int CH = RB / 16;                         // 16-byte chunks of a row
    static constexpr int STAGE = (BM + BN) * RB;               // A rows, then B rows
    static constexpr int A_INS = BM * CH / NT;                 // 16-byte A slots per thread and step
    static constexpr int B_INS = BN * CH / NT;
    static constexpr int LOADS = A_INS + B_INS;                // DMA loads per wave and step
    static_assert(BK == 64 || BK == 32, "K step");
    static_assert(A_INS * NT == BM * CH && B_INS * NT == BN * CH, "whole slots");
    static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS");
    // position of chunk c of a row: XOR-swizzled by the row so that the 16 rows one quarter of
    // a wave reads at the same chunk fall in different banks (128-byte rows: pairs of rows share
    // a bank group; 64-byte rows: quadruples)
    static __device__ __forceinline__ int pos(int row, int c) {
        return CH == 8 ? c ^ ((row >> 1) & 7) : c ^ ((row >> 2) & 3);
    }
};

template <int BM, int BN, int NS, int TI, int TJ, int BK>
__global__ __launch_bounds__((DmaGemm<BM, BN, NS, TI, TJ, BK>::NT)) void gemm_bf16_nt_dma_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, float *__restrict__ C, int M, int N, int64_t lda,
    int64_t ldb, int64_t ldc, int tiles_n, int all_steps, int steps_per_split, int64_t split_stride) {
    using S = DmaGemm<BM, BN, NS, TI, TJ, BK>;
    constexpr int RB = S::RB, CH = S::CH;
    __shared__ __attribute__((aligned(16))) uint8_t smem[NS * S::STAGE];
    const int G = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int tile = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int tiles_m = G / tiles_n;
    const int group = tile / (kGGroupM * tiles_n);
    const int first_m = group * kGGroupM;
    const int gsz = tiles_m - first_m < kGGroupM ? tiles_m - first_m : kGGroupM;
    const int in_group = tile - group * kGGroupM * tiles_n;
    const int tm = first_m + in_group % gsz, tn = in_group / gsz;
    const int m0 = tm * BM, n0 = tn * BN;
    C += (int64_t)blockIdx.y * split_stride;

    constexpr int NW = S::NW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / S::WN, wn = wave % S::WN;  // wave block: rows wm*32*TI + ..., columns wn*32*TJ + ...
    const int lr = lane & 31, lg = lane >> 5;
    const int s0 = blockIdx.y * steps_per_split;
    const int s1 = s0 + steps_per_split < all_steps ? s0 + steps_per_split : all_steps;

    // the source of each of the lane's LDS slots: slot -> (row, position), position p holds
    // the chunk whose swizzled position is p (the swizzle is its own inverse)
    const uint16_t *asrc[S::A_INS];
#pragma unroll
    for (int i = 0; i < S::A_INS; ++i) {
        const int slot = (i * NW + wave) * 64 + lane, row = slot / CH, c16 = S::pos(row, slot % CH);
        const int gr = m0 + row < M ? m0 + row : M - 1;
        asrc[i] = A + (int64_t)gr * lda + 8 * c16;
    }
    const uint16_t *bsrc[S::B_INS];
#pragma unroll
    for (int i = 0; i < S::B_INS; ++i) {
        const int slot = (i * NW + wave) * 64 + lane, row = slot / CH, c16 = S::pos(row, slot % CH);
        const int gr = n0 + row < N ? n0 + row : N - 1;
        bsrc[i] = B + (int64_t)gr * ldb + 8 * c16;
    }
    auto issue = [&](int ks) {
        // LDS byte offset of the step's stage (low half of its generic address) plus the wave's slots
        const uint8_t *base = smem + (ks % NS) * S::STAGE;
        const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base + wave * 64 * 16);
#pragma unroll
        for (int i = 0; i < S::A_INS; ++i) lds_dma16(asrc[i] + ks * BK, lds + i * NW * 64 * 16);
#pragma unroll
        for (int i = 0; i < S::B_INS; ++i) lds_dma16(bsrc[i] + ks * BK, lds + BM * RB + i * NW * 64 * 16);
    };

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

    auto compute = [&](const uint8_t *sa) {
        const uint8_t *sb = sa + BM * RB;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {  // 16 of K per MFMA: chunk 2 kk + lg of the row
            const int c16 = 2 * kk + lg;
            bf16x8 af[TI], bfr[TJ];
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const int row = wm * 32 * TI + i * 32 + lr;
                af[i] = *reinterpret_cast<const bf16x8 *>(sa + row * RB + (S::pos(row, c16) << 4));
            }
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int row = wn * 32 * TJ + j * 32 + lr;
                bfr[j] = *reinterpret_cast<const bf16x8 *>(sb + row * RB + (S::pos(row, c16) << 4));
            }
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };
    // step ks: wait for its loads (this wave's: they retire in order, and those of the steps
    // after it that are already in flight may stay; the barrier then covers every wave's, and
    // every wave has finished with the stage the next loads reuse), start the loads of step
    // ks + NS - 1, multiply
    if (s0 < s1) {
#pragma unroll
        for (int p = 0; p < NS - 1; ++p)
            if (s0 + p < s1) issue(s0 + p);
        for (int ks = s0; ks < s1; ++ks) {
            const int ahead = s1 - 1 - ks < NS - 2 ? s1 - 1 - ks : NS - 2;  // later steps already issued
            vmcnt_wait(ahead * S::LOADS);
            asm volatile("" ::: "memory");  // keep LDS accesses on their side of the barrier
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (ks + NS - 1 < s1) issue(ks + NS - 1);
            compute(smem + (ks % NS) * S::STAGE);
        }
    }

    // register r of lane l holds row (r / 4) * 8 + (l / 32) * 4 + r % 4, column l % 32 of its tile
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int col = n0 + wn * 32 * TJ + j * 32 + lr;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 32 * TI + i * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
                if (row < M) C[(int64_t)row * ldc + col] = acc[i][j][r];
            }
        }
}

// the LDS-DMA configuration the products run with: 256 x 256 blocks, eight waves of 128 x 64,
// two 64 KB stages (measured on MI355X at the 1.3B layer's products, du 32768 x 2048 x 2048
// and dW 2048 x 2048 x 32768: 36-37 % of the dense bf16 peak; 256 x 128 blocks of 64 x 64
// waves with three stages 31-32 %, 256 x 256 of 64 x 128 waves 34 %, of four 128 x 128 waves
// (one wave per SIMD) 32 %, 128 x 128 blocks 27-31 %; K steps of 32 with four 32 KB stages, three
// steps of loads in flight, 34-35 %: the barrier every 16 MFMAs costs more than the cover gains)
constexpr int kDmaBM = 256, kDmaBN = 256, kDmaNS = 2, kDmaTI = 4, kDmaTJ = 2, kDmaBK = 64;
using DmaConfig = DmaGemm<kDmaBM, kDmaBN, kDmaNS, kDmaTI, kDmaTJ, kDmaBK>;

// C[r][c] = sum over the splits in order of part[split][r][c] (row stride ldc in both)
__global__ __launch_bounds__(256) void split_sum_kernel(const float *__restrict__ part, int splits,
                                                        int64_t split_stride, int M, int N, int64_t ldc,
                                                        float *__restrict__ C) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int64_t r = i / N, c = i - r * N;
    const int64_t o = r * ldc + c;
    float v = part[o];
    for (int s_ = 1; s_ < splits; ++s_) v += part[s_ * split_stride + o];
    C[o] = v;
}

// Splits along K for a product of few tiles: enough workgroups for two rounds of
// the CUs' resident workgroups (one per CU for the LDS-DMA kernel, which runs when
// K is a whole number of K steps; two for the staged one), each split at least 8 K steps.
int gemm_bf16_splits(int m, int n, int k) {
    const bool dma = k % kGK == 0;
    const int tiles = dma ? ((m + kDmaBM - 1) / kDmaBM) * ((n + kDmaBN - 1) / kDmaBN)
                          : ((m + kGM - 1) / kGM) * ((n + kGN - 1) / kGN);
    const int want = dma ? 256 : 512;
    const int steps = (k + kGK - 1) / kGK;
    int sp = 1;
    while (sp < 16 && tiles * sp < want && steps / (2 * sp) >= 8) sp *= 2;
    return sp;
}

hipError_t launch_gemm_bf16_nt(const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb, int m, int n, int k,
                               float *c, int64_t ldc, float *part, hipStream_t st) {
    if (m <= 0 || n <= 0) return hipSuccess;
    const int steps = (k + kGK - 1) / kGK;
    const int sp = part ? gemm_bf16_splits(m, n, k) : 1;
    const int per_split = (steps + sp - 1) / sp;
    const int64_t stride = (int64_t)m * ldc;
    // the LDS-DMA kernel wherever every 16-byte slot it fills is whole and aligned
    const bool dma = k % kGK == 0 && lda % 8 == 0 && ldb % 8 == 0 && (reinterpret_cast<uintptr_t>(a) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(b) & 15u) == 0;
    if (dma) {
        const int tiles_m = (m + kDmaBM - 1) / kDmaBM, tiles_n = (n + kDmaBN - 1) / kDmaBN;
        const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)sp);
        const int dsteps = k / kDmaBK, dper = per_split * (kGK / kDmaBK);  // the same K range per split
        launch_k(gemm_bf16_nt_dma_kernel<kDmaBM, kDmaBN, kDmaNS, kDmaTI, kDmaTJ, kDmaBK>, grid, DmaConfig::NT, 0, st,
                 a, b, sp > 1 ? part : c, m, n, lda, ldb, ldc, tiles_n, dsteps, dper, stride);
    } else {
        const int tiles_m = (m + kGM - 1) / kGM, tiles_n = (n + kGN - 1) / kGN;
        const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)sp);
        launch_k(gemm_bf16_nt_kernel, grid, 256, 0, st, a, b, sp > 1 ? part : c, m, n, k, lda, ldb, ldc, tiles_n,
                 per_split, stride);
    }
    if (sp > 1)
        launch_k(split_sum_kernel, (unsigned)(((int64_t)m * n + 255) / 256), 256, 0, st, part, sp, stride, m, n, ldc,
                 c);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Operand layouts
// ---------------------------------------------------------------------------------------
// bf16 bit patterns of t = c - 1 for the offset codes c = 0, 1, 2
__device__ __forceinline__ uint32_t tern_bf16(uint32_t c) { return c == 0 ? 0xBF80u : (c == 2 ? 0x3F80u : 0u); }

// packed [n][k/16] -> t^T bf16 [k][ldn] (ldn >= n, ldn % 8 == 0, columns n..ldn-1 zero): a 64 (k) x 64 (n)
// tile per workgroup through LDS; each thread reads one word (16 k of one n) and the tile is
// written out n-contiguous.
__global__ __launch_bounds__(256) void expand_ternary_t_kernel(const uint32_t *__restrict__ packed, int n, int k,
                                                               uint16_t *__restrict__ out, int ldn) {
    __shared__ uint16_t tile[64][64 + 2];  // [k][n]
    const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    {  // 64 n x 4 words
        const int nn = tid >> 2, w = tid & 3;
        const int gn = n0 + nn, gw = (k0 >> 4) + w;
        const uint32_t word = (gn < n && 16 * gw < k) ? packed[(int64_t)gn * (k >> 4) + gw] : 0x55555555u;  // code 1: t = 0
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t c = (word >> (8 * (e & 3) + 2 * (e >> 2))) & 3u;
            tile[16 * w + e][nn] = (uint16_t)tern_bf16(c);
        }
    }
    __syncthreads();
    // 64 k rows x 64 n: each thread writes 16 consecutive n of one k row (two 16-byte stores)
    const int kk = tid >> 2, part = tid & 3;
    const int gk = k0 + kk;
    if (gk >= k) return;
    uint32_t v[8];
#pragma unroll
    for (int p = 0; p < 8; ++p)
        v[p] = (uint32_t)tile[kk][16 * part + 2 * p] | ((uint32_t)tile[kk][16 * part + 2 * p + 1] << 16);
    // two 8-element pieces, each written only inside the row (ldn % 8 == 0)
    const int gn = n0 + 16 * part;
    uint4 *o = reinterpret_cast<uint4 *>(out + (int64_t)gk * ldn + gn);
    if (gn < ldn) o[0] = make_uint4(v[0], v[1], v[2], v[3]);
    if (gn + 8 < ldn) o[1] = make_uint4(v[4], v[5], v[6], v[7]);
}

hipError_t launch_expand_ternary_t(const uint32_t *packed, int n, int k, uint16_t *out, int ldn, hipStream_t st) {
    if (n <= 0 || k <= 0) return hipSuccess;
    const dim3 grid((unsigned)((ldn + 63) / 64), (unsigned)((k + 63) / 64));
    launch_k(expand_ternary_t_kernel, grid, 256, 0, st, packed, n, k, out, ldn);
    return hipGetLastError();
}

// out [cols][ldm] bf16 = transpose of src [rows][cols] (cols % 4 == 0) with each row r scaled
// by 1 / s[r] (SCALE) or as it is; zeros for r in [rows, ldm). 64 x 64 tiles through LDS, fp32
// in LDS; the product is rounded once, to bf16.
template <typename T, bool SCALE>
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const T *__restrict__ src, const float *__restrict__ s,
                                                             int64_t rows, int cols, uint16_t *__restrict__ out,
                                                             int64_t ldm) {
    __shared__ float tile[64][64 + 1];  // [row][col]
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    const int c0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    // read: 64 rows x 64 cols, 16 elements per thread (4 rows x 4 consecutive cols, one
    // 4-element piece each: cols % 4 == 0, so a piece is whole and aligned or wholly past the end)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int rr = (tid >> 4) + 16 * q, cc = 4 * (tid & 15);
        const int64_t gr = r0 + rr;
        const int gc = c0 + cc;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (gr < rows && gc < cols) {
            const int64_t o = gr * cols + gc;
            if constexpr (sizeof(T) == 1) {
                const uint32_t w = *reinterpret_cast<const uint32_t *>(src + o);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (float)(int8_t)((w >> (8 * e)) & 0xffu);
            } else {
                const float4 x = load_act4(src, o);
                v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
            }
            if constexpr (SCALE) {
                const float inv = s[gr];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = __fdiv_rn(v[e], inv);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[rr][cc + e] = v[e];
    }
    __syncthreads();
    // write: 64 cols (out rows) x 64 rows (out columns), 16 per thread, 8-element (16-byte) pieces
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int oc = (tid >> 3) + 32 * q;  // out row = src column
        const int orr = 8 * (tid & 7);       // first of 8 out columns = src rows
        const int gc = c0 + oc;
        const int64_t gr = r0 + orr;
        if (gc >= cols || gr >= ldm) continue;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
            w[p] = (uint32_t)f32_to_bf16(tile[orr + 2 * p][oc]) | ((uint32_t)f32_to_bf16(tile[orr + 2 * p + 1][oc]) << 16);
        *reinterpret_cast<uint4 *>(out + (int64_t)gc * ldm + gr) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

hipError_t launch_transpose_bf16(const void *src, int src_kind, const float *s, int64_t rows, int cols, uint16_t *out,
                                 int64_t ldm, hipStream_t st) {
    if (cols <= 0 || ldm <= 0) return hipSuccess;
    const dim3 grid((unsigned)((ldm + 63) / 64), (unsigned)((cols + 63) / 64));
    switch (src_kind) {
        case 0: launch_k(transpose_bf16_kernel<float, true>, grid, 256, 0, st, static_cast<const float *>(src), s, rows, cols, out, ldm); break;
        case 1: launch_k(transpose_bf16_kernel<uint16_t, true>, grid, 256, 0, st, static_cast<const uint16_t *>(src), s, rows, cols, out, ldm); break;
        default: launch_k(transpose_bf16_kernel<int8_t, false>, grid, 256, 0, st, static_cast<const int8_t *>(src), s, rows, cols, out, ldm); break;
    }
    return hipGetLastError();
}

}  // namespace mmf
