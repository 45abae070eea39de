// Exact int8 x ternary contraction with fused epilogues (gfx950).
//
// FusedBitLinear's product of int8 activation codes with ternary weights
// ("MatMul-Free LLM 深度分析报告", table "创新之处" and section "关键设计决策": the
// published code still runs a float GEMM on the ternary values; here the
// product is exact integer arithmetic). The weights stay packed 2 bits per
// value in HBM (16 per 32-bit word, offset codes c = t + 1) and are decoded
// in registers with one shift and one mask per 4 values: a word decodes
// straight into the 16-byte int8 operand of one MFMA lane. The int8 MFMA
// computes sum c*q; sum t*q = sum c*q - sum q is exact (|acc| < 2^24), with
// sum q a by-product of the activation quantiser (prefill) or of one more MFMA
// against an all-ones operand (decode).
//
// Prefill (m > 64): 128 x (NG * 64 * JN) output tiles (JN = 4, 2, 1 for one,
// two, three groups), four waves of 64 x (NG * 32 * JN), v_mfma_i32_32x32x32_i8,
// K staged 128 bytes at a time through
// double-buffered LDS (activation tile XOR-swizzled, packed weights padded to
// a 48-byte row stride: both conflict-free for 16-lane groups). Tiles are
// assigned XCD-major, and grouped eight row strips at a time, so that the
// workgroups of one XCD share activation strips and weight tiles in its L2.
// Decode (m <= 64): one workgroup per 16-row block and 16 to 64 output
// channels, up to 16 waves splitting K, v_mfma_i32_16x16x64_i8, partial sums
// reduced in LDS.
//
// NG groups of output channels share an output tile so that the epilogue sees
// the matching channels of several projections in one lane: i/f/g for the
// token mixer's gates, the two halves of gate_proj for the SiLU-gated MLP
// ("MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，剩下什麼", section
// "HGRNBitBlock 的結構").
#include "device_common.hpp"
#include "launch.hpp"
#include "epilogue.hpp"

#include <atomic>
#include <mutex>

namespace mmf {

// ----------------------------------------------------------------------------
// Prefill: tiled int8 MFMA contraction
// ----------------------------------------------------------------------------
constexpr int kBM = 128;      // rows per tile
constexpr int kBK = 128;      // k (bytes of codes) per LDS stage
constexpr int kBStride = 48;  // bytes per packed-weight row in LDS (32 used)
constexpr int kGroupM = 8;    // row strips per group of the tile order

template <int NG, int JN, bool SHARED_A>
struct TileShape {
    static constexpr int BNC = 64 * JN;                 // channels per group per tile
    static constexpr int NA = SHARED_A ? 1 : NG;        // activation tiles per stage
    static constexpr int BROWS = NG * BNC;              // packed rows per stage
    static constexpr int A_STAGE = NA * kBM * kBK;
    static constexpr int B_STAGE = BROWS * kBStride;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int A_LD = (kBM * kBK / 16) / 256; // 16-byte loads per thread per tile
    static constexpr int B_CH = BROWS * 2;              // 16-byte chunks of packed weights per stage
    static constexpr int B_LD = (B_CH + 255) / 256;
};

// Epilogue of one wave's block of the 32x32 MFMA tiles: rows mw + [0, 64) and
// columns cw + [0, 32 JN) of each of the NG groups (register r of lane l holds
// row (r/4)*8 + (l/32)*4 + r%4 and column l%32 of its tile). For each batch of
// 8 registers, every load the epilogue needs (quantiser sums and scales, the
// residual or the old state) is issued before the batch's first store: the
// compiler has to assume that a store may alias any later load, so loads mixed
// in with the stores would each wait for the stores before them. RT is the
// element type of that operand, fixed at compile time so that a bf16 operand's
// widening is not tied to its load. Rows past M and columns past nc load from
// a clamped, valid address and are not stored.
template <int EPI, int NG, int JN, typename RT>
__device__ __forceinline__ void wave_epilogue_t(const ContractArgs &p, const i32x16 (&acc)[2][NG][JN], int64_t mw,
                                                int cw, int lane) {
    constexpr bool PRE = EPI == EPI_RESID || EPI == EPI_GATES_STEP;
    const RT *pre_src = static_cast<const RT *>(EPI == EPI_RESID ? p.res : p.out0);
    constexpr int RB = 8;
    const int lr = lane & 31, lg = lane >> 5;
    const int64_t M = p.m;
    float sw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sw[g] = weight_sw(p.mu[g]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += RB) {
            int32_t sq[RB][NG];
            float dq[RB][NG];
            float pre[RB][JN];
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                const int r = r0 + rr;
                const int64_t m = mw + i * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
                const int64_t mc = m < M ? m : M - 1;
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    sq[rr][g] = p.sumq[g][mc];
                    dq[rr][g] = __builtin_amdgcn_rcpf(p.s[g][mc] * sw[g]);
                }
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    const int c = cw + j * 32 + lr;
                    pre[rr][j] = PRE ? load_act(pre_src, mc * p.nc + (c < p.nc ? c : p.nc - 1)) : 0.0f;
                }
            }
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                const int r = r0 + rr;
                const int64_t m = mw + i * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
                if (m >= M) continue;
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    const int c = cw + j * 32 + lr;
                    if (c < p.nc) {
                        int32_t v[NG];
#pragma unroll
                        for (int g = 0; g < NG; ++g) v[g] = acc[i][g][j][r] - sq[rr][g];
                        epilogue_vals<EPI, NG, PRE>(p, m, c, v, dq[rr], pre[rr][j]);
                    }
                }
            }
        }
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return f32_to_bf16(v); }

// The same epilogue without stage probes and with every element type fixed at
// compile time (RT residual, OT output of linear/resid, AT the g or z output),
// addressed as one wave-uniform base plus 32-bit lane offsets. FULL: the wave's
// block lies inside the output, so no row or column checks. Bit-identical to
// epilogue_vals: the same operations in the same order.
template <int EPI, int NG, int JN, typename RT, typename OT, typename AT, bool FULL>
__device__ __forceinline__ void fast_epilogue(const ContractArgs &p, const i32x16 (&acc)[2][NG][JN], int64_t mw,
                                              int cw, int lane) {
    constexpr int RB = 8;
    const int lr = lane & 31, lg = lane >> 5;
    const int64_t M = p.m;
    const int nc = p.nc;
    const int64_t wbase = mw * nc + cw;          // element (mw, cw), wave-uniform
    const int lane_rel = lg * 4 * nc + lr;        // lane's offset from it (row lg*4, column lr)
    float sw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sw[g] = weight_sw(p.mu[g]);
    const RT *res = static_cast<const RT *>(p.res) + wbase;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += RB) {
            int32_t sq[RB][NG];
            float dq[RB][NG];
            float pre[RB][JN];
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                const int r = r0 + rr;
                const int rowoff = i * 32 + (r >> 2) * 8 + (r & 3);
                int64_t m = mw + lg * 4 + rowoff;
                if (!FULL) m = m < M ? m : M - 1;
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    sq[rr][g] = p.sumq[g][m];
                    dq[rr][g] = __builtin_amdgcn_rcpf(p.s[g][m] * sw[g]);
                }
                if constexpr (EPI == EPI_RESID) {
#pragma unroll
                    for (int j = 0; j < JN; ++j) {
                        int rel = lane_rel + rowoff * nc + j * 32;
                        if (!FULL) {
                            const int c = cw + j * 32 + lr;
                            rel = (int)(m - mw) * nc + (c < nc ? c : nc - 1) - cw;
                        }
                        pre[rr][j] = to_f32(res[rel]);
                    }
                }
            }
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
                const int r = r0 + rr;
                const int rowoff = i * 32 + (r >> 2) * 8 + (r & 3);
                if (!FULL && mw + lg * 4 + rowoff >= M) continue;
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    if (!FULL && cw + j * 32 + lr >= nc) continue;
                    const int rel = lane_rel + rowoff * nc + j * 32;
                    float y[NG];
#pragma unroll
                    for (int g = 0; g < NG; ++g) y[g] = (float)(acc[i][g][j][r] - sq[rr][g]) * dq[rr][g];
                    if constexpr (EPI == EPI_LINEAR) {
                        (static_cast<OT *>(p.out0) + wbase)[rel] = from_f32<OT>(y[0]);
                    } else if constexpr (EPI == EPI_RESID) {
                        (static_cast<OT *>(p.out0) + wbase)[rel] = from_f32<OT>(pre[rr][j] + y[0]);
                    } else if constexpr (EPI == EPI_GATES) {
                        const float f = sigmoid_fast(y[1]);
                        const float xt = (1.0f - f) * silu_fast(y[0]);
                        (static_cast<float *>(p.out0) + wbase)[rel] = f;
                        (static_cast<float *>(p.out1) + wbase)[rel] = xt;
                        (static_cast<AT *>(p.out2) + wbase)[rel] = from_f32<AT>(y[2]);
                    } else if constexpr (EPI == EPI_GLU) {
                        (static_cast<AT *>(p.out0) + wbase)[rel] = from_f32<AT>(silu_fast(y[0]) * y[1]);
                    }
                }
            }
        }
}

template <int EPI, int NG, int JN, bool FULL>
__device__ __forceinline__ void fast_dispatch(const ContractArgs &p, const i32x16 (&acc)[2][NG][JN], int64_t mw,
                                              int cw, int lane) {
    const bool ob = p.out_type == ACT_BF16, rb = p.res_type == ACT_BF16, ab = p.aux_type == ACT_BF16;
    if constexpr (EPI == EPI_GATES || EPI == EPI_GLU) {
        if (ab) fast_epilogue<EPI, NG, JN, float, float, uint16_t, FULL>(p, acc, mw, cw, lane);
        else fast_epilogue<EPI, NG, JN, float, float, float, FULL>(p, acc, mw, cw, lane);
    } else if constexpr (EPI == EPI_RESID) {
        if (ob && rb) fast_epilogue<EPI, NG, JN, uint16_t, uint16_t, float, FULL>(p, acc, mw, cw, lane);
        else if (ob) fast_epilogue<EPI, NG, JN, float, uint16_t, float, FULL>(p, acc, mw, cw, lane);
        else if (rb) fast_epilogue<EPI, NG, JN, uint16_t, float, float, FULL>(p, acc, mw, cw, lane);
        else fast_epilogue<EPI, NG, JN, float, float, float, FULL>(p, acc, mw, cw, lane);
    } else if constexpr (EPI == EPI_LINEAR) {
        if (ob) fast_epilogue<EPI, NG, JN, float, uint16_t, float, FULL>(p, acc, mw, cw, lane);
        else fast_epilogue<EPI, NG, JN, float, float, float, FULL>(p, acc, mw, cw, lane);
    }
}

template <int EPI, int NG, int JN>
__device__ __forceinline__ void wave_epilogue(const ContractArgs &p, const i32x16 (&acc)[2][NG][JN], int64_t mw,
                                              int cw, int lane) {
    // fast path: no stage probes (and not the decode step's state update, which
    // reaches this kernel only for batches above the GEMV path's limit)
    if (EPI != EPI_GATES_STEP && !p.acc_probe && !p.aux_probe) {
        if (mw + 64 <= p.m && cw + 32 * JN <= p.nc)
            fast_dispatch<EPI, NG, JN, true>(p, acc, mw, cw, lane);
        else
            fast_dispatch<EPI, NG, JN, false>(p, acc, mw, cw, lane);
        return;
    }
    // the residual comes in the activation type; the recurrent state is fp32
    if constexpr (EPI == EPI_RESID) {
        if (p.res_type == ACT_BF16) {
            wave_epilogue_t<EPI, NG, JN, uint16_t>(p, acc, mw, cw, lane);
            return;
        }
    }
    wave_epilogue_t<EPI, NG, JN, float>(p, acc, mw, cw, lane);
}

// Two workgroups per CU, except with one activation tile per group and three
// groups (i/f/g with distinct gains), whose registers allow one.
template <int NG, bool SHARED_A>
constexpr int tgemm_min_blocks() { return !SHARED_A && NG == 3 ? 1 : 2; }

template <int NG, int JN, bool SHARED_A, int EPI>
__global__ __launch_bounds__(256, (tgemm_min_blocks<NG, SHARED_A>())) void tgemm_kernel(const ContractArgs p,
                                                                                        const int tiles_n) {
    using S = TileShape<NG, JN, SHARED_A>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::STAGE];

    // XCD-major tile order: the idx-th workgroup dispatched to XCD x (blocks are
    // dealt round-robin over 8 XCDs) takes the idx-th tile of x's contiguous range.
    const int G = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int tile = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    // Grouped order: kGroupM row strips at a time, row-fastest, sweeping the
    // columns. The tiles one XCD has in flight then share a few activation
    // strips and a few packed-weight tiles, both kept in its L2.
    const int tiles_m = G / tiles_n;
    const int group = tile / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gsz = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
    const int in_group = tile - group * kGroupM * tiles_n;
    const int tm = first_m + in_group % gsz, tn = in_group / gsz;
    const int64_t m0 = (int64_t)tm * kBM;
    const int n0 = tn * S::BNC;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lg = lane >> 5;
    const int K = p.k, KW = K >> 4;
    const int64_t M = p.m;
    const int ktiles = (K + kBK - 1) / kBK;
    const bool bvec = (KW & 3) == 0;

    uint4 ra[S::NA][S::A_LD];
    uint4 rb[S::B_LD];

    auto gload = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int a = 0; a < S::NA; ++a) {
#pragma unroll
            for (int i = 0; i < S::A_LD; ++i) {
                const int ci = tid + 256 * i;
                const int row = ci >> 3, c16 = ci & 7;
                const int64_t gm = m0 + row;
                const int kk = k0 + 16 * c16;
                ra[a][i] = (gm < M && kk < K) ? *reinterpret_cast<const uint4 *>(p.A[a] + gm * K + kk)
                                              : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < S::B_LD; ++i) {
            const int ci = tid + 256 * i;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (ci < S::B_CH) {
                const int row = ci >> 1, half = ci & 1;
                const int gi = row / S::BNC, r = row - gi * S::BNC;
                const int gn = n0 + r;
                const int w0 = (k0 >> 4) + 4 * half;
                if (gn < p.nc) {
                    const uint32_t *src = p.B[gi] + (int64_t)gn * KW + w0;
                    if (bvec && w0 + 4 <= KW) {
                        v = *reinterpret_cast<const uint4 *>(src);
                    } else {
                        v.x = w0 + 0 < KW ? src[0] : 0u;
                        v.y = w0 + 1 < KW ? src[1] : 0u;
                        v.z = w0 + 2 < KW ? src[2] : 0u;
                        v.w = w0 + 3 < KW ? src[3] : 0u;
                    }
                }
            }
            rb[i] = v;
        }
    };

    auto sstore = [&](int buf) {
        uint8_t *sa = smem + buf * S::STAGE;
        uint8_t *sb = sa + S::A_STAGE;
#pragma unroll
        for (int a = 0; a < S::NA; ++a) {
#pragma unroll
            for (int i = 0; i < S::A_LD; ++i) {
                const int ci = tid + 256 * i;
                const int row = ci >> 3, c16 = ci & 7;
                *reinterpret_cast<uint4 *>(sa + a * kBM * kBK + row * kBK + ((c16 ^ ((row >> 1) & 7)) << 4)) = ra[a][i];
            }
        }
#pragma unroll
        for (int i = 0; i < S::B_LD; ++i) {
            const int ci = tid + 256 * i;
            if (ci < S::B_CH) *reinterpret_cast<uint4 *>(sb + (ci >> 1) * kBStride + (ci & 1) * 16) = rb[i];
        }
    };

    i32x16 acc[2][NG][JN];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int j = 0; j < JN; ++j) acc[i][g][j] = i32x16{};

    auto compute = [&](int buf) {
        const uint8_t *sa = smem + buf * S::STAGE;
        const uint8_t *sb = sa + S::A_STAGE;
        uint4 bw[NG][JN];
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int j = 0; j < JN; ++j) {
                const int brow = g * S::BNC + wn * (32 * JN) + j * 32 + lr;
                bw[g][j] = *reinterpret_cast<const uint4 *>(sb + brow * kBStride + lg * 16);
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            i32x4 af[2][S::NA];
            const int c = 4 * lg + ks;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + lr;
#pragma unroll
                for (int a = 0; a < S::NA; ++a)
                    af[i][a] = *reinterpret_cast<const i32x4 *>(sa + a * kBM * kBK + row * kBK + ((c ^ ((row >> 1) & 7)) << 4));
            }
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    const uint32_t word = ks == 0 ? bw[g][j].x : ks == 1 ? bw[g][j].y : ks == 2 ? bw[g][j].z : bw[g][j].w;
                    const i32x4 b = decode_word(word);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][g][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i][SHARED_A ? 0 : g], b, acc[i][g][j], 0, 0, 0);
                }
        }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < ktiles; ++kt) {
        if (kt + 1 < ktiles) gload(kt + 1);
        compute(kt & 1);
        if (kt + 1 < ktiles) sstore((kt + 1) & 1);
        __syncthreads();
    }

    wave_epilogue<EPI, NG, JN>(p, acc, m0 + wm * 64, n0 + wn * (32 * JN), lane);
}

// ----------------------------------------------------------------------------
// Prefill, K % 128 == 0: three LDS stages filled by 16-byte LDS-DMA loads
// ----------------------------------------------------------------------------
// Same tiles, MFMAs and epilogue as tgemm_kernel, but the global -> LDS copy
// goes straight into LDS (global_load_lds_dwordx4: lane L of an instruction
// fills LDS bytes [16L, 16L + 16) past the instruction's base), two K steps
// ahead of the MFMAs, with no staging registers. A lane picks the source of
// its LDS slot, which is how the activation tile gets its XOR swizzle; rows
// past M or N are clamped to a valid row (their outputs are never stored).
// Packed weights use a 32-byte row stride with the two 16-byte halves swapped
// on every other group of 8 rows (conflict-free reads for 16-lane groups).
// One bare barrier per K step: each wave first waits (vmcnt, loads retire in
// order) for its own loads of the step, so after the barrier the whole step
// is in LDS and every wave has finished with the stage the next loads reuse.
template <int NG, int JN>
struct DmaShape {
    static constexpr int BNC = 64 * JN;
    static constexpr int BROWS = NG * BNC;
    static constexpr int A_BYTES = kBM * kBK;                      // 16 KB
    static constexpr int B_SLOTS = (2 * BROWS + 255) / 256 * 256;  // 16-byte slots, whole waves
    static constexpr int STAGE = A_BYTES + B_SLOTS * 16;
    static constexpr int A_INS = A_BYTES / 16 / 256;              // DMA instructions per wave per step
    static constexpr int B_INS = B_SLOTS / 256;
    static constexpr int LOADS = A_INS + B_INS;
};
constexpr int kStages = 3;

template <int NG, int JN, int EPI>
__global__ __launch_bounds__(256, 2) void tgemm_dma_kernel(const ContractArgs p, const int tiles_n) {
    using S = DmaShape<NG, JN>;
    // one LDS object per stage, so the compiler can tell the stage being read
    // from the stages LDS-DMA loads are still filling
    __shared__ __attribute__((aligned(16))) uint8_t st0[S::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[S::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[S::STAGE];

    const int G = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int tile = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int tiles_m = G / tiles_n;
    const int group = tile / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gsz = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
    const int in_group = tile - group * kGroupM * tiles_n;
    const int tm = first_m + in_group % gsz, tn = in_group / gsz;
    const int64_t m0 = (int64_t)tm * kBM;
    const int n0 = tn * S::BNC;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lg = lane >> 5;
    const int K = p.k, KW = K >> 4;
    const int64_t M = p.m;
    const int ktiles = K / kBK;

    // per-lane sources of its DMA slots (advanced by the K offset each step)
    const int8_t *asrc[S::A_INS];
#pragma unroll
    for (int i = 0; i < S::A_INS; ++i) {
        const int slot = (i * 4 + wave) * 64 + lane;
        const int row = slot >> 3, pc = slot & 7;
        const int c16 = pc ^ ((row >> 1) & 7);
        const int64_t gm = m0 + row < M ? m0 + row : M - 1;
        asrc[i] = p.A[0] + gm * K + 16 * c16;
    }
    const uint32_t *bsrc[S::B_INS];
#pragma unroll
    for (int i = 0; i < S::B_INS; ++i) {
        const int slot = (i * 4 + wave) * 64 + lane;
        int row = slot >> 1;
        const int half = (slot & 1) ^ ((row >> 3) & 1);
        if (row >= S::BROWS) row = 0;  // padding slots: any valid source
        const int gi = row / S::BNC, r = row - gi * S::BNC;
        const int gn = n0 + r < p.nc ? n0 + r : p.nc - 1;
        bsrc[i] = p.B[gi] + (int64_t)gn * KW + 4 * half;
    }
    auto issue = [&](int kt, uint8_t *base) {
        // LDS byte offset of the stage (low half of its generic address)
        const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base + wave * 64 * 16);
#pragma unroll
        for (int i = 0; i < S::A_INS; ++i) lds_dma16(asrc[i] + kt * kBK, lds + i * 4 * 64 * 16);
#pragma unroll
        for (int i = 0; i < S::B_INS; ++i)
            lds_dma16(bsrc[i] + kt * (kBK / 16), lds + S::A_BYTES + i * 4 * 64 * 16);
    };

    i32x16 acc[2][NG][JN];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int j = 0; j < JN; ++j) acc[i][g][j] = i32x16{};

    auto compute = [&](const uint8_t *sa) {
        const uint8_t *sb = sa + S::A_BYTES;
        uint4 bw[NG][JN];
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int j = 0; j < JN; ++j) {
                const int brow = g * S::BNC + wn * (32 * JN) + j * 32 + lr;
                bw[g][j] = *reinterpret_cast<const uint4 *>(sb + brow * 32 + ((lg ^ ((brow >> 3) & 1)) << 4));
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            i32x4 af[2];
            const int c = 4 * lg + ks;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + lr;
                af[i] = *reinterpret_cast<const i32x4 *>(sa + row * kBK + ((c ^ ((row >> 1) & 7)) << 4));
            }
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    const uint32_t word = ks == 0 ? bw[g][j].x : ks == 1 ? bw[g][j].y : ks == 2 ? bw[g][j].z : bw[g][j].w;
                    const i32x4 b = decode_word(word);
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][g][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], b, acc[i][g][j], 0, 0, 0);
                }
        }
    };

    // step kt: wait for its loads, barrier, start the loads of step kt+2 into
    // the stage step kt-1 used, then compute step kt
    auto step = [&](int kt, const uint8_t *cur, uint8_t *next2) {
        vmcnt_wait(kt + 1 < ktiles ? S::LOADS : 0);  // this wave's loads of step kt have landed
        asm volatile("" ::: "memory");                 // keep LDS accesses on their side of the barrier
        __builtin_amdgcn_s_barrier();                  // ... and everyone's; next2 is no longer read
        asm volatile("" ::: "memory");
        if (kt + 2 < ktiles) issue(kt + 2, next2);
        compute(cur);
    };
    issue(0, st0);
    if (ktiles > 1) issue(1, st1);
    for (int kt = 0; kt < ktiles; kt += kStages) {
        step(kt, st0, st2);
        if (kt + 1 < ktiles) step(kt + 1, st1, st0);
        if (kt + 2 < ktiles) step(kt + 2, st2, st1);
    }

    wave_epilogue<EPI, NG, JN>(p, acc, m0 + wm * 64, n0 + wn * (32 * JN), lane);
}

// ----------------------------------------------------------------------------
// Decode: m <= 64 rows, latency-bound weight streaming
// ----------------------------------------------------------------------------
// One workgroup per CB blocks of 16 output channels (x NG groups). K is cut
// into slices of 4*WPL words, dealt to up to 16 waves. A lane (column lc,
// word group lg) owns WPL consecutive words of its column in a slice and
// issues every load of the slice -- weights as 16-byte runs, activation codes
// of its row block as 16-byte chunks -- before its first MFMA: with up to two
// slices per wave (SPW = 2) both slices' loads go first, so a GEMV costs about
// one memory round trip; with more, two register sets alternate. The codes
// of a slice are 4x the bytes of one 16-channel block of weights, so the CB
// blocks share each activation fragment. The sum of the codes of a row comes
// from one more MFMA per word against an all-ones operand (sum q in the same
// lane layout as sum c*q), so each wave stores sum (c - 1) q = sum t*q of its
// slices and the quantiser need not form sum q. Each wave's partial sums go to
// its own LDS slot and are summed in wave order (exact integers). RT is the
// element type of the residual (EPI_RESID) or state (EPI_GATES_STEP) operand.
//
// Workgroup size limit of a GEMV variant: the ones with per-group activation
// codes and several groups hold more registers than a 1024-thread workgroup
// leaves a wave (128), so they run 512 threads (256).
template <int NG, bool SHARED_A>
constexpr int gemv_max_threads() { return NG >= 2 && !SHARED_A ? 512 : 1024; }

// Three or four outputs per thread mean fewer than 2 CB waves (at most 448
// threads): such launches get the registers of a 512-thread workgroup.
template <int NG, bool SHARED_A, int EPT>
constexpr int gemv_bound() { return EPT >= 3 ? 512 : gemv_max_threads<NG, SHARED_A>(); }

template <int NG, bool SHARED_A, int EPI, int WPL, typename RT, int EPT, int SPW, int CB>
__global__ __launch_bounds__((gemv_bound<NG, SHARED_A, EPT>())) void tgemv_kernel(const ContractArgs p,
                                                                               const int nslices) {
    // one block of 16 rows per workgroup (grid.y covers the row blocks): with
    // more rows per workgroup each one reads all their codes and fewer
    // workgroups pull weights (measured 1.5x slower at 64 rows)
    constexpr int MB = 1;
    constexpr int NA = SHARED_A ? 1 : NG;
    constexpr int PART = MB * CB * NG * 256;  // one wave's partial sums
    extern __shared__ int32_t part[];         // [waves][PART]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int lc = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16 * CB;
    const int K = p.k, KW = K >> 4;
    const int64_t M = p.m;
    const int64_t row0 = (int64_t)blockIdx.y * 16 * MB;  // first row of this workgroup's row blocks
    int gn[CB];  // columns past nc load a valid row; never stored
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) gn[cb] = min(n0 + cb * 16 + lc, p.nc - 1);
    // weight scales, the quantiser's per-row scales and the epilogue operands
    // (residual / old state) do not depend on the contraction: load
    // them before it, unconditionally (clamped to a valid element; the values
    // of outputs that are not stored go unused) so that no wait for them comes
    // before the contraction's own loads. Output idx of the workgroup: row block
    // idx / (256 CB), channel block (idx / 256) % CB, row (idx / 16) % 16, channel idx % 16.
    float mu_v[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) mu_v[g] = *p.mu[g];
    constexpr bool PRE = EPI == EPI_RESID || EPI == EPI_GATES_STEP;
    float pre[EPT], sc_e[EPT][NG];
    const RT *pre_src = static_cast<const RT *>(EPI == EPI_RESID ? p.res : p.out0);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int idx = tid + e * blockDim.x;
        const int64_t m = row0 + (int64_t)(idx / (256 * CB)) * 16 + ((idx >> 4) & 15);
        const int64_t mc = m < M ? m : M - 1;
        const int c = n0 + ((idx >> 8) % CB) * 16 + (idx & 15);
        pre[e] = PRE ? load_act(pre_src, mc * p.nc + (c < p.nc ? c : p.nc - 1)) : 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) sc_e[e][g] = p.s[g][mc];
    }

    i32x4 acc[MB][CB][NG], accq[MB][NA];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[mb][cb][g] = i32x4{};
#pragma unroll
        for (int q = 0; q < NA; ++q) accq[mb][q] = i32x4{};
    }

    // Every load of a slice is unconditional: words past the row end are
    // clamped and their weights zeroed (offset code 0 adds nothing to sum c*q;
    // the all-ones operand is zeroed for them too), rows past m are clamped
    // (their sums are never stored). An activation fragment
    // serves the CB channel blocks and NG groups of the workgroup.
    const bool whole = (KW % (4 * WPL)) == 0;
    auto load_slice = [&](int sl, uint32_t (&bw)[CB][NG][WPL], i32x4 (&a)[MB][NA][WPL], bool is_whole) {
        const int w0 = sl * 4 * WPL + lg * WPL;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint32_t *src = p.B[g] + (int64_t)gn[cb] * KW;
                if (is_whole) {
#pragma unroll
                    for (int q = 0; q < WPL / 4; ++q) {
                        const uint4 v = reinterpret_cast<const uint4 *>(src + w0)[q];
                        bw[cb][g][4 * q] = v.x; bw[cb][g][4 * q + 1] = v.y;
                        bw[cb][g][4 * q + 2] = v.z; bw[cb][g][4 * q + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < WPL; ++j) {
                        const uint32_t v = src[min(w0 + j, KW - 1)];
                        bw[cb][g][j] = w0 + j < KW ? v : 0u;
                    }
                }
            }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int64_t row = min(row0 + mb * 16 + lc, M - 1);
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const i32x4 *src = reinterpret_cast<const i32x4 *>(p.A[q] + row * K);
#pragma unroll
                for (int j = 0; j < WPL; ++j) a[mb][q][j] = src[is_whole ? w0 + j : min(w0 + j, KW - 1)];
            }
        }
    };
    auto mma_slice = [&](const uint32_t (&bw)[CB][NG][WPL], const i32x4 (&a)[MB][NA][WPL], int sl) {
#pragma unroll
        for (int j = 0; j < WPL; ++j) {
            const int32_t o = sl * 4 * WPL + lg * WPL + j < KW ? 0x01010101 : 0;
            const i32x4 ones = {o, o, o, o};
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const i32x4 b = decode_word(bw[cb][g][j]);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb][cb][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb][SHARED_A ? 0 : g][j], b,
                                                                               acc[mb][cb][g], 0, 0, 0);
                }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < NA; ++q)
                    accq[mb][q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb][q][j], ones, accq[mb][q], 0, 0, 0);
        }
    };
    if constexpr (SPW == 2) {
        // two slices per wave at most (whole rows): both slices' loads are issued
        // before the first MFMA, so the wave pays one memory round trip, not two;
        // a wave without a second slice loads the last one again and skips it
        uint32_t bw0[CB][NG][WPL], bw1[CB][NG][WPL];
        i32x4 a0[MB][NA][WPL], a1[MB][NA][WPL];
        load_slice(wave, bw0, a0, true);
        load_slice(min(wave + nw, nslices - 1), bw1, a1, true);
        mma_slice(bw0, a0, wave);
        if (wave + nw < nslices) mma_slice(bw1, a1, wave + nw);
    } else if (nslices <= nw) {
        if (wave < nslices) {  // one slice per wave
            uint32_t bw[CB][NG][WPL];
            i32x4 a[MB][NA][WPL];
            load_slice(wave, bw, a, whole);
            mma_slice(bw, a, wave);
        }
    } else if constexpr (MB > 2 || (EPT > 2 && CB * NG > 8) || (EPT == 2 && CB * NG >= 4)) {
        // no registers for a second set (with two outputs per thread and four
        // channel blocks a launch has fewer than 16 slices: one per wave, above;
        // three or four outputs per thread come with a 512-thread bound, whose
        // registers hold two sets for up to eight channel blocks)
        for (int sl = wave; sl < nslices; sl += nw) {
            uint32_t bw[CB][NG][WPL];
            i32x4 a[MB][NA][WPL];
            load_slice(sl, bw, a, whole);
            mma_slice(bw, a, sl);
        }
    } else if (wave < nslices) {
        // more slices: two register sets, the next slice's loads in flight
        // during the current one's MFMAs (the last loads repeat the final
        // slice and go unused)
        uint32_t bw0[CB][NG][WPL], bw1[CB][NG][WPL];
        i32x4 a0[MB][NA][WPL], a1[MB][NA][WPL];
        const int last = nslices - 1;
        int sl = wave;
        load_slice(sl, bw0, a0, whole);
        while (true) {
            load_slice(min(sl + nw, last), bw1, a1, whole);
            mma_slice(bw0, a0, sl);
            sl += nw;
            if (sl >= nslices) break;
            load_slice(min(sl + nw, last), bw0, a0, whole);
            mma_slice(bw1, a1, sl);
            sl += nw;
            if (sl >= nslices) break;
        }
    }
    // each wave's partial sums of t*q into its own LDS slot; summed below in wave order
    int32_t *mine = part + wave * PART;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    mine[((mb * CB + cb) * NG + g) * 256 + (4 * lg + i) * 16 + lc] =
                        acc[mb][cb][g][i] - accq[mb][SHARED_A ? 0 : g][i];
    __syncthreads();
    float sw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sw[g] = __fdiv_rn(1.0f, fmaxf(mu_v[g], 1e-5f));
    const int active = nw < nslices ? nw : nslices;  // waves that ran a slice
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int idx = tid + e * blockDim.x;
        const int mb = idx / (256 * CB), cb = (idx >> 8) % CB, r = (idx >> 4) & 15, c = idx & 15;
        const int64_t m = row0 + mb * 16 + r;
        const int ch = n0 + cb * 16 + c;
        if (idx < MB * CB * 256 && m < M && ch < p.nc) {
            int32_t v[NG];
            float dq[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int o = ((mb * CB + cb) * NG + g) * 256 + r * 16 + c;
                int32_t sum = 0;
                for (int w = 0; w < active; ++w) sum += part[w * PART + o];
                v[g] = sum;
                dq[g] = __builtin_amdgcn_rcpf(sc_e[e][g] * sw[g]);
            }
            epilogue_vals<EPI, NG, true>(p, m, ch, v, dq, pre[e]);
        }
    }
}

// ----------------------------------------------------------------------------
// Decode at one row: the contraction quantises its own input row
// ----------------------------------------------------------------------------
// What a self-quantising contraction reads as its input rows.
enum RowIn : int {
    ROW_X = 0,           // x as it is (no gain)
    ROW_GNORM = 1,       // the gated g_norm of (h, g) (one row)
    ROW_GAIN = 2,        // x with its FusedBitLinear gain (one row)
    ROW_GNORM_GAIN = 3,  // the gated g_norm, then o_proj's gain (one row)
};

// quant_code's int8 code clamp(rint(y s), -128, 127) in the low byte of the
// result, in two VALU operations fewer: clamped first (the clamp commutes with
// rint, its bounds being integers), then 1.5 * 2^23 is added, which rounds to
// the nearest integer with ties to even (the sum lies in [2^23, 2^24), where
// binary32 values are 1 apart) and leaves the bit pattern 0x4B400000 + q
// (pack_codes4 keeps the low byte). A NaN product clamps to -128 in both.
__device__ __forceinline__ uint32_t code_bits(float y, float s) {
    const float p = fminf(fmaxf(__fmul_rn(y, s), -128.0f), 127.0f);
    return __float_as_uint(__fadd_rn(p, 12582912.0f));
}

// A 4-element chunk at element c4 of the input row that starts at element
// row_off: x (and its FusedBitLinear gain into o); or h with g and the g_norm
// gain (1 where there is none: multiplying by 1 is exact), and o_proj's gain
// into o.
template <int IN, typename XT>
__device__ __forceinline__ void load_row_chunk(const RowSrc &src, int64_t row_off, int64_t c4, float (&x)[4],
                                               float (&g)[4], float (&w)[4], float (&o)[4]) {
    if constexpr (IN == ROW_GAIN || IN == ROW_GNORM_GAIN) {
        const float4 v = *reinterpret_cast<const float4 *>(src.gain + c4);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    if constexpr (IN == ROW_GNORM || IN == ROW_GNORM_GAIN) {
        const float4 h = load_act4(static_cast<const float *>(src.x) + row_off, c4);
        const float4 gg = load_act4(static_cast<const XT *>(src.g) + row_off, c4);
        const float4 ww = src.gnw ? *reinterpret_cast<const float4 *>(src.gnw + c4) : make_float4(1.f, 1.f, 1.f, 1.f);
        x[0] = h.x; x[1] = h.y; x[2] = h.z; x[3] = h.w;
        g[0] = gg.x; g[1] = gg.y; g[2] = gg.z; g[3] = gg.w;
        w[0] = ww.x; w[1] = ww.y; w[2] = ww.z; w[3] = ww.w;
    } else {
        const float4 v = load_act4(static_cast<const XT *>(src.x) + row_off, c4);
        x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
}

// y = ((h r_h) w) silu(g), rounded after each product as the g_norm quantiser does.
__device__ __forceinline__ void gated_norm4(float (&x)[4], const float (&g)[4], const float (&w)[4], float rh) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __fmul_rn(__fmul_rn(__fmul_rn(x[e], rh), w[e]), silu_fast(g[e]));
}

// With a single row, quantising it costs each workgroup a few VALU operations
// per thread, less than the launch of a separate quantiser. Every thread loads
// its 4-element chunks of the raw row first, then the weights of its wave's
// slices (SPW per wave), so the weights are in flight while the row is reduced:
// sum x^2 (binary64) and max |x| meet in LDS in one round (no gain: max |x r| =
// (max |x|) r exactly), the codes go to LDS, and each wave reads its
// activation fragments from there (all 16 fragment rows read the one row).
// The MFMAs, the all-ones sum of codes and the epilogue are those of the GEMV;
// only row 0 is stored. Same codes and scale as the separate quantiser (its
// operations, binary64 sum in another order). IN = ROW_GNORM: the row is the
// gated g_norm of (h, g): a first round forms sum h^2 and r_h, then
// y = ((h r_h) w) silu(g) is quantised as x is, in the g_norm quantiser's
// order of roundings. IN = ROW_GAIN: a first round forms sum x^2 and r, then
// y = (x r) w, and the last round takes max |y| alone (the gain breaks
// max |y| = (max |x|) r), as the quantiser does with a gain.
// IN = ROW_GNORM_GAIN: both, in that order (three rounds).
template <int NG, int EPI, typename XT, typename RT, int CB, int SPW, int IN>
__global__ __launch_bounds__(1024) void tgemv_row_kernel(const ContractArgs p, const RowSrc src, float eps,
                                                         const int nslices) {
    constexpr int WPL = 4, MAXCH = 4;
    constexpr int PART = CB * NG * 16;  // row 0 of each wave's partial sums
    extern __shared__ int32_t part[];   // [waves][PART], then the row's codes
    __shared__ double red_d[16];
    __shared__ double red_h[16];
    __shared__ float red_f[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int lc = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16 * CB;
    const int K = p.k, KW = K >> 4, nch = K >> 2, T = blockDim.x;
    uint32_t *codes = reinterpret_cast<uint32_t *>(part + nw * PART);
    // 1. the row (straight-line, clamped chunk indices)
    float xv[MAXCH][4];
    constexpr bool GN = IN == ROW_GNORM || IN == ROW_GNORM_GAIN, GAIN = IN == ROW_GAIN || IN == ROW_GNORM_GAIN;
    [[maybe_unused]] float gv[GN ? MAXCH : 1][4], wv[GN ? MAXCH : 1][4], ov[GAIN ? MAXCH : 1][4];
#pragma unroll
    for (int j = 0; j < MAXCH; ++j)
        load_row_chunk<IN, XT>(src, 0, 4 * (int64_t)min(tid + j * T, nch - 1), xv[j], gv[GN ? j : 0],
                               wv[GN ? j : 0], ov[GAIN ? j : 0]);
    // 2. the weights of the wave's slices (a wave without a second slice loads the last again)
    int gn[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) gn[cb] = min(n0 + cb * 16 + lc, p.nc - 1);
    const bool whole = (KW % (4 * WPL)) == 0;
    uint32_t bw[SPW][CB][NG][WPL];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        const int sl = min(wave + sp * nw, nslices - 1);
        const int w0 = sl * 4 * WPL + lg * WPL;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint32_t *src = p.B[g] + (int64_t)gn[cb] * KW;
                if (whole) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(src + w0);
                    bw[sp][cb][g][0] = v.x; bw[sp][cb][g][1] = v.y; bw[sp][cb][g][2] = v.z; bw[sp][cb][g][3] = v.w;
                } else {
#pragma unroll
                    for (int j = 0; j < WPL; ++j) {
                        const uint32_t v = src[min(w0 + j, KW - 1)];
                        bw[sp][cb][g][j] = w0 + j < KW ? v : 0u;
                    }
                }
            }
    }
    // epilogue operands of row 0 (threads < 16 CB)
    float mu_v[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) mu_v[g] = *p.mu[g];
    constexpr bool PRE = EPI == EPI_RESID || EPI == EPI_GATES_STEP;
    const int ec = n0 + (tid >> 4) * 16 + (tid & 15);
    float pre = 0.0f;
    if constexpr (PRE) {
        const RT *pre_src = static_cast<const RT *>(EPI == EPI_RESID ? p.res : p.out0);
        pre = load_act(pre_src, (int64_t)(ec < p.nc ? ec : p.nc - 1));
    }
    // rounds before the last: sum h^2 for the gated g_norm (red_h), sum x^2
    // before a gain (red_d); each round has its own slots, so no wave can
    // overwrite a slot another wave is still reading
    auto block_rms = [&](double *slots) {
        double sh = 0.0;
#pragma unroll
        for (int j = 0; j < MAXCH; ++j)
            if (tid + j * T < nch)
#pragma unroll
                for (int e = 0; e < 4; ++e) sh += (double)xv[j][e] * (double)xv[j][e];
        sh = wave_sum(sh);
        if (lane == 0) slots[wave] = sh;
        __syncthreads();
        sh = 0.0;
        for (int w = 0; w < nw; ++w) sh += slots[w];
        return rms_factor(sh, K, eps);
    };
    const bool probe0 = blockIdx.x == 0;  // workgroup 0 writes the optional stage outputs
    if constexpr (GN) {
        const float rh = block_rms(red_h);
#pragma unroll
        for (int j = 0; j < MAXCH; ++j) gated_norm4(xv[j], gv[j], wv[j], rh);
        if (probe0 && src.u_out) {
#pragma unroll
            for (int j = 0; j < MAXCH; ++j) {
                const int c = tid + j * T;
                if (c < nch) *reinterpret_cast<float4 *>(src.u_out + 4 * c) = make_float4(xv[j][0], xv[j][1], xv[j][2], xv[j][3]);
            }
        }
    }
    if constexpr (GAIN) {
        const float r1 = block_rms(red_d);
#pragma unroll
        for (int j = 0; j < MAXCH; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[j][e] = __fmul_rn(__fmul_rn(xv[j][e], r1), ov[j][e]);
    }
    // 3. sum x^2 and max |x| in one round (max |y| alone with a gain)
    double ss = 0.0;
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXCH; ++j)
        if (tid + j * T < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (!GAIN) ss += (double)xv[j][e] * (double)xv[j][e];
                mx = fmaxf(mx, fabsf(xv[j][e]));
            }
    if constexpr (!GAIN) ss = wave_sum(ss);
    mx = wave_max(mx);
    if (lane == 0) {
        if constexpr (!GAIN) red_d[wave] = ss;
        red_f[wave] = mx;
    }
    __syncthreads();
    ss = 0.0;
    mx = 0.0f;
    for (int w = 0; w < nw; ++w) {
        if constexpr (!GAIN) ss += red_d[w];
        mx = fmaxf(mx, red_f[w]);
    }
    // with a gain the row is already y = (x r) w: its codes take no further factor
    const float r = GAIN ? 1.0f : rms_factor(ss, K, eps);
    const float sc = quant_scale(GAIN ? mx : __fmul_rn(mx, r));
    auto qv = [&](float v) { return (int)code_bits(GAIN ? v : __fmul_rn(v, r), sc); };
    // 4. the codes to LDS (and, from workgroup 0, to the optional outputs)
    uint32_t *codes_g = probe0 ? reinterpret_cast<uint32_t *>(src.codes_out) : nullptr;
#pragma unroll
    for (int j = 0; j < MAXCH; ++j) {
        const int c = tid + j * T;
        if (c < nch) {
            const uint32_t v = pack_codes4(qv(xv[j][0]), qv(xv[j][1]), qv(xv[j][2]), qv(xv[j][3]));
            codes[c] = v;
            if (codes_g) codes_g[c] = v;
        }
    }
    if (probe0 && src.scale_out && tid == 0) *src.scale_out = sc;
    __syncthreads();
    // 5. the contraction
    i32x4 acc[CB][NG], accq = i32x4{};
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[cb][g] = i32x4{};
    const i32x4 *cw = reinterpret_cast<const i32x4 *>(codes);
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        const int sl = wave + sp * nw;
        if (sl < nslices) {
#pragma unroll
            for (int j = 0; j < WPL; ++j) {
                const int w = sl * 4 * WPL + lg * WPL + j;
                const i32x4 a = cw[min(w, KW - 1)];
                const int32_t o = w < KW ? 0x01010101 : 0;
                const i32x4 ones = {o, o, o, o};
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        acc[cb][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, decode_word(bw[sp][cb][g][j]), acc[cb][g],
                                                                           0, 0, 0);
                accq = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, ones, accq, 0, 0, 0);
            }
        }
    }
    // row 0 of the result lives in register 0 of lanes 0..15
    if (lg == 0) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int g = 0; g < NG; ++g) part[wave * PART + (cb * NG + g) * 16 + lc] = acc[cb][g][0] - accq[0];
    }
    __syncthreads();
    // 6. the epilogue of row 0: 16 CB outputs
    const int active = nw < nslices ? nw : nslices;
    if (tid < 16 * CB && ec < p.nc) {
        const int cb = tid >> 4, c = tid & 15;
        int32_t v[NG];
        float dq[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            int32_t sum = 0;
            for (int w = 0; w < active; ++w) sum += part[w * PART + (cb * NG + g) * 16 + c];
            v[g] = sum;
            dq[g] = __builtin_amdgcn_rcpf(sc * __fdiv_rn(1.0f, fmaxf(mu_v[g], 1e-5f)));
        }
        epilogue_vals<EPI, NG, true>(p, 0, ec, v, dq, pre);
    }
}

// ----------------------------------------------------------------------------
// Host dispatch
// ----------------------------------------------------------------------------
static const char *epi_name(EpiKind e) {
    switch (e) {
        case EPI_LINEAR: return "linear";
        case EPI_RESID: return "resid";
        case EPI_GATES: return "gates";
        case EPI_GATES_STEP: return "gates_step";
        case EPI_GLU: return "glu";
    }
    return "?";
}

template <int NG, int JN, bool SH, int EPI>
static void run_gemm(const ContractArgs &a, hipStream_t st) {
    using S = TileShape<NG, JN, SH>;
    const int64_t tiles_m = (a.m + kBM - 1) / kBM;
    const int tiles_n = (a.nc + S::BNC - 1) / S::BNC;
    launch_k(tgemm_kernel<NG, JN, SH, EPI>, (unsigned)(tiles_m * tiles_n), 256, 0, st, a, tiles_n);
}

template <int NG, bool SH, int EPI, int WPL, typename RT, int CB>
static void run_gemv_cb(const ContractArgs &a, hipStream_t st) {
    const int kw = a.k >> 4;
    const int nslices = (kw + 4 * WPL - 1) / (4 * WPL);
    constexpr int MB = 1;  // row blocks per workgroup
    // per-wave partial sums take MB*CB*NG KB of LDS per wave: at most 64 KB in all
    constexpr int kThreadWaves = gemv_max_threads<NG, SH>() / 64;
    constexpr int kMaxWaves = 64 / (MB * CB * NG) < kThreadWaves ? 64 / (MB * CB * NG) : kThreadWaves;
    static_assert(kMaxWaves >= MB * CB, "the epilogue needs a wave per row and channel block");
    int waves = nslices < kMaxWaves ? nslices : kMaxWaves;
    if (waves < MB * CB) waves = MB * CB;  // the epilogue covers MB*CB*256 outputs with at most 4 per thread
    // x: channel blocks; y: groups of MB row blocks (rows past m are clamped, never stored)
    const dim3 grid((unsigned)((a.nc + 16 * CB - 1) / (16 * CB)), (unsigned)((a.m + 16 * MB - 1) / (16 * MB)));
    const size_t lds = (size_t)waves * MB * CB * NG * 256 * sizeof(int32_t);
    const int ept = (MB * CB * 256 + waves * 64 - 1) / (waves * 64);
    // up to two whole slices per wave: both loaded before the MFMAs (one round trip)
    const bool two = MB * CB <= 2 && nslices > waves && nslices <= 2 * waves && kw % (4 * WPL) == 0;
    if constexpr (MB * CB <= 2) {
        if (two) {
            switch (ept) {
                case 1: launch_k(tgemv_kernel<NG, SH, EPI, WPL, RT, 1, 2, CB>, grid, waves * 64, lds, st, a, nslices); break;
                default: launch_k(tgemv_kernel<NG, SH, EPI, WPL, RT, 2, 2, CB>, grid, waves * 64, lds, st, a, nslices); break;
            }
            return;
        }
    }
    switch (ept) {
        case 1: launch_k(tgemv_kernel<NG, SH, EPI, WPL, RT, 1, 1, CB>, grid, waves * 64, lds, st, a, nslices); break;
        case 2: launch_k(tgemv_kernel<NG, SH, EPI, WPL, RT, 2, 1, CB>, grid, waves * 64, lds, st, a, nslices); break;
        case 3: launch_k(tgemv_kernel<NG, SH, EPI, WPL, RT, 3, 1, CB>, grid, waves * 64, lds, st, a, nslices); break;
        default: launch_k(tgemv_kernel<NG, SH, EPI, WPL, RT, 4, 1, CB>, grid, waves * 64, lds, st, a, nslices); break;
    }
}

template <int NG, int JN, int EPI>
static void run_gemm_dma(const ContractArgs &a, hipStream_t st) {
    using S = DmaShape<NG, JN>;
    static_assert(S::LOADS == 5 || S::LOADS == 6 || S::LOADS == 7, "vmcnt_wait covers 5..7 loads per step");
    const int64_t tiles_m = (a.m + kBM - 1) / kBM;
    const int tiles_n = (a.nc + S::BNC - 1) / S::BNC;
    launch_k(tgemm_dma_kernel<NG, JN, EPI>, (unsigned)(tiles_m * tiles_n), 256, 0, st, a, tiles_n);
}

// Channel blocks per workgroup for one row block: the most (1, 2, 4, or 8 for a
// single group, with ng * cb <= 4 otherwise) that still leaves kGemvMinGroups
// workgroups. Every workgroup reads the codes of all its rows over the whole
// K, as many bytes as a 64-channel block of packed weights, so wider
// workgroups cut that traffic; too few of them leave the latency-bound small
// shapes with too few CUs pulling weights (measured on MI355X: 2048 outputs
// keep 16-channel workgroups, 5632 x 2 take two blocks, 11264 x 1 four; a
// 32768 x 32768 weight streams at 4.4 TB/s with eight blocks against 3.75 with
// four, and at 5.4 with the codes traffic removed in a timing-only copy).
constexpr int kGemvMinGroups = 160;
static int gemv_channel_blocks(int nc, int ng, int k, int row_blocks) {
    int cb = 1;
    if (k < 1024) return cb;  // fewer than 4 slices: too few waves for the wider epilogue
    for (int c = 2; c <= 8; c *= 2)
        if (ng * c <= (ng == 1 ? 8 : 4) && (nc + 16 * c - 1) / (16 * c) * row_blocks >= kGemvMinGroups) cb = c;
    return cb;
}

template <int NG, bool SH, int EPI, typename RT>
static void run_gemv_t(const ContractArgs &a, hipStream_t st) {
    // 4 words (64 k) per lane per slice: measured fastest at the 1.3B decode shapes
    // one workgroup per 16-row block and CB channel blocks: the channel blocks
    // share each activation fragment (a workgroup reads its rows' codes once,
    // 4x the bytes of a 16-channel block of weights)
    switch (gemv_channel_blocks(a.nc, NG, a.k, (int)((a.m + 15) / 16))) {
        case 8:
            if constexpr (NG == 1) { run_gemv_cb<NG, SH, EPI, 4, RT, 8>(a, st); break; }
            [[fallthrough]];
        case 4:
            if constexpr (NG == 1) { run_gemv_cb<NG, SH, EPI, 4, RT, 4>(a, st); break; }
            [[fallthrough]];
        case 2:
            if constexpr (NG <= 2) { run_gemv_cb<NG, SH, EPI, 4, RT, 2>(a, st); break; }
            [[fallthrough]];
        default: run_gemv_cb<NG, SH, EPI, 4, RT, 1>(a, st); break;
    }
}

template <int NG, bool SH, int EPI>
static void run_gemv(const ContractArgs &a, hipStream_t st) {
    // the residual comes in the activation type; the recurrent state is fp32
    if constexpr (EPI == EPI_RESID) {
        if (a.res_type == ACT_BF16) {
            run_gemv_t<NG, SH, EPI, uint16_t>(a, st);
            return;
        }
    }
    run_gemv_t<NG, SH, EPI, float>(a, st);
}

// Decode at a few rows: the same, with a wave per input row (RPW rows per wave
// at most): the row's sums are wave reductions, its codes go to LDS at a
// padded row stride (K + 16 bytes: the 16 fragment rows fall in different
// banks) with its scale, and the epilogue is the GEMV's over the 16-row block.
// IN = ROW_GAIN: each row with its gain (sum x^2, then max |(x r) w| alone).
template <int NG, int EPI, typename XT, typename RT, int CB, int SPW, int CPL, int RPW, int IN, bool FULL>
__global__ __launch_bounds__(1024) void tgemv_rows_kernel(const ContractArgs p, const RowSrc src, float eps,
                                                          const int nslices) {
    constexpr int WPL = 4;
    constexpr int PART = CB * NG * 256;
    extern __shared__ int32_t part[];  // [waves][PART], then codes [16][K + 16], then scales [16]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int lc = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16 * CB;
    const int K = p.k, KW = K >> 4, nch = K >> 2, stride = K + 16;
    // a launch may give the rows to two workgroups per channel block (gridDim.y = 2,
    // 8 rows each): this workgroup's rows are row0 .. row0 + M - 1
    const int rows_per = 16 / (int)gridDim.y;
    const int row0 = (int)blockIdx.y * rows_per;
    const int M = min((int)p.m - row0, rows_per);
    int8_t *codes = reinterpret_cast<int8_t *>(part + nw * PART);
    float *srow = reinterpret_cast<float *>(codes + 16 * stride);
    // 1. this wave's rows (straight-line, clamped)
    static_assert(IN == ROW_X || IN == ROW_GAIN, "several rows: x, with or without its gain");
    constexpr bool GAIN = IN == ROW_GAIN;
    float xv[RPW][CPL][4], unused[4];
    [[maybe_unused]] float ov[GAIN ? CPL : 1][4];  // the gain (the same for every row)
    // FULL: rows of exactly 64 CPL chunks (k = 2048 at CPL = 8), so no chunk index
    // needs clamping nor any chunk a bounds test; chosen at launch, since a branch
    // here makes the compiler wait for the row loads before the weight loads go out
    // (measured 33.1 -> 37.8 us per 1.3B layer at 16 rows; 31.95 as a template)
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rr = min(wave + i * nw, M - 1);
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            load_row_chunk<IN, XT>(src, (int64_t)(row0 + rr) * K, 4 * (int64_t)(FULL ? lane + 64 * j : min(lane + 64 * j, nch - 1)),
                                   xv[i][j], unused, unused, GAIN ? ov[j] : unused);
    }
    // 2. the weights of the wave's slices
    int gn[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) gn[cb] = min(n0 + cb * 16 + lc, p.nc - 1);
    const bool whole = (KW % (4 * WPL)) == 0;
    uint32_t bw[SPW][CB][NG][WPL];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        const int sl = min(wave + sp * nw, nslices - 1);
        const int w0 = sl * 4 * WPL + lg * WPL;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint32_t *src = p.B[g] + (int64_t)gn[cb] * KW;
                if (whole) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(src + w0);
                    bw[sp][cb][g][0] = v.x; bw[sp][cb][g][1] = v.y; bw[sp][cb][g][2] = v.z; bw[sp][cb][g][3] = v.w;
                } else {
#pragma unroll
                    for (int j = 0; j < WPL; ++j) {
                        const uint32_t v = src[min(w0 + j, KW - 1)];
                        bw[sp][cb][g][j] = w0 + j < KW ? v : 0u;
                    }
                }
            }
    }
    // epilogue operands (output idx: row (idx / 16) % 16, channel block idx / 256, channel idx % 16)
    constexpr int EPT = 4;
    constexpr bool PRE = EPI == EPI_RESID || EPI == EPI_GATES_STEP;
    float pre[EPT];
    const RT *pre_src = static_cast<const RT *>(EPI == EPI_RESID ? p.res : p.out0);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int idx = tid + e * (int)blockDim.x;
        const int m = min((idx >> 4) & 15, M - 1);
        const int c = n0 + ((idx >> 8) % CB) * 16 + (idx & 15);
        pre[e] = PRE ? load_act(pre_src, (int64_t)(row0 + m) * p.nc + (c < p.nc ? c : p.nc - 1)) : 0.0f;
    }
    float mu_v[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) mu_v[g] = *p.mu[g];
    // 3. each row: sum x^2 and max |x| (wave reductions), scale, codes to LDS
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = wave + i * nw;
        if (r < M) {
            double ss = 0.0;
            float mx = 0.0f;
#pragma unroll
            for (int j = 0; j < CPL; ++j)
                if (FULL || lane + 64 * j < nch)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ss += (double)xv[i][j][e] * (double)xv[i][j][e];
                        mx = fmaxf(mx, fabsf(xv[i][j][e]));
                    }
            ss = wave_sum(ss);
            const float rr = rms_factor(ss, K, eps);
            if constexpr (GAIN) {  // y = (x r) w: its max |y| alone decides the scale
                mx = 0.0f;
#pragma unroll
                for (int j = 0; j < CPL; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xv[i][j][e] = __fmul_rn(__fmul_rn(xv[i][j][e], rr), ov[j][e]);
                        if (FULL || lane + 64 * j < nch) mx = fmaxf(mx, fabsf(xv[i][j][e]));
                    }
            }
            mx = wave_max(mx);
            const float sc = quant_scale(GAIN ? mx : __fmul_rn(mx, rr));
            auto qv = [&](float v) { return (int)code_bits(GAIN ? v : __fmul_rn(v, rr), sc); };
            uint32_t *codes_g = blockIdx.x == 0 && src.codes_out
                                    ? reinterpret_cast<uint32_t *>(src.codes_out + (int64_t)(row0 + r) * K) : nullptr;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = lane + 64 * j;
                if (FULL || c < nch) {
                    const uint32_t v = pack_codes4(qv(xv[i][j][0]), qv(xv[i][j][1]), qv(xv[i][j][2]), qv(xv[i][j][3]));
                    *reinterpret_cast<uint32_t *>(codes + r * stride + 4 * c) = v;
                    if (codes_g) codes_g[c] = v;
                }
            }
            if (lane == 0) {
                srow[r] = sc;
                if (blockIdx.x == 0 && src.scale_out) src.scale_out[row0 + r] = sc;
            }
        }
    }
    __syncthreads();
    // 4. the contraction (fragment row lc reads input row min(lc, M - 1))
    i32x4 acc[CB][NG], accq = i32x4{};
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[cb][g] = i32x4{};
    const int8_t *arow = codes + min(lc, M - 1) * stride;
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        const int sl = wave + sp * nw;
        if (sl < nslices) {
#pragma unroll
            for (int j = 0; j < WPL; ++j) {
                const int w = sl * 4 * WPL + lg * WPL + j;
                const i32x4 a = *reinterpret_cast<const i32x4 *>(arow + 16 * min(w, KW - 1));
                const int32_t o = w < KW ? 0x01010101 : 0;
                const i32x4 ones = {o, o, o, o};
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        acc[cb][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, decode_word(bw[sp][cb][g][j]), acc[cb][g],
                                                                           0, 0, 0);
                accq = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, ones, accq, 0, 0, 0);
            }
        }
    }
    int32_t *mine = part + wave * PART;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) mine[(cb * NG + g) * 256 + (4 * lg + i) * 16 + lc] = acc[cb][g][i] - accq[i];
    __syncthreads();
    // 5. the epilogue of the 16-row block
    float sw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sw[g] = __fdiv_rn(1.0f, fmaxf(mu_v[g], 1e-5f));
    const int active = nw < nslices ? nw : nslices;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int idx = tid + e * (int)blockDim.x;
        const int cb = (idx >> 8) % CB, r = (idx >> 4) & 15, c = idx & 15;
        const int ch = n0 + cb * 16 + c;
        if (idx < CB * 256 && r < M && ch < p.nc) {
            int32_t v[NG];
            float dq[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                int32_t sum = 0;
                for (int w = 0; w < active; ++w) sum += part[w * PART + (cb * NG + g) * 256 + r * 16 + c];
                v[g] = sum;
                dq[g] = __builtin_amdgcn_rcpf(srow[r] * sw[g]);
            }
            epilogue_vals<EPI, NG, true>(p, row0 + r, ch, v, dq, pre[e]);
        }
    }
}

// The multi-row kernels take more dynamic LDS than the default 64 KB. The
// limit belongs to the kernel on each device: it is raised on a device before
// the kernel's first launch there, and a failure is returned, not launched.
template <auto KERNEL>
static hipError_t raise_lds_limit() {
    constexpr int kDevices = 64;  // devices past this raise it on every launch
    static std::atomic<bool> done[kDevices];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < kDevices && done[dev].load(std::memory_order_acquire)) return hipSuccess;
    std::lock_guard<std::mutex> lock(mu);
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(KERNEL), hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
    if (e == hipSuccess && dev < kDevices) done[dev].store(true, std::memory_order_release);
    return e;
}

// Compute units of the current device (cached per device).
static int contract_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <auto KERNEL>
static hipError_t launch_rows(const ContractArgs &a, const RowSrc &src, float eps, int nslices, dim3 grid, int waves,
                              size_t lds, hipStream_t st) {
    const hipError_t e = raise_lds_limit<KERNEL>();
    if (e != hipSuccess) return e;
    launch_k(KERNEL, grid, waves * 64, lds, st, a, src, eps, nslices);
    return hipSuccess;
}

template <int NG, int EPI, typename XT, typename RT, int CB, int IN>
static hipError_t run_row_cb(const ContractArgs &a, const RowSrc &src, float eps, hipStream_t st) {
    const int kw = a.k >> 4;
    const int nslices = (kw + 15) / 16;
    dim3 grid((unsigned)((a.nc + 16 * CB - 1) / (16 * CB)));
    if (a.m == 1) {
        const int waves = nslices < 16 ? nslices : 16;
        const size_t lds = (size_t)waves * CB * NG * 16 * sizeof(int32_t) + (size_t)a.k;
        if (nslices <= waves)
            launch_k(tgemv_row_kernel<NG, EPI, XT, RT, CB, 1, IN>, grid, waves * 64, lds, st, a, src, eps, nslices);
        else
            launch_k(tgemv_row_kernel<NG, EPI, XT, RT, CB, 2, IN>, grid, waves * 64, lds, st, a, src, eps, nslices);
        return hipSuccess;
    }
    // 2 to 16 rows of at most 2048, with or without a gain: a wave per row (8
    // chunks of 4 per lane); the gated g_norm runs at one row only
    if constexpr (IN == ROW_X || IN == ROW_GAIN) {
        // more than 8 rows and channel blocks for at most half the CUs: two
        // workgroups per channel block, 8 rows each, so that each CU quantises
        // half the rows (every workgroup quantises all of its rows, and that
        // vector work, not the weights, bounds these kernels; measured on the
        // 1.3B i/f/g at 16 rows: 31.8 -> 30.5 us per layer; gate_proj, whose
        // 352 halves would double up on CUs, was slower split: 31.2)
        const unsigned split = a.m > 8 && 2 * grid.x <= (unsigned)contract_cu_count() ? 2 : 1;
        const int m = (int)(split == 2 ? 8 : a.m);
        int waves = nslices < 16 ? nslices : 16;
        if (waves < m) waves = m;
        grid.y = split;
        const size_t lds =
            (size_t)waves * CB * NG * 256 * sizeof(int32_t) + (size_t)16 * (a.k + 16) + 16 * sizeof(float);
        // rows of at most 2048 make at most 8 slices: one per wave
        if (nslices > waves || a.k > 64 * 4 * 8) return hipErrorInvalidValue;
        if (a.k == 64 * 4 * 8)  // 64 lanes x 8 chunks of 4: every chunk of a row is a whole one
            return launch_rows<tgemv_rows_kernel<NG, EPI, XT, RT, CB, 1, 8, 1, IN, true>>(a, src, eps, nslices, grid,
                                                                                          waves, lds, st);
        return launch_rows<tgemv_rows_kernel<NG, EPI, XT, RT, CB, 1, 8, 1, IN, false>>(a, src, eps, nslices, grid, waves,
                                                                                       lds, st);
    }
    return hipErrorInvalidValue;  // the gated g_norm takes one row only
}

template <int NG, int EPI, typename XT, typename RT, int IN>
static hipError_t run_row_in(const ContractArgs &a, const RowSrc &src, float eps, hipStream_t st) {
    // four channel blocks take 10240 outputs or more: not with the gated g_norm (o_proj square,
    // at most 8192 wide) or with a gain, whose registers would not fit them
    constexpr bool CB4 = NG == 1 && IN == ROW_X;
    switch (gemv_channel_blocks(a.nc, NG, a.k, 1)) {
        case 8:  // the row kernels stop at four channel blocks
        case 4:
            if constexpr (CB4) return run_row_cb<NG, EPI, XT, RT, 4, IN>(a, src, eps, st);
            [[fallthrough]];
        case 2:
            if constexpr (NG <= 2) return run_row_cb<NG, EPI, XT, RT, 2, IN>(a, src, eps, st);
            [[fallthrough]];
        default: return run_row_cb<NG, EPI, XT, RT, 1, IN>(a, src, eps, st);
    }
}

// x with or without its gain
template <int NG, int EPI, typename XT, typename RT>
static hipError_t run_row(const ContractArgs &a, const RowSrc &src, float eps, hipStream_t st) {
    return src.gain ? run_row_in<NG, EPI, XT, RT, ROW_GAIN>(a, src, eps, st)
                    : run_row_in<NG, EPI, XT, RT, ROW_X>(a, src, eps, st);
}

// One row up to k = 8192; 2 to 16 rows up to k = 2048, one wave per row
// (12 with a gain: its second reduction per row made 16 rows slower than the
// separate quantiser, measured 35.4 against 34.5 us per 1.3B layer) (a wider row leaves the multi-row
// kernel too few registers, and its codes in LDS would limit the workgroups
// per CU).
bool contract_row_supported(int64_t m, int k, EpiKind epi, bool gain) {
    const bool kind = epi == EPI_GATES_STEP || epi == EPI_GLU || epi == EPI_RESID || epi == EPI_LINEAR;
    if (!kind || k % 16 || m < 1) return false;
    if (m == 1) return k <= 8192;
    return k <= 2048 && m <= (gain ? 12 : 16);
}

// The gated g_norm in o_proj (with or without o_proj's own gain): one row up
// to k = 8192 (at several rows, each
// workgroup reading h and g of every row and a second reduction per row cost
// more than the g_norm quantiser's launch: measured slower at 8 and 16 rows).
bool contract_row_gnorm_supported(int64_t m, int k) { return m == 1 && k % 16 == 0 && k <= 8192; }

hipError_t launch_contract_row(const ContractArgs &a, EpiKind epi, const void *xp, ActType xt, const float *gain,
                               float eps, int8_t *codes_out, float *scale_out, hipStream_t st, std::string *path) {
    if (!contract_row_supported(a.m, a.k, epi, gain != nullptr)) return hipErrorInvalidValue;
    const bool xb = xt == ACT_BF16, rb = a.res_type == ACT_BF16;
    const RowSrc x{xp, nullptr, nullptr, gain, codes_out, scale_out, nullptr};
    hipError_t e = hipSuccess;
    switch (epi) {
        case EPI_GATES_STEP:
            if (xb) e = run_row<3, EPI_GATES_STEP, uint16_t, float>(a, x, eps, st);
            else e = run_row<3, EPI_GATES_STEP, float, float>(a, x, eps, st);
            break;
        case EPI_GLU:
            if (xb) e = run_row<2, EPI_GLU, uint16_t, float>(a, x, eps, st);
            else e = run_row<2, EPI_GLU, float, float>(a, x, eps, st);
            break;
        case EPI_RESID:
            if (xb && rb) e = run_row<1, EPI_RESID, uint16_t, uint16_t>(a, x, eps, st);
            else if (xb) e = run_row<1, EPI_RESID, uint16_t, float>(a, x, eps, st);
            else if (rb) e = run_row<1, EPI_RESID, float, uint16_t>(a, x, eps, st);
            else e = run_row<1, EPI_RESID, float, float>(a, x, eps, st);
            break;
        case EPI_LINEAR:
            if (xb) e = run_row<1, EPI_LINEAR, uint16_t, float>(a, x, eps, st);
            else e = run_row<1, EPI_LINEAR, float, float>(a, x, eps, st);
            break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if (path) *path += std::string("tgemv_row<") + epi_name(epi) + ">;";
    return hipGetLastError();
}

template <int IN>
static hipError_t run_row_gnorm(const ContractArgs &a, const RowSrc &src, bool gb, float eps, hipStream_t st) {
    const bool rb = a.res_type == ACT_BF16;
    if (gb && rb) return run_row_in<1, EPI_RESID, uint16_t, uint16_t, IN>(a, src, eps, st);
    if (gb) return run_row_in<1, EPI_RESID, uint16_t, float, IN>(a, src, eps, st);
    if (rb) return run_row_in<1, EPI_RESID, float, uint16_t, IN>(a, src, eps, st);
    return run_row_in<1, EPI_RESID, float, float, IN>(a, src, eps, st);
}

hipError_t launch_contract_row_gnorm(const ContractArgs &a, const float *h, const void *g, ActType gt,
                                     const float *gnw, const float *ogain, float eps, int8_t *codes_out,
                                     float *scale_out, float *u_out, hipStream_t st, std::string *path) {
    if (!contract_row_gnorm_supported(a.m, a.k)) return hipErrorInvalidValue;
    const RowSrc src{h, g, gnw, ogain, codes_out, scale_out, u_out};
    const bool gb = gt == ACT_BF16;
    const hipError_t e = ogain ? run_row_gnorm<ROW_GNORM_GAIN>(a, src, gb, eps, st)
                               : run_row_gnorm<ROW_GNORM>(a, src, gb, eps, st);
    if (e != hipSuccess) return e;
    if (path) *path += "tgemv_row<resid,gnorm>;";
    return hipGetLastError();
}

static bool use_gemv(int64_t m) { return m <= 64; }
bool contract_sums_codes(int64_t m) { return use_gemv(m); }
// the LDS-DMA kernel needs whole 128-byte K steps and one activation tensor
static bool dma_ok(const ContractArgs &a, bool shared_a) { return shared_a && (a.k % kBK) == 0; }

std::string contract_variant(int64_t m, int k, EpiKind epi, bool shared_a) {
    const char *kind = use_gemv(m) ? "tgemv<" : (shared_a && k % kBK == 0) ? "tgemm_dma<" : "tgemm<";
    return std::string(kind) + epi_name(epi) + (shared_a ? "" : ",split_a") + ">";
}

hipError_t launch_contract(const ContractArgs &a, EpiKind epi, int ng, bool shared_a, hipStream_t st,
                           std::string *path) {
    if (a.m <= 0 || a.nc <= 0) return hipSuccess;
    const bool gemv = use_gemv(a.m);
    if (gemv) {
        switch (epi) {
            case EPI_LINEAR: run_gemv<1, true, EPI_LINEAR>(a, st); break;
            case EPI_RESID: run_gemv<1, true, EPI_RESID>(a, st); break;
            case EPI_GLU: run_gemv<2, true, EPI_GLU>(a, st); break;
            case EPI_GATES:
                if (shared_a) run_gemv<3, true, EPI_GATES>(a, st); else run_gemv<3, false, EPI_GATES>(a, st);
                break;
            case EPI_GATES_STEP:
                if (shared_a) run_gemv<3, true, EPI_GATES_STEP>(a, st); else run_gemv<3, false, EPI_GATES_STEP>(a, st);
                break;
        }
    } else if (dma_ok(a, shared_a)) {
        switch (epi) {
            case EPI_LINEAR: run_gemm_dma<1, 4, EPI_LINEAR>(a, st); break;
            case EPI_RESID: run_gemm_dma<1, 4, EPI_RESID>(a, st); break;
            case EPI_GLU: run_gemm_dma<2, 2, EPI_GLU>(a, st); break;
            case EPI_GATES: run_gemm_dma<3, 1, EPI_GATES>(a, st); break;
            case EPI_GATES_STEP: run_gemm_dma<3, 1, EPI_GATES_STEP>(a, st); break;
        }
    } else {
        switch (epi) {
            case EPI_LINEAR: run_gemm<1, 4, true, EPI_LINEAR>(a, st); break;
            case EPI_RESID: run_gemm<1, 4, true, EPI_RESID>(a, st); break;
            case EPI_GLU: run_gemm<2, 2, true, EPI_GLU>(a, st); break;
            case EPI_GATES:
                if (shared_a) run_gemm<3, 1, true, EPI_GATES>(a, st); else run_gemm<3, 1, false, EPI_GATES>(a, st);
                break;
            case EPI_GATES_STEP:
                if (shared_a) run_gemm<3, 1, true, EPI_GATES_STEP>(a, st); else run_gemm<3, 1, false, EPI_GATES_STEP>(a, st);
                break;
        }
    }
    (void)ng;
    if (path) *path += contract_variant(a.m, a.k, epi, shared_a) + ";";
    return hipGetLastError();
}

}  // namespace mmf
