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
// sum q a by-product of the activation quantiser.
//
// Prefill (m > 64): 128 x (NG * 64 * JN) output tiles (JN = 4, 2, 1 for one,
// two, three groups), four waves of 64 x (NG * 32 * JN), v_mfma_i32_32x32x32_i8, K staged 128 bytes at a time through
// double-buffered LDS (activation tile XOR-swizzled, packed weights padded to
// a 48-byte row stride: both conflict-free for 16-lane groups). Tiles are
// assigned XCD-major so that the workgroups of one XCD share activation rows
// in their L2.
// Decode (m <= 64): one workgroup per 16 output channels, four waves splitting
// K, v_mfma_i32_16x16x64_i8 per 16 rows of m, partial sums reduced in LDS.
//
// NG groups of output channels share an output tile so that the epilogue sees
// the matching channels of several projections in one lane: i/f/g for the
// token mixer's gates, the two halves of gate_proj for the SiLU-gated MLP
// ("MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，剩下什麼", section
// "HGRNBitBlock 的結構").
#include "device_common.hpp"
#include "launch.hpp"
#include "epilogue.hpp"

namespace mmf {

// ----------------------------------------------------------------------------
// Prefill: tiled int8 MFMA contraction
// ----------------------------------------------------------------------------
constexpr int kBM = 128;      // rows per tile
constexpr int kBK = 128;      // k (bytes of codes) per LDS stage
constexpr int kBStride = 48;  // bytes per packed-weight row in LDS (32 used)

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

template <int NG, int JN, bool SHARED_A, int EPI>
__global__ __launch_bounds__(256, 2) void tgemm_kernel(const ContractArgs p, const int tiles_n) {
    using S = TileShape<NG, JN, SHARED_A>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::STAGE];

    // XCD-major tile order: the idx-th workgroup dispatched to XCD x (blocks are
    // dealt round-robin over 8 XCDs) takes the idx-th tile of x's contiguous range.
    const int G = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, idx = bid >> 3;
    const int per = G >> 3, rem = G & 7;
    const int tile = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
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

    float sw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sw[g] = weight_sw(p.mu[g]);
    // per output row: the row's dequant factors once, then its JN column subtiles
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
            if (m >= M) continue;
            int32_t sq[NG];
            float dq[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                sq[g] = p.sumq[g][m];
                dq[g] = __builtin_amdgcn_rcpf(p.s[g][m] * sw[g]);
            }
#pragma unroll
            for (int j = 0; j < JN; ++j) {
                const int c = n0 + wn * (32 * JN) + j * 32 + lr;
                if (c < p.nc) {
                    int32_t v[NG];
#pragma unroll
                    for (int g = 0; g < NG; ++g) v[g] = acc[i][g][j][r] - sq[g];
                    epilogue_vals<EPI, NG>(p, m, c, v, dq);
                }
            }
        }
}

// ----------------------------------------------------------------------------
// Decode: m <= 64 rows, latency-bound weight streaming
// ----------------------------------------------------------------------------
// One workgroup per 16 output channels (x NG groups). K is cut into slices of
// 4*WPL words; one wave per slice (up to 16 waves; further slices loop). A lane
// (column lc, word group lg) owns WPL consecutive words of its column in the
// slice and issues every load of the slice -- weights as 16-byte runs,
// activation codes of its row block as 16-byte chunks -- before its first
// MFMA, so a GEMV costs about one memory round trip. Wave partial sums are
// combined with LDS integer atomics (exact, order-free).
template <int NG, int MB, bool SHARED_A, int EPI, int WPL>
__global__ __launch_bounds__(1024) void tgemv_kernel(const ContractArgs p, const int nslices) {
    constexpr int NA = SHARED_A ? 1 : NG;
    __shared__ int32_t red[MB * NG * 256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int lc = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int K = p.k, KW = K >> 4;
    const int64_t M = p.m;
    const int gn = n0 + lc;
    const bool bvec = (KW & 3) == 0;
    for (int i = tid; i < MB * NG * 256; i += blockDim.x) red[i] = 0;

    i32x4 acc[MB][NG];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[mb][g] = i32x4{};

    for (int sl = wave; sl < nslices; sl += nw) {
        const int w0 = sl * 4 * WPL + lg * WPL;
        uint32_t bw[NG][WPL];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint32_t *src = p.B[g] + (int64_t)gn * KW + w0;
            if (gn < p.nc && bvec && w0 + WPL <= KW) {
#pragma unroll
                for (int q = 0; q < WPL / 4; ++q) {
                    const uint4 v = reinterpret_cast<const uint4 *>(src)[q];
                    bw[g][4 * q] = v.x; bw[g][4 * q + 1] = v.y; bw[g][4 * q + 2] = v.z; bw[g][4 * q + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < WPL; ++j) bw[g][j] = (gn < p.nc && w0 + j < KW) ? src[j] : 0u;
            }
        }
        i32x4 a[MB][NA][WPL];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int64_t row = mb * 16 + lc;
#pragma unroll
            for (int q = 0; q < NA; ++q) {
                const i32x4 *src = reinterpret_cast<const i32x4 *>(p.A[q] + row * K) + w0;
#pragma unroll
                for (int j = 0; j < WPL; ++j) a[mb][q][j] = (row < M && w0 + j < KW) ? src[j] : i32x4{};
            }
        }
#pragma unroll
        for (int j = 0; j < WPL; ++j)
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const i32x4 b = decode_word(bw[g][j]);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mb][SHARED_A ? 0 : g][j], b, acc[mb][g], 0, 0, 0);
            }
    }
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) atomicAdd(&red[(mb * NG + g) * 256 + (4 * lg + i) * 16 + lc], acc[mb][g][i]);
    __syncthreads();
    float sw[3];
#pragma unroll
    for (int g = 0; g < 3; ++g) sw[g] = g < NG ? weight_sw(p.mu[g]) : 1.0f;
    for (int idx = tid; idx < MB * 256; idx += blockDim.x) {
        const int mb = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        const int64_t m = mb * 16 + r;
        if (m < M && n0 + c < p.nc) {
            int32_t raw[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) raw[g] = red[(mb * NG + g) * 256 + r * 16 + c];
            epilogue<EPI, NG>(p, sw, m, n0 + c, raw);
        }
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
    tgemm_kernel<NG, JN, SH, EPI><<<(unsigned)(tiles_m * tiles_n), 256, 0, st>>>(a, tiles_n);
}

template <int NG, int MB, bool SH, int EPI, int WPL>
static void run_gemv_mb(const ContractArgs &a, hipStream_t st) {
    const int kw = a.k >> 4;
    const int nslices = (kw + 4 * WPL - 1) / (4 * WPL);
    const int waves = nslices < 16 ? nslices : 16;
    tgemv_kernel<NG, MB, SH, EPI, WPL><<<(unsigned)((a.nc + 15) / 16), waves * 64, 0, st>>>(a, nslices);
}

template <int NG, bool SH, int EPI>
static void run_gemv(const ContractArgs &a, hipStream_t st) {
    constexpr int NA = SH ? 1 : NG;
    switch ((int)((a.m + 15) / 16)) {
        case 1: run_gemv_mb<NG, 1, SH, EPI, (NA <= 2 ? 8 : 4)>(a, st); break;
        case 2: run_gemv_mb<NG, 2, SH, EPI, (NA <= 1 ? 8 : 4)>(a, st); break;
        case 3: run_gemv_mb<NG, 3, SH, EPI, 4>(a, st); break;
        default: run_gemv_mb<NG, 4, SH, EPI, 4>(a, st); break;
    }
}

static bool use_gemv(int64_t m) { return m <= 64; }

std::string contract_variant(int64_t m, EpiKind epi, bool shared_a) {
    return std::string(use_gemv(m) ? "tgemv<" : "tgemm<") + epi_name(epi) + (shared_a ? "" : ",split_a") + ">";
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
    if (path) *path += contract_variant(a.m, epi, shared_a) + ";";
    return hipGetLastError();
}

}  // namespace mmf
