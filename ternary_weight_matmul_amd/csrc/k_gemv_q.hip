// Decode contraction with its input quantiser fused in (gfx950).
//
// A decode step of the HGRNBit block ("MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，
// 剩下什麼", section "HGRNBitBlock 的結構") quantises a few rows (one per sequence)
// before each of its four ternary contractions: x before i/f/g, the g_norm
// gate output before o_proj, x1 before gate_proj and z before down_proj
// ("MatMul-Free LLM 深度分析报告", list "可复用的模式与技巧": the RMSNorm and the
// activation quantiser belong to the same fused step). With b <= 16 rows the
// quantiser is tiny next to a kernel boundary (about 2 us in a HIP graph on
// MI355X), so each contraction kernel here quantises its b input rows itself:
// every workgroup redundantly, one wave per row, into LDS. A decode step is
// then four kernels instead of eight, and the codes never go through memory.
//
// Workgroup: 16 waves, CB blocks of 16 output channels. A unit of work is one
// (block, 256-k slice) pair; wave w takes units w and w + 16 and issues all
// its weight loads (16 bytes per lane per group and unit) first, then the
// epilogue operand, the gains and its input row, so that one memory round
// trip covers them all. The row quantisers (row_quant.hpp) reproduce the
// reduction order of the separate quantiser kernels, so both decode paths give
// the same bits. Partial sums of a block meet in LDS by integer atomic adds
// (exact, order-free).
#include "device_common.hpp"
#include "launch.hpp"
#include "epilogue.hpp"
#include "row_quant.hpp"

#include <mutex>
#include <type_traits>

namespace mmf {

constexpr int kQWaves = 16;
constexpr int kQThreads = kQWaves * 64;
constexpr int kQUnits = 2;  // units per wave at most

struct QuantContractArgs {
    ContractArgs c;      // contraction: B, mu, m (= b rows), nc, k, outputs, residual
    const void *x;       // QK_ROW: rows to quantise [b][k]; QK_GNORM: h [b][k] fp32
    const void *g;       // QK_GNORM: g [b][k]
    const float *gain;   // quantiser gain (RMSNorm weight) or null
    const float *gnw;    // QK_GNORM: g_norm weight or null
    float eps;
};

static size_t q_lds_bytes(int k, int ng, int cb, int qk) {
    return (size_t)16 * (k + 16) + (size_t)cb * ng * 1024 + (size_t)(qk == QK_GNORM ? 2 : 1) * k * 4 + 128;
}

template <int NG, int EPI, int QK, typename XT, typename GT, typename RT, int NC, int CB>
__global__ __launch_bounds__(kQThreads) void tgemv_q_kernel(const QuantContractArgs a) {
    const ContractArgs &p = a.c;
    extern __shared__ __attribute__((aligned(16))) char dyn[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lc = lane & 15, lg = lane >> 4;
    const int K = p.k, KW = K >> 4, nsl = K >> 8;
    const int b = (int)p.m;
    const int stride = K + 16;
    const int nunits = CB * nsl;
    const int n0 = blockIdx.x * (16 * CB);
    int8_t *codes = reinterpret_cast<int8_t *>(dyn);
    int32_t *accl = reinterpret_cast<int32_t *>(dyn + 16 * stride);
    float *gl = reinterpret_cast<float *>(dyn + 16 * stride + CB * NG * 1024);
    float *gl2 = gl + K;  // QK_GNORM: o_proj gain after the g_norm weight
    float *sl = gl + (QK == QK_GNORM ? 2 * K : K);
    int32_t *sql = reinterpret_cast<int32_t *>(sl + 16);

    // 1. weights of this wave's units
    uint4 wv[kQUnits][NG];
#pragma unroll
    for (int i = 0; i < kQUnits; ++i) {
        const int u = wave + kQWaves * i;
        if (u < nunits) {
            const int cb = u / nsl, s16 = (u - cb * nsl) * 16;
            const int ch = min(n0 + cb * 16 + lc, p.nc - 1);  // channels past nc load a valid row, never stored
#pragma unroll
            for (int g = 0; g < NG; ++g)
                wv[i][g] = *reinterpret_cast<const uint4 *>(p.B[g] + (int64_t)ch * KW + s16 + 4 * lg);
        }
    }
    float sw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sw[g] = weight_sw(p.mu[g]);

    // 2. the epilogue operand of this thread's output (residual or old state)
    constexpr bool PRE = EPI == EPI_RESID || EPI == EPI_GATES_STEP;
    const int ecb = tid >> 8, er = (tid >> 4) & 15, ec = tid & 15;
    const int ech = n0 + ecb * 16 + ec;
    float pre = 0.0f;
    if (PRE && tid < CB * 256) {
        const RT *src = static_cast<const RT *>(EPI == EPI_RESID ? p.res : p.out0);
        pre = load_act(src, (int64_t)min(er, b - 1) * p.nc + min(ech, p.nc - 1));
    }

    // 3. gains into LDS
    const int nch = K >> 2;
    if constexpr (QK == QK_GNORM) {
        for (int c = tid; c < nch; c += kQThreads) {
            if (a.gnw) reinterpret_cast<float4 *>(gl)[c] = reinterpret_cast<const float4 *>(a.gnw)[c];
            if (a.gain) reinterpret_cast<float4 *>(gl2)[c] = reinterpret_cast<const float4 *>(a.gain)[c];
        }
    } else {
        if (a.gain)
            for (int c = tid; c < nch; c += kQThreads)
                reinterpret_cast<float4 *>(gl)[c] = reinterpret_cast<const float4 *>(a.gain)[c];
    }

    // 4. this wave's input row (wave r quantises row r)
    const bool qwave = wave < b;
    typename RawRow<XT>::type raw[NC];
    typename RawRow<GT>::type graw[QK == QK_GNORM ? NC : 1];
    if (qwave) {
        wave_row_load<XT, NC, false>(static_cast<const XT *>(a.x) + (int64_t)wave * K, K, raw);
        if constexpr (QK == QK_GNORM)
            wave_row_load<GT, NC, false>(static_cast<const GT *>(a.g) + (int64_t)wave * K, K, graw);
    }
    for (int i = tid; i < CB * NG * 256; i += kQThreads) accl[i] = 0;
    __syncthreads();

    // 5. quantise into LDS
    if (qwave) {
        if constexpr (QK == QK_GNORM) {
            static_assert(std::is_same<XT, float>::value, "g_norm reads the fp32 state");
            wave_row_gnorm_quant<GT, NC>(raw, graw, K, a.gnw ? gl : nullptr, a.gain ? gl2 : nullptr, a.eps,
                                         codes + wave * stride, sl + wave, sql + wave);
        } else {
            wave_row_quant<XT, NC>(raw, K, a.gain ? gl : nullptr, a.eps, codes + wave * stride, sl + wave,
                                   sql + wave);
        }
    }
    __syncthreads();

    // 6. contraction of this wave's units; rows past b read row b - 1 (never stored)
    const int8_t *arow = codes + min(lc, b - 1) * stride;
#pragma unroll
    for (int i = 0; i < kQUnits; ++i) {
        const int u = wave + kQWaves * i;
        if (u < nunits) {
            const int cb = u / nsl, s16 = (u - cb * nsl) * 16;
            i32x4 acc[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[g] = i32x4{};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const i32x4 af = *reinterpret_cast<const i32x4 *>(arow + 16 * (s16 + 4 * lg + j));
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const uint32_t word = j == 0 ? wv[i][g].x : j == 1 ? wv[i][g].y : j == 2 ? wv[i][g].z : wv[i][g].w;
                    acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, decode_word(word), acc[g], 0, 0, 0);
                }
            }
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) atomicAdd(accl + (cb * NG + g) * 256 + (4 * lg + e) * 16 + lc, acc[g][e]);
        }
    }
    __syncthreads();

    // 7. epilogue: one thread per output (row er, channel ech)
    if (tid < CB * 256 && er < b && ech < p.nc) {
        int32_t v[NG];
        float dq[NG];
        const float srow = sl[er];
        const int32_t sqrow = sql[er];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            v[g] = accl[(ecb * NG + g) * 256 + er * 16 + ec] - sqrow;
            dq[g] = __builtin_amdgcn_rcpf(srow * sw[g]);
        }
        epilogue_vals<EPI, NG, true>(p, er, ech, v, dq, pre);
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static const char *q_epi_name(int epi) {
    switch (epi) {
        case EPI_GATES_STEP: return "gates_step";
        case EPI_RESID: return "resid";
        case EPI_GLU: return "glu";
    }
    return "?";
}

// chunk rounds per lane the row registers must hold, for the element types
static int q_pick_nc(int k, int qk, ActType xt, ActType gt) {
    const int need = k >> 8;
    int opts[3] = {8, 12, 28};
    int nopt = 3;
    if (qk == QK_GNORM) nopt = gt == ACT_F32 ? 1 : 2;  // fp32 h plus g rows
    else if (xt == ACT_F32) nopt = 2;
    for (int i = 0; i < nopt; ++i)
        if (need <= opts[i]) return opts[i];
    return 0;
}

static int q_pick_cb(int k) { return (k >> 8) >= 16 ? 1 : 2; }

bool quant_contract_supported(int64_t b, int nc, int k, EpiKind epi, int qk, ActType xt, ActType gt) {
    if (b < 1 || b > 16 || nc < 1 || k < 256 || k % 256) return false;
    if (epi != EPI_GATES_STEP && epi != EPI_RESID && epi != EPI_GLU) return false;
    if (q_pick_nc(k, qk, xt, gt) == 0) return false;
    const int cb = q_pick_cb(k);
    if (cb * (k >> 8) > kQUnits * kQWaves) return false;
    const int ng = epi == EPI_GATES_STEP ? 3 : epi == EPI_GLU ? 2 : 1;
    return q_lds_bytes(k, ng, cb, qk) <= (size_t)160 * 1024;
}

template <int NG, int EPI, int QK, typename XT, typename GT, typename RT, int NC, int CB>
static hipError_t run_q(const QuantContractArgs &a, hipStream_t st) {
    const void *fn = reinterpret_cast<const void *>(&tgemv_q_kernel<NG, EPI, QK, XT, GT, RT, NC, CB>);
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [&] { attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024); });
    if (attr != hipSuccess) return attr;
    const size_t lds = q_lds_bytes(a.c.k, NG, CB, QK);
    const unsigned grid = (unsigned)((a.c.nc + 16 * CB - 1) / (16 * CB));
    tgemv_q_kernel<NG, EPI, QK, XT, GT, RT, NC, CB><<<grid, kQThreads, lds, st>>>(a);
    return hipGetLastError();
}

template <int NG, int EPI, int QK, typename XT, typename GT, typename RT, int NC>
static hipError_t run_q_cb(const QuantContractArgs &a, int cb, hipStream_t st) {
    return cb == 1 ? run_q<NG, EPI, QK, XT, GT, RT, NC, 1>(a, st) : run_q<NG, EPI, QK, XT, GT, RT, NC, 2>(a, st);
}

template <int NG, int EPI, int QK, typename XT, typename GT, typename RT>
static hipError_t run_q_nc(const QuantContractArgs &a, int nc, int cb, hipStream_t st) {
    if constexpr (QK == QK_GNORM && std::is_same<GT, float>::value) {
        return run_q_cb<NG, EPI, QK, XT, GT, RT, 8>(a, cb, st);
    } else if constexpr (QK == QK_ROW && std::is_same<XT, float>::value) {
        return nc == 8 ? run_q_cb<NG, EPI, QK, XT, GT, RT, 8>(a, cb, st) : run_q_cb<NG, EPI, QK, XT, GT, RT, 12>(a, cb, st);
    } else if constexpr (QK == QK_GNORM) {
        return nc == 8 ? run_q_cb<NG, EPI, QK, XT, GT, RT, 8>(a, cb, st) : run_q_cb<NG, EPI, QK, XT, GT, RT, 12>(a, cb, st);
    } else {
        switch (nc) {
            case 8: return run_q_cb<NG, EPI, QK, XT, GT, RT, 8>(a, cb, st);
            case 12: return run_q_cb<NG, EPI, QK, XT, GT, RT, 12>(a, cb, st);
            default: return run_q_cb<NG, EPI, QK, XT, GT, RT, 28>(a, cb, st);
        }
    }
}

hipError_t launch_quant_contract(const ContractArgs &c, EpiKind epi, int qk, const void *x, ActType xt,
                                 const void *g, ActType gt, const float *gain, const float *gnw, float eps,
                                 hipStream_t st, std::string *path) {
    if (!quant_contract_supported(c.m, c.nc, c.k, epi, qk, xt, gt)) return hipErrorInvalidValue;
    QuantContractArgs a{};
    a.c = c;
    a.x = x; a.g = g; a.gain = gain; a.gnw = gnw; a.eps = eps;
    const int nc = q_pick_nc(c.k, qk, xt, gt), cb = q_pick_cb(c.k);
    if (path) *path += std::string("tgemv_q<") + (qk == QK_GNORM ? "gnorm_resid" : q_epi_name(epi)) + ">;";
    const bool xf = xt == ACT_F32, gf = gt == ACT_F32;
    switch (epi) {
        case EPI_GATES_STEP:  // quantised x, state in place
            if (qk != QK_ROW) return hipErrorInvalidValue;
            return xf ? run_q_nc<3, EPI_GATES_STEP, QK_ROW, float, float, float>(a, nc, cb, st)
                      : run_q_nc<3, EPI_GATES_STEP, QK_ROW, uint16_t, uint16_t, float>(a, nc, cb, st);
        case EPI_GLU:  // quantised x1 (fp32)
            if (qk != QK_ROW || !xf) return hipErrorInvalidValue;
            return run_q_nc<2, EPI_GLU, QK_ROW, float, float, float>(a, nc, cb, st);
        case EPI_RESID:
            if (qk == QK_GNORM) {  // g_norm gate of (h, g) + o_proj, residual x in g's type
                if (!xf || c.res_type != gt) return hipErrorInvalidValue;
                return gf ? run_q_nc<1, EPI_RESID, QK_GNORM, float, float, float>(a, nc, cb, st)
                          : run_q_nc<1, EPI_RESID, QK_GNORM, float, uint16_t, uint16_t>(a, nc, cb, st);
            }
            // quantised z + down_proj, residual x1 (fp32)
            if (c.res_type != ACT_F32) return hipErrorInvalidValue;
            return xf ? run_q_nc<1, EPI_RESID, QK_ROW, float, float, float>(a, nc, cb, st)
                      : run_q_nc<1, EPI_RESID, QK_ROW, uint16_t, uint16_t, float>(a, nc, cb, st);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace mmf
