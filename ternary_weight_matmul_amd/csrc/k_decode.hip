// Fused decode step kernels for up to 16 rows (gfx950).
//
// A decode step of the HGRNBit block ("MatMul-Free LM：把矩陣乘法從語言模型裡拿掉
// 之後，剩下什麼", section "HGRNBitBlock 的結構") is four ternary contractions, each
// fed by a row quantiser (RMSNorm + absmax int8, "MatMul-Free LLM 深度分析报告",
// list "可復用的模式與技巧" -- fused there as well). With at most 16 rows the
// work of a stage is tiny next to the weights it streams, so a stage is one
// kernel:
//   1. every lane issues the loads of its packed-weight words first
//      (weights do not depend on the input, so they are in flight during 2);
//   2. wave r of the 16-wave workgroup quantises input row r into LDS (each
//      workgroup redundantly: the rows sit in L2), lanes across K, the row kept
//      in registers, reductions within the wave; for the o_proj stage the row
//      is first turned into the g_norm RMSNorm-Swish output u;
//   3. v_mfma_i32_16x16x64_i8 with activation fragments from LDS;
//   4. wave partial sums meet in LDS (integer atomics), then the fused epilogue.
// One workgroup per 16*NCB output channels; its 64 lane groups split K.
#include "device_common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace mmf {

constexpr int kDecRows = 16;

// Per-row results of the in-kernel quantiser, in LDS.
struct RowStats {
    float *rs;  // absmax scale s
    int *rsq;   // sum of codes
};

// The quantiser input of one row: four consecutive elements at 4c.
template <int QIN>
__device__ __forceinline__ float4 qin_load4(const DecodeArgs &a, int r, int c) {
    const int64_t off = (int64_t)r * a.c.k + 4 * c;
    if constexpr (QIN == QIN_BF16) return load_act4(static_cast<const uint16_t *>(a.qin), off);
    else return *reinterpret_cast<const float4 *>(static_cast<const float *>(a.qin) + off);
}

__device__ __forceinline__ float4 gain4(const float *gain, int c) {
    return gain ? *reinterpret_cast<const float4 *>(gain + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f);
}

// y = (v * r) * gain, the quantiser's binary32 steps
__device__ __forceinline__ float4 scale4(float4 v, float r, const float *gain, int c) {
    float4 y = make_float4(__fmul_rn(v.x, r), __fmul_rn(v.y, r), __fmul_rn(v.z, r), __fmul_rn(v.w, r));
    if (gain) {
        const float4 g = gain4(gain, c);
        y = make_float4(__fmul_rn(y.x, g.x), __fmul_rn(y.y, g.y), __fmul_rn(y.z, g.z), __fmul_rn(y.w, g.w));
    }
    return y;
}

__device__ __forceinline__ float absmax4(float4 y) {
    return fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w)));
}

// codes of 4 elements -> LDS row (and the probe copy); returns their sum
__device__ __forceinline__ int emit4(float4 y, float sc, int8_t *lrow, int8_t *prow, int c) {
    const int q0 = quant_code(y.x, sc), q1 = quant_code(y.y, sc), q2 = quant_code(y.z, sc), q3 = quant_code(y.w, sc);
    const uint32_t word = pack_codes4(q0, q1, q2, q3);
    *reinterpret_cast<uint32_t *>(lrow + 4 * c) = word;
    if (prow) *reinterpret_cast<uint32_t *>(prow + 4 * c) = word;
    return q0 + q1 + q2 + q3;
}

// One wave quantises row r of the input into the LDS row `lrow`. NV > 0: the
// row is cached in registers (NV float4 chunks per lane, K <= 256*NV); NV == 0:
// three streaming passes over the row (sum of squares, absmax, codes).
template <int QIN, int NV>
__device__ void wave_quantize_row(const DecodeArgs &a, int r, int8_t *lrow, const RowStats &st) {
    const int lane = threadIdx.x & 63;
    const int K = a.c.k, nch = K >> 2;
    const bool probe = blockIdx.x == 0;
    int8_t *prow = (probe && a.codes_out) ? a.codes_out + (int64_t)r * K : nullptr;
    float r_in;
    float sc;
    int tot = 0;
    if constexpr (NV > 0) {
        float4 v[NV];
        double ss = 0.0;
        if constexpr (QIN == QIN_GNORM) {
            // u = ((h * rh) * g_norm_w) * SiLU(g): the prefill g_norm kernel's steps
            float4 gg[NV];
            const float *h = static_cast<const float *>(a.qin) + (int64_t)r * K;
            const float *g = a.g + (int64_t)r * K;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int c = min(lane + 64 * j, nch - 1);  // unconditional loads; tail masked below
                v[j] = *reinterpret_cast<const float4 *>(h + 4 * c);
                gg[j] = *reinterpret_cast<const float4 *>(g + 4 * c);
            }
#pragma unroll
            for (int j = 0; j < NV; ++j)
                if (lane + 64 * j >= nch) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int j = 0; j < NV; ++j)
                ss += (double)v[j].x * v[j].x + (double)v[j].y * v[j].y + (double)v[j].z * v[j].z + (double)v[j].w * v[j].w;
            const float rh = rms_factor(wave_sum(ss), K, a.eps);
            ss = 0.0;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int c = lane + 64 * j;
                float4 u = make_float4(v[j].x * rh, v[j].y * rh, v[j].z * rh, v[j].w * rh);
                if (a.gnw && c < nch) {
                    const float4 w = *reinterpret_cast<const float4 *>(a.gnw + 4 * c);
                    u = make_float4(u.x * w.x, u.y * w.y, u.z * w.z, u.w * w.w);
                }
                u = make_float4(u.x * silu_fast(gg[j].x), u.y * silu_fast(gg[j].y), u.z * silu_fast(gg[j].z),
                                u.w * silu_fast(gg[j].w));
                if (c >= nch) u = make_float4(0.f, 0.f, 0.f, 0.f);
                v[j] = u;
                ss += (double)u.x * u.x + (double)u.y * u.y + (double)u.z * u.z + (double)u.w * u.w;
                if (probe && a.u_out && c < nch) *reinterpret_cast<float4 *>(a.u_out + (int64_t)r * K + 4 * c) = u;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NV; ++j) v[j] = qin_load4<QIN>(a, r, min(lane + 64 * j, nch - 1));
#pragma unroll
            for (int j = 0; j < NV; ++j)
                if (lane + 64 * j >= nch) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int j = 0; j < NV; ++j)
                ss += (double)v[j].x * v[j].x + (double)v[j].y * v[j].y + (double)v[j].z * v[j].z + (double)v[j].w * v[j].w;
        }
        r_in = rms_factor(wave_sum(ss), K, a.eps);
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = lane + 64 * j;
            if (c < nch) {
                v[j] = scale4(v[j], r_in, a.gain, c);
                amax = fmaxf(amax, absmax4(v[j]));
            }
        }
        sc = quant_scale(wave_max(amax));
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = lane + 64 * j;
            if (c < nch) tot += emit4(v[j], sc, lrow, prow, c);
        }
    } else {
        static_assert(QIN != QIN_GNORM, "the g_norm stage keeps its row in registers");
        constexpr int B8 = 8;  // chunks per lane in flight per batch
        double ss = 0.0;
        for (int base = 0; base < nch; base += 64 * B8) {
            float4 v[B8];
#pragma unroll
            for (int j = 0; j < B8; ++j) v[j] = qin_load4<QIN>(a, r, min(base + lane + 64 * j, nch - 1));
#pragma unroll
            for (int j = 0; j < B8; ++j)
                if (base + lane + 64 * j < nch)
                    ss += (double)v[j].x * v[j].x + (double)v[j].y * v[j].y + (double)v[j].z * v[j].z + (double)v[j].w * v[j].w;
        }
        r_in = rms_factor(wave_sum(ss), K, a.eps);
        float amax = 0.0f;
        for (int base = 0; base < nch; base += 64 * B8) {
            float4 v[B8];
#pragma unroll
            for (int j = 0; j < B8; ++j) v[j] = qin_load4<QIN>(a, r, min(base + lane + 64 * j, nch - 1));
#pragma unroll
            for (int j = 0; j < B8; ++j) {
                const int c = base + lane + 64 * j;
                if (c < nch) amax = fmaxf(amax, absmax4(scale4(v[j], r_in, a.gain, c)));
            }
        }
        sc = quant_scale(wave_max(amax));
        for (int base = 0; base < nch; base += 64 * B8) {
            float4 v[B8];
#pragma unroll
            for (int j = 0; j < B8; ++j) v[j] = qin_load4<QIN>(a, r, min(base + lane + 64 * j, nch - 1));
#pragma unroll
            for (int j = 0; j < B8; ++j) {
                const int c = base + lane + 64 * j;
                if (c < nch) tot += emit4(scale4(v[j], r_in, a.gain, c), sc, lrow, prow, c);
            }
        }
    }
    tot = wave_sum_int(tot);
    if (lane == 0) {
        st.rs[r] = sc;
        st.rsq[r] = tot;
        if (probe && a.scale_out) a.scale_out[r] = sc;
    }
}

// One workgroup of 16 waves per 16*NCB output channels (x NG groups). Lane
// (wave w, word group lg, column lc) owns words [(4w + lg) * WPL, +WPL) of
// its columns, so 64 lane groups cover K.
template <int NG, int NCB, int EPI, int QIN, int WPL, int NV>
__global__ __launch_bounds__(1024) void decode_fused_kernel(const DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const ContractArgs &p = a.c;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lc = lane & 15, lg = lane >> 4;
    const int K = p.k, KW = K >> 4, M = (int)p.m;
    const int ldc = K + 16;
    int8_t *codes = reinterpret_cast<int8_t *>(lds);
    int32_t *red = reinterpret_cast<int32_t *>(lds + kDecRows * ldc);
    RowStats st;
    st.rs = reinterpret_cast<float *>(red + NG * NCB * 256);
    st.rsq = reinterpret_cast<int *>(st.rs + kDecRows);

    // 1. packed weights, issued before the quantiser
    const int n0 = blockIdx.x * 16 * NCB;
    const int w0 = (wave * 4 + lg) * WPL;
    const bool bvec = (KW & 3) == 0 && (WPL & 3) == 0;
    uint32_t bw[NG][NCB][WPL];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int gn = n0 + cb * 16 + lc;
            const uint32_t *src = p.B[g] + (int64_t)gn * KW + w0;
            if (bvec && gn < p.nc && w0 + WPL <= KW) {
#pragma unroll
                for (int u = 0; u < WPL / 4; ++u) {
                    const uint4 v = reinterpret_cast<const uint4 *>(src)[u];
                    bw[g][cb][4 * u] = v.x; bw[g][cb][4 * u + 1] = v.y; bw[g][cb][4 * u + 2] = v.z; bw[g][cb][4 * u + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < WPL; ++j) bw[g][cb][j] = (gn < p.nc && w0 + j < KW) ? src[j] : 0u;
            }
        }
    for (int i = tid; i < NG * NCB * 256; i += 1024) red[i] = 0;

    // 2. wave w quantises input row w
    if (wave < M) wave_quantize_row<QIN, NV>(a, wave, codes + wave * ldc, st);
    __syncthreads();

    // 3. contraction over this lane's words, activation fragments from LDS
    i32x4 acc[NG][NCB];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[g][cb] = i32x4{};
#pragma unroll
    for (int j = 0; j < WPL; ++j) {
        const int w = w0 + j;
        const i32x4 av = (lc < M && w < KW) ? *reinterpret_cast<const i32x4 *>(codes + lc * ldc + 16 * w) : i32x4{};
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                acc[g][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, decode_word(bw[g][cb][j]), acc[g][cb], 0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                atomicAdd(&red[((g * NCB + cb) * 16 + 4 * lg + i) * 16 + lc], acc[g][cb][i]);
    __syncthreads();

    // 4. epilogue
    float sw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sw[g] = weight_sw(p.mu[g]);
    for (int idx = tid; idx < NCB * 256; idx += 1024) {
        const int cb = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        const int col = n0 + cb * 16 + c;
        if (r < M && col < p.nc) {
            int32_t v[NG];
            float dq[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                v[g] = red[((g * NCB + cb) * 16 + r) * 16 + c] - st.rsq[r];
                dq[g] = __builtin_amdgcn_rcpf(st.rs[r] * sw[g]);
            }
            epilogue_vals<EPI, NG>(p, r, col, v, dq);
        }
    }
}

static size_t decode_lds_bytes(int k, int ng, int ncb) {
    return (size_t)kDecRows * (k + 16) + (size_t)ng * ncb * 256 * 4 + 2 * kDecRows * 4;
}

bool decode_fused_ok(int64_t m, int k) { return m >= 1 && m <= kDecRows && k <= kDecMaxK; }

template <int NG, int NCB, int EPI, int QIN, int WPL, int NV>
static hipError_t run_decode(const DecodeArgs &a, hipStream_t st) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&decode_fused_kernel<NG, NCB, EPI, QIN, WPL, NV>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)decode_lds_bytes(kDecMaxK, NG, NCB));
    if (attr != hipSuccess) return attr;
    const unsigned grid = (unsigned)((a.c.nc + 16 * NCB - 1) / (16 * NCB));
    decode_fused_kernel<NG, NCB, EPI, QIN, WPL, NV><<<grid, 1024, decode_lds_bytes(a.c.k, NG, NCB), st>>>(a);
    return hipGetLastError();
}

// words per lane so that 64 lane groups cover K; row-cache depth for the quantiser
template <int NG, int NCB, int EPI, int QIN>
static hipError_t run_decode_k(const DecodeArgs &a, hipStream_t st) {
    const int wpl_need = ((a.c.k >> 4) + 63) / 64;
    const int nv_need = ((a.c.k >> 2) + 63) / 64;
    if (wpl_need <= 2) {
        if (nv_need <= 8) return run_decode<NG, NCB, EPI, QIN, 2, 8>(a, st);
        return hipErrorInvalidValue;
    }
    if constexpr (QIN == QIN_GNORM) {
        return hipErrorInvalidValue;
    } else {
        if (wpl_need <= 4) {
            if (nv_need <= 16) return run_decode<NG, NCB, EPI, QIN, 4, 16>(a, st);
            return hipErrorInvalidValue;
        }
        return run_decode<NG, NCB, EPI, QIN, 8, 0>(a, st);
    }
}

bool decode_fused_supports(int k, QuantIn qin) {
    return k <= (qin == QIN_GNORM ? 2048 : kDecMaxK);
}

hipError_t launch_decode_fused(const DecodeArgs &a, EpiKind epi, QuantIn qin, hipStream_t st, std::string *path) {
    hipError_t e = hipErrorInvalidValue;
    const char *name = "?";
    if (epi == EPI_GATES_STEP && qin == QIN_F32) { e = run_decode_k<3, 2, EPI_GATES_STEP, QIN_F32>(a, st); name = "gates_step,f32"; }
    else if (epi == EPI_GATES_STEP && qin == QIN_BF16) { e = run_decode_k<3, 2, EPI_GATES_STEP, QIN_BF16>(a, st); name = "gates_step,bf16"; }
    else if (epi == EPI_RESID && qin == QIN_GNORM) { e = run_decode_k<1, 4, EPI_RESID, QIN_GNORM>(a, st); name = "resid,gnorm"; }
    else if (epi == EPI_GLU && qin == QIN_F32) { e = run_decode_k<2, 4, EPI_GLU, QIN_F32>(a, st); name = "glu,f32"; }
    else if (epi == EPI_RESID && qin == QIN_F32) { e = run_decode_k<1, 4, EPI_RESID, QIN_F32>(a, st); name = "resid,f32"; }
    if (path) *path += std::string("decode_fused<") + name + ">;";
    return e;
}

}  // namespace mmf
