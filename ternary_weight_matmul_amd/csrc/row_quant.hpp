// One row's quantiser computed by the first 256 threads (four waves) of a
// workgroup, for few rows (decode): RMSNorm + per-token absmax int8, and the
// g_norm RMSNorm-Swish gate followed by o_proj's quantiser ("MatMul-Free LLM
// 深度分析报告", list "可复用的模式与技巧": both fusions; eps from "MatMul-Free
// LM：把矩陣乘法從語言模型裡拿掉之後，剩下什麼", section "HGRNBitBlock 的結構").
//
// Every thread of the workgroup calls these functions (they contain workgroup
// barriers); threads from 256 on contribute nothing. Thread t owns the 4-element
// chunks t, t + 256, ... of the row; chunk slots past the row end are skipped
// (uniformly) or loaded from a clamped index and masked. The four waves'
// partial reductions meet in LDS in a fixed order, so the result does not
// depend on the caller: the separate decode kernels and the persistent decode
// step produce the same bits. NT: the row was written by another workgroup of
// the same launch and is read with non-temporal loads.
//
// Without a gain, y = x * r is monotone in |x| (r > 0, round-to-nearest is
// monotone and symmetric), so max |y| = (max |x|) * r exactly: the sum of
// squares and max |x| are reduced in the same round. With sumq == nullptr the
// sum of the codes is not formed (the decode GEMV computes it from the codes
// itself), which saves the last round.
#pragma once
#include "device_common.hpp"

namespace mmf {

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ float4 row_ld4(const float *p) {
    if constexpr (NT) {
        const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p));
        return make_float4(v[0], v[1], v[2], v[3]);
    } else {
        return *reinterpret_cast<const float4 *>(p);
    }
}
template <bool NT>
__device__ __forceinline__ float4 row_ld4(const uint16_t *p) {
    uint32_t lo, hi;
    if constexpr (NT) {
        const u32x2v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2v *>(p));
        lo = v[0];
        hi = v[1];
    } else {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        lo = v.x;
        hi = v.y;
    }
    return make_float4(__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u), __uint_as_float(hi << 16),
                       __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ void rq_set4(float (&d)[4], float4 v) { d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w; }

// Reductions over the waves of threads [0, 256); LDS slots used once each.
__device__ __forceinline__ double rq_sum(double v, double *sh) {
    v = wave_sum(v);
    const int t = threadIdx.x;
    if (t < 256 && (t & 63) == 0) sh[t >> 6] = v;
    __syncthreads();
    return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}
__device__ __forceinline__ float rq_max(float v, float *sh) {
    v = wave_max(v);
    const int t = threadIdx.x;
    if (t < 256 && (t & 63) == 0) sh[t >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}
// Sum and max in one round (two LDS arrays, one barrier).
__device__ __forceinline__ void rq_sum_max(double &v, float &mx, double *shd, float *shf) {
    v = wave_sum(v);
    mx = wave_max(mx);
    const int t = threadIdx.x;
    if (t < 256 && (t & 63) == 0) {
        shd[t >> 6] = v;
        shf[t >> 6] = mx;
    }
    __syncthreads();
    v = (shd[0] + shd[1]) + (shd[2] + shd[3]);
    mx = fmaxf(fmaxf(shf[0], shf[1]), fmaxf(shf[2], shf[3]));
}
__device__ __forceinline__ int rq_sum_int(int v, int *sh) {
    v = wave_sum_int(v);
    const int t = threadIdx.x;
    if (t < 256 && (t & 63) == 0) sh[t >> 6] = v;
    __syncthreads();
    return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

struct RowQuantLds {
    double d[2][4];
    float f[4];
    int i[4];
};

// Stores of the quantiser's results: plain, or device-scope (SC1: written
// through to memory, for readers on other XCDs within the same launch).
template <bool SC1>
__device__ __forceinline__ void rq_store(uint32_t *p, uint32_t v) {
    if constexpr (SC1) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// Codes of the 4-element chunks owned by the thread, the scale s (from the
// row's max |y|, already reduced) and, when sumq != nullptr, the sum of codes.
template <int NV, bool SC1 = false>
__device__ __forceinline__ void rq_emit(const float (&v)[NV][4], float row_amax, int nch, int8_t *qr, float *s,
                                        int32_t *sumq, RowQuantLds &sh) {
    const int tid = threadIdx.x;
    const float sc = quant_scale(row_amax);
    int tot = 0;
    uint32_t *qw = reinterpret_cast<uint32_t *>(qr);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = tid + 256 * j;
        if (tid < 256 && c < nch) {
            const int a0 = quant_code(v[j][0], sc), a1 = quant_code(v[j][1], sc);
            const int a2 = quant_code(v[j][2], sc), a3 = quant_code(v[j][3], sc);
            tot += a0 + a1 + a2 + a3;
            rq_store<SC1>(qw + c, pack_codes4(a0, a1, a2, a3));
        }
    }
    if (sumq) tot = rq_sum_int(tot, sh.i);
    if (tid == 0) {
        rq_store<SC1>(reinterpret_cast<uint32_t *>(s), __float_as_uint(sc));
        if (sumq) rq_store<SC1>(reinterpret_cast<uint32_t *>(sumq), (uint32_t)tot);
    }
}

// q = clamp(rint(((x * r) * gain) * s)), r = 1/sqrt(mean(x^2) + eps), s = 127 / max|y|
template <typename T, int NV, bool NT, bool SC1 = false>
__device__ __forceinline__ void row_quant(const T *xr, int k, const float *gain, float eps, int8_t *qr, float *s,
                                          int32_t *sumq, RowQuantLds &sh) {
    const int tid = threadIdx.x;
    const int nch = k >> 2;
    float v[NV][4], gv[NV][4];
    // straight-line loads under one wave-uniform branch (slots past the row end
    // read the last chunk and go unused): a branch per slot would make the
    // compiler wait for each load before the next
    if (tid < 256) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = min(tid + 256 * j, nch - 1);
            rq_set4(v[j], row_ld4<NT>(xr + 4 * (int64_t)c));
            rq_set4(gv[j], gain ? *reinterpret_cast<const float4 *>(gain + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f));
        }
    }
    double ss = 0.0;
    float xmax = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (tid < 256 && tid + 256 * j < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ss += (double)v[j][e] * (double)v[j][e];
                xmax = fmaxf(xmax, fabsf(v[j][e]));
            }
    float r, amax;
    if (!gain) {
        rq_sum_max(ss, xmax, sh.d[0], sh.f);
        r = rms_factor(ss, k, eps);
        amax = __fmul_rn(xmax, r);
    } else {
        r = rms_factor(rq_sum(ss, sh.d[0]), k, eps);
        amax = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (tid < 256 && tid + 256 * j < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float y = __fmul_rn(v[j][e], r);
                if (gain) {
                    y = __fmul_rn(y, gv[j][e]);
                    amax = fmaxf(amax, fabsf(y));
                }
                v[j][e] = y;
            }
    if (gain) amax = rq_max(amax, sh.f);
    rq_emit<NV, SC1>(v, amax, nch, qr, s, sumq, sh);
}

// u = ((h * r_h) * g_norm_w) * SiLU(g), then o_proj's quantiser of u; u_out optional
template <typename TG, int NV, bool NT, bool SC1 = false>
__device__ __forceinline__ void row_gnorm_quant(const float *hr, const TG *gr, int d, const float *gnw,
                                                const float *ogain, float eps, int8_t *qr, float *s, int32_t *sumq,
                                                float *u_out, RowQuantLds &sh) {
    const int tid = threadIdx.x;
    const int nch = d >> 2;
    float u[NV][4], gs[NV][4], wn[NV][4], og[NV][4];
    if (tid < 256) {  // straight-line loads, as in row_quant
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = min(tid + 256 * j, nch - 1);
            rq_set4(u[j], row_ld4<NT>(hr + 4 * (int64_t)c));
            rq_set4(gs[j], row_ld4<NT>(gr + 4 * (int64_t)c));
            rq_set4(wn[j], gnw ? *reinterpret_cast<const float4 *>(gnw + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f));
            rq_set4(og[j], ogain ? *reinterpret_cast<const float4 *>(ogain + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f));
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (tid < 256 && tid + 256 * j < nch) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gs[j][e] = silu_fast(gs[j][e]);
                ss += (double)u[j][e] * (double)u[j][e];
            }
        }
    const float rh = rms_factor(rq_sum(ss, sh.d[0]), d, eps);
    double su = 0.0;
    float umax = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = tid + 256 * j;
        if (tid < 256 && c < nch) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float y = u[j][e] * rh;
                if (gnw) y = y * wn[j][e];
                y = y * gs[j][e];
                u[j][e] = y;
                su += (double)y * (double)y;
                umax = fmaxf(umax, fabsf(y));
            }
            if (u_out) *reinterpret_cast<float4 *>(u_out + 4 * c) = make_float4(u[j][0], u[j][1], u[j][2], u[j][3]);
        }
    }
    float r, amax;
    if (!ogain) {
        rq_sum_max(su, umax, sh.d[1], sh.f);
        r = rms_factor(su, d, eps);
        amax = __fmul_rn(umax, r);
    } else {
        r = rms_factor(rq_sum(su, sh.d[1]), d, eps);
        amax = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (tid < 256 && tid + 256 * j < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float y = __fmul_rn(u[j][e], r);
                if (ogain) {
                    y = __fmul_rn(y, og[j][e]);
                    amax = fmaxf(amax, fabsf(y));
                }
                u[j][e] = y;
            }
    if (ogain) amax = rq_max(amax, sh.f);
    rq_emit<NV, SC1>(u, amax, nch, qr, s, sumq, sh);
}

}  // namespace mmf
