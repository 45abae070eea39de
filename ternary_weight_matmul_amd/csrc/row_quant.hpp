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

// Codes of the 4-element chunks owned by the thread, the scale s and sum q.
template <int NV>
__device__ __forceinline__ void rq_emit(const float (&v)[NV][4], float amax, int nch, int8_t *qr, float *s, int32_t *sumq,
                                        RowQuantLds &sh) {
    const int tid = threadIdx.x;
    const float sc = quant_scale(rq_max(amax, sh.f));
    int tot = 0;
    uint32_t *qw = reinterpret_cast<uint32_t *>(qr);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = tid + 256 * j;
        if (tid < 256 && c < nch) {
            const int a0 = quant_code(v[j][0], sc), a1 = quant_code(v[j][1], sc);
            const int a2 = quant_code(v[j][2], sc), a3 = quant_code(v[j][3], sc);
            tot += a0 + a1 + a2 + a3;
            qw[c] = pack_codes4(a0, a1, a2, a3);
        }
    }
    tot = rq_sum_int(tot, sh.i);
    if (tid == 0) {
        *s = sc;
        *sumq = tot;
    }
}

// q = clamp(rint(((x * r) * gain) * s)), r = 1/sqrt(mean(x^2) + eps), s = 127 / max|y|
template <typename T, int NV, bool NT>
__device__ __forceinline__ void row_quant(const T *xr, int k, const float *gain, float eps, int8_t *qr, float *s,
                                          int32_t *sumq, RowQuantLds &sh) {
    const int tid = threadIdx.x;
    const int nch = k >> 2;
    float v[NV][4], gv[NV][4];
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (tid < 256 && 256 * j < nch) {
            const int c = min(tid + 256 * j, nch - 1);
            rq_set4(v[j], row_ld4<NT>(xr + 4 * (int64_t)c));
            rq_set4(gv[j], gain ? *reinterpret_cast<const float4 *>(gain + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f));
        }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (tid < 256 && tid + 256 * j < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += (double)v[j][e] * (double)v[j][e];
    const float r = rms_factor(rq_sum(ss, sh.d[0]), k, eps);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (tid < 256 && tid + 256 * j < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float y = __fmul_rn(v[j][e], r);
                if (gain) y = __fmul_rn(y, gv[j][e]);
                v[j][e] = y;
                amax = fmaxf(amax, fabsf(y));
            }
    rq_emit<NV>(v, amax, nch, qr, s, sumq, sh);
}

// u = ((h * r_h) * g_norm_w) * SiLU(g), then o_proj's quantiser of u; u_out optional
template <typename TG, int NV, bool NT>
__device__ __forceinline__ void row_gnorm_quant(const float *hr, const TG *gr, int d, const float *gnw,
                                                const float *ogain, float eps, int8_t *qr, float *s, int32_t *sumq,
                                                float *u_out, RowQuantLds &sh) {
    const int tid = threadIdx.x;
    const int nch = d >> 2;
    float u[NV][4], gs[NV][4], wn[NV][4], og[NV][4];
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (tid < 256 && 256 * j < nch) {
            const int c = min(tid + 256 * j, nch - 1);
            rq_set4(u[j], row_ld4<NT>(hr + 4 * (int64_t)c));
            rq_set4(gs[j], row_ld4<NT>(gr + 4 * (int64_t)c));
            rq_set4(wn[j], gnw ? *reinterpret_cast<const float4 *>(gnw + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f));
            rq_set4(og[j], ogain ? *reinterpret_cast<const float4 *>(ogain + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f));
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
            }
            if (u_out) *reinterpret_cast<float4 *>(u_out + 4 * c) = make_float4(u[j][0], u[j][1], u[j][2], u[j][3]);
        }
    }
    const float r = rms_factor(rq_sum(su, sh.d[1]), d, eps);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (tid < 256 && tid + 256 * j < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float y = __fmul_rn(u[j][e], r);
                if (ogain) y = __fmul_rn(y, og[j][e]);
                u[j][e] = y;
                amax = fmaxf(amax, fabsf(y));
            }
    rq_emit<NV>(u, amax, nch, qr, s, sumq, sh);
}

// ---------------------------------------------------------------------------
// The same two quantisers computed by ONE wave for one row, for kernels that
// quantise their own input rows (a wave per row) into LDS. The reduction order
// is that of the 256-thread functions above, so the codes, s and sum q are the
// same bits: lane l plays the threads l, l + 64, l + 128 and l + 192 (chunk
// c = l + 64 m belongs to thread l + 64 (m % 4)); each thread's sum runs over
// its chunks in order; the four thread-waves' sums are formed by wave_sum and
// combined as (w0 + w1) + (w2 + w3). Max and integer sums do not depend on the
// order. The lane keeps the raw row (NC chunks at most: nc_chunks(k) <= NC)
// and recomputes the scaled values in each pass; gains are read from LDS.
// ---------------------------------------------------------------------------
template <typename T> struct RawRow;
template <> struct RawRow<float> { typedef float4 type; };
template <> struct RawRow<uint16_t> { typedef uint2 type; };

template <bool NT>
__device__ __forceinline__ float4 raw_ld(const float *p) { return row_ld4<NT>(p); }
template <bool NT>
__device__ __forceinline__ uint2 raw_ld(const uint16_t *p) {
    if constexpr (NT) {
        const u32x2v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2v *>(p));
        return make_uint2(v[0], v[1]);
    } else {
        return *reinterpret_cast<const uint2 *>(p);
    }
}
__device__ __forceinline__ float4 raw_f4(float4 v) { return v; }
__device__ __forceinline__ float4 raw_f4(uint2 v) {
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                       __uint_as_float(v.y & 0xffff0000u));
}
__device__ __forceinline__ float f4_at(const float4 &v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
__device__ __forceinline__ float4 lds_f4(const float *p, int c) {
    return p ? *reinterpret_cast<const float4 *>(p + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f);
}

// Loads of the row's chunks owned by this lane (issued together; slots past
// the row end load the last chunk and are never used).
template <typename T, int NC, bool NT>
__device__ __forceinline__ void wave_row_load(const T *xr, int k, typename RawRow<T>::type (&raw)[NC]) {
    const int lane = threadIdx.x & 63, nch = k >> 2;
#pragma unroll
    for (int m = 0; m < NC; ++m)
        if (64 * m < nch) raw[m] = raw_ld<NT>(xr + 4 * (int64_t)min(lane + 64 * m, nch - 1));
}

__device__ __forceinline__ double wave_sum4(const double (&ss)[4]) {
    const double a = wave_sum(ss[0]), b = wave_sum(ss[1]), c = wave_sum(ss[2]), d = wave_sum(ss[3]);
    return (a + b) + (c + d);
}

// Codes of the row into qr (LDS), s and sum q into *s / *sumq (LDS, lane 0).
// y(m, e) recomputes the scaled value of element e of the lane's chunk m.
template <int NC, typename Y>
__device__ __forceinline__ void wave_emit(int nch, const Y &y, int8_t *qr, float *s, int32_t *sumq) {
    const int lane = threadIdx.x & 63;
    float amax = 0.0f;
#pragma unroll
    for (int m = 0; m < NC; ++m)
        if (lane + 64 * m < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(y(m, e)));
    const float sc = quant_scale(wave_max(amax));
    int tot = 0;
    uint32_t *qw = reinterpret_cast<uint32_t *>(qr);
#pragma unroll
    for (int m = 0; m < NC; ++m) {
        const int c = lane + 64 * m;
        if (c < nch) {
            const int a0 = quant_code(y(m, 0), sc), a1 = quant_code(y(m, 1), sc);
            const int a2 = quant_code(y(m, 2), sc), a3 = quant_code(y(m, 3), sc);
            tot += a0 + a1 + a2 + a3;
            qw[c] = pack_codes4(a0, a1, a2, a3);
        }
    }
    tot = wave_sum_int(tot);
    if (lane == 0) {
        *s = sc;
        *sumq = tot;
    }
}

// row_quant of a row already loaded by wave_row_load; gain in LDS (or null)
template <typename T, int NC>
__device__ __forceinline__ void wave_row_quant(const typename RawRow<T>::type (&raw)[NC], int k, const float *gain,
                                               float eps, int8_t *qr, float *s, int32_t *sumq) {
    const int lane = threadIdx.x & 63, nch = k >> 2;
    double ss[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int m = 0; m < NC; ++m)
        if (lane + 64 * m < nch) {
            const float4 v = raw_f4(raw[m]);
            ss[m & 3] += (double)v.x * (double)v.x;
            ss[m & 3] += (double)v.y * (double)v.y;
            ss[m & 3] += (double)v.z * (double)v.z;
            ss[m & 3] += (double)v.w * (double)v.w;
        }
    const float r = rms_factor(wave_sum4(ss), k, eps);
    auto y = [&](int m, int e) {
        float v = __fmul_rn(f4_at(raw_f4(raw[m]), e), r);
        if (gain) v = __fmul_rn(v, f4_at(lds_f4(gain, lane + 64 * m), e));
        return v;
    };
    wave_emit<NC>(nch, y, qr, s, sumq);
}

// row_gnorm_quant of rows h (fp32) and g loaded by wave_row_load; g_norm weight
// and o_proj gain in LDS (or null)
template <typename TG, int NC>
__device__ __forceinline__ void wave_row_gnorm_quant(const float4 (&hraw)[NC], const typename RawRow<TG>::type (&graw)[NC],
                                                     int d, const float *gnw, const float *ogain, float eps, int8_t *qr,
                                                     float *s, int32_t *sumq) {
    const int lane = threadIdx.x & 63, nch = d >> 2;
    double ss[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int m = 0; m < NC; ++m)
        if (lane + 64 * m < nch) {
            const float4 v = hraw[m];
            ss[m & 3] += (double)v.x * (double)v.x;
            ss[m & 3] += (double)v.y * (double)v.y;
            ss[m & 3] += (double)v.z * (double)v.z;
            ss[m & 3] += (double)v.w * (double)v.w;
        }
    const float rh = rms_factor(wave_sum4(ss), d, eps);
    auto u = [&](int m, int e) {
        float v = f4_at(hraw[m], e) * rh;
        if (gnw) v = v * f4_at(lds_f4(gnw, lane + 64 * m), e);
        return v * silu_fast(f4_at(raw_f4(graw[m]), e));
    };
    double su[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int m = 0; m < NC; ++m)
        if (lane + 64 * m < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = u(m, e);
                su[m & 3] += (double)v * (double)v;
            }
    const float r = rms_factor(wave_sum4(su), d, eps);
    auto y = [&](int m, int e) {
        float v = __fmul_rn(u(m, e), r);
        if (ogain) v = __fmul_rn(v, f4_at(lds_f4(ogain, lane + 64 * m), e));
        return v;
    };
    wave_emit<NC>(nch, y, qr, s, sumq);
}

}  // namespace mmf
