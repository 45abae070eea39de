// Row quantisers and the ternary weight packer (gfx950).
//
// RMSNorm fused with per-token absmax int8 quantisation, as the FusedBitLinear
// of the MatMul-free LM does ("MatMul-Free LLM 深度分析报告", list
// "可复用的模式与技巧"); eps of the RMSNorm from "MatMul-Free LM：把矩陣乘法從語言
// 模型裡拿掉之後，剩下什麼", section "HGRNBitBlock 的結構". The g_norm RMSNorm-Swish
// gate is fused with the o_proj quantiser in one pass over the row.
//
// One wavefront owns one row: the row is read once from HBM with 16-byte
// (fp32) or 8-byte (bf16) coalesced loads and kept in registers, the sum of
// squares is reduced in binary64 and the absmax in binary32 with cross-lane
// shuffles, and the int8 codes leave as one 32-bit store per 4 elements.
#include "device_common.hpp"
#include "launch.hpp"
#include "row_quant.hpp"

namespace mmf {

// ----------------------------------------------------------------------------
// norm_quant: q = clamp(rint(((x * r) * gain) * s)), r = rms factor, s = 127/amax
// ----------------------------------------------------------------------------
// A 16-byte chunk of a row kept as loaded: 4 fp32 or 8 bf16 elements. The
// bf16 chunk stays packed in registers (half the registers of fp32) and is
// widened at each use.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
    using R = float4;
    static constexpr int E = 4;
    static __device__ __forceinline__ float get(const R &r, int e) {
        return e == 0 ? r.x : e == 1 ? r.y : e == 2 ? r.z : r.w;
    }
};
template <> struct Chunk<uint16_t> {
    using R = uint4;
    static constexpr int E = 8;
    static __device__ __forceinline__ float get(const R &r, int e) {
        const uint32_t w = (e >> 1) == 0 ? r.x : (e >> 1) == 1 ? r.y : (e >> 1) == 2 ? r.z : r.w;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// y = (v * r) * gain of element e of chunk c
template <typename T>
__device__ __forceinline__ float scaled(const typename Chunk<T>::R &raw, int e, float r, const float *gain, int c) {
    float y = __fmul_rn(Chunk<T>::get(raw, e), r);
    if (gain) y = __fmul_rn(y, gain[Chunk<T>::E * c + e]);
    return y;
}

template <typename T, int NV>
__global__ __launch_bounds__(256) void norm_quant_kernel(const T *__restrict__ x, int64_t m, int k,
                                                         const float *__restrict__ gain, float eps,
                                                         int8_t *__restrict__ q, float *__restrict__ s,
                                                         int32_t *__restrict__ sumq) {
    using C = Chunk<T>;
    constexpr int E = C::E;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= m) return;
    const int nch = k / E;
    const typename C::R *xr = reinterpret_cast<const typename C::R *>(x + row * (int64_t)k);
    // every load first: a chunk index past the row end is clamped (its values are
    // masked below); chunk slots no lane of the wave needs are skipped uniformly
    typename C::R raw[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (kWave * j < nch) raw[j] = xr[min(lane + kWave * j, nch - 1)];
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (lane + kWave * j < nch)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double v = C::get(raw[j], e);
                ss += v * v;
            }
    const float r = rms_factor(wave_sum(ss), k, eps);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + kWave * j;
        if (c < nch)
#pragma unroll
            for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(scaled<T>(raw[j], e, r, gain, c)));
    }
    const float sc = quant_scale(wave_max(amax));
    int tot = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + kWave * j;
        if (c < nch) {
            uint32_t w[E / 4];
#pragma unroll
            for (int h = 0; h < E / 4; ++h) {
                int a[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = quant_code(scaled<T>(raw[j], 4 * h + e, r, gain, c), sc);
                    tot += a[e];
                }
                w[h] = pack_codes4(a[0], a[1], a[2], a[3]);
            }
            int8_t *qc = q + row * (int64_t)k + (int64_t)E * c;
            if constexpr (E == 8)
                *reinterpret_cast<uint2 *>(qc) = make_uint2(w[0], w[1]);
            else
                *reinterpret_cast<uint32_t *>(qc) = w[0];
        }
    }
    tot = wave_sum_int(tot);
    if (lane == 0) {
        s[row] = sc;
        if (sumq) sumq[row] = tot;
    }
}

// Rows longer than the register cache: three passes over the row (the later
// passes hit L2).
template <typename T>
__global__ __launch_bounds__(256) void norm_quant_long_kernel(const T *__restrict__ x, int64_t m, int k,
                                                              const float *__restrict__ gain, float eps,
                                                              int8_t *__restrict__ q, float *__restrict__ s,
                                                              int32_t *__restrict__ sumq) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= m) return;
    const T *xr = x + row * (int64_t)k;
    double ss = 0.0;
    for (int i = lane; i < k; i += kWave) {
        const float a = load_act(xr, i);
        ss += (double)a * (double)a;
    }
    const float r = rms_factor(wave_sum(ss), k, eps);
    float amax = 0.0f;
    for (int i = lane; i < k; i += kWave) {
        float y = __fmul_rn(load_act(xr, i), r);
        if (gain) y = __fmul_rn(y, gain[i]);
        amax = fmaxf(amax, fabsf(y));
    }
    const float sc = quant_scale(wave_max(amax));
    int tot = 0;
    int8_t *qr = q + row * (int64_t)k;
    for (int i = lane; i < k; i += kWave) {
        float y = __fmul_rn(load_act(xr, i), r);
        if (gain) y = __fmul_rn(y, gain[i]);
        const int c = quant_code(y, sc);
        tot += c;
        qr[i] = (int8_t)c;
    }
    tot = wave_sum_int(tot);
    if (lane == 0) {
        s[row] = sc;
        if (sumq) sumq[row] = tot;
    }
}

// Few rows (decode): one 256-thread workgroup per row (row_quant.hpp).
__device__ __forceinline__ float4 load_f4(const float *p, int c) { return *reinterpret_cast<const float4 *>(p + 4 * c); }
__device__ __forceinline__ void set4(float (&d)[4], float4 v) { d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w; }

template <typename T, int NV>
__global__ __launch_bounds__(256) void norm_quant_row_kernel(const T *__restrict__ x, int64_t m, int k,
                                                             const float *__restrict__ gain, float eps,
                                                             int8_t *__restrict__ q, float *__restrict__ s,
                                                             int32_t *__restrict__ sumq) {
    __shared__ RowQuantLds sh;
    const int64_t row = blockIdx.x;
    row_quant<T, NV, false>(x + row * (int64_t)k, k, gain, eps, q + row * (int64_t)k, s + row,
                            sumq ? sumq + row : nullptr, sh);
}

// Few rows too long for a 256-thread workgroup's registers (k > 8192): one
// 1024-thread workgroup per row walks it in 4-element chunks, three passes at
// most (Σx² and max |x| together, then max |y| only with a gain, then the
// codes, stored four to a word); the later passes hit L2. The sixteen waves'
// partial results meet in LDS in a fixed order.
template <typename T>
__global__ __launch_bounds__(1024) void norm_quant_longrow_kernel(const T *__restrict__ x, int64_t m, int k,
                                                                 const float *__restrict__ gain, float eps,
                                                                 int8_t *__restrict__ q, float *__restrict__ s,
                                                                 int32_t *__restrict__ sumq) {
    __shared__ double shd[16];
    __shared__ float shf[16];
    __shared__ int shi[16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t row = blockIdx.x;
    const T *xr = x + row * (int64_t)k;
    const int nch = k >> 2;
    double ss = 0.0;
    float xm = 0.0f;
    for (int c = tid; c < nch; c += 1024) {
        const float4 v = load_act4(xr, 4 * (int64_t)c);
        ss += (double)v.x * (double)v.x;
        ss += (double)v.y * (double)v.y;
        ss += (double)v.z * (double)v.z;
        ss += (double)v.w * (double)v.w;
        xm = fmaxf(fmaxf(xm, fabsf(v.x)), fmaxf(fabsf(v.y), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    ss = wave_sum(ss);
    xm = wave_max(xm);
    if (lane == 0) {
        shd[wave] = ss;
        shf[wave] = xm;
    }
    __syncthreads();
    double tot_ss = 0.0;
    float tot_xm = 0.0f;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        tot_ss += shd[w];
        tot_xm = fmaxf(tot_xm, shf[w]);
    }
    const float r = rms_factor(tot_ss, k, eps);
    float amax;
    if (!gain) {
        amax = __fmul_rn(tot_xm, r);  // r > 0: max |x r| = (max |x|) r exactly
    } else {
        float ym = 0.0f;
        for (int c = tid; c < nch; c += 1024) {
            const float4 v = load_act4(xr, 4 * (int64_t)c);
            const float4 g = *reinterpret_cast<const float4 *>(gain + 4 * (int64_t)c);
            ym = fmaxf(ym, fabsf(__fmul_rn(__fmul_rn(v.x, r), g.x)));
            ym = fmaxf(ym, fabsf(__fmul_rn(__fmul_rn(v.y, r), g.y)));
            ym = fmaxf(ym, fabsf(__fmul_rn(__fmul_rn(v.z, r), g.z)));
            ym = fmaxf(ym, fabsf(__fmul_rn(__fmul_rn(v.w, r), g.w)));
        }
        ym = wave_max(ym);
        __syncthreads();  // shf is reused
        if (lane == 0) shf[wave] = ym;
        __syncthreads();
        amax = 0.0f;
#pragma unroll
        for (int w = 0; w < 16; ++w) amax = fmaxf(amax, shf[w]);
    }
    const float sc = quant_scale(amax);
    uint32_t *qw = reinterpret_cast<uint32_t *>(q + row * (int64_t)k);
    int tot = 0;
    for (int c = tid; c < nch; c += 1024) {
        const float4 v = load_act4(xr, 4 * (int64_t)c);
        float y0 = __fmul_rn(v.x, r), y1 = __fmul_rn(v.y, r), y2 = __fmul_rn(v.z, r), y3 = __fmul_rn(v.w, r);
        if (gain) {
            const float4 g = *reinterpret_cast<const float4 *>(gain + 4 * (int64_t)c);
            y0 = __fmul_rn(y0, g.x);
            y1 = __fmul_rn(y1, g.y);
            y2 = __fmul_rn(y2, g.z);
            y3 = __fmul_rn(y3, g.w);
        }
        const int a0 = quant_code(y0, sc), a1 = quant_code(y1, sc), a2 = quant_code(y2, sc), a3 = quant_code(y3, sc);
        tot += a0 + a1 + a2 + a3;
        qw[c] = pack_codes4(a0, a1, a2, a3);
    }
    if (sumq) {
        tot = wave_sum_int(tot);
        if (lane == 0) shi[wave] = tot;
        __syncthreads();
        if (tid == 0) {
            int t = 0;
#pragma unroll
            for (int w = 0; w < 16; ++w) t += shi[w];
            sumq[row] = t;
        }
    }
    if (tid == 0) s[row] = sc;
}

constexpr int kFewRows = 2048;  // below this many rows a row gets a whole workgroup

constexpr int kMaxCachedChunks = 32;  // 64 lanes * 32 chunks of 16 bytes per row in registers

// 16-byte chunks of e elements per lane when a wave owns the row
// (powers of two up to 8, then 12, 16, 24, 32: a row of 5632 fp32 values takes 24, not 32,
// and the registers of the 8 chunk slots it would never fill)
static int chunk_bucket(int k, int e = 4) {
    const int nch = (k / e + kWave - 1) / kWave;
    if (nch > 16) return nch <= 24 ? 24 : 32;
    if (nch > 8) return nch <= 12 ? 12 : 16;
    int b = 1;
    while (b < nch) b *= 2;
    return b;
}

// float4 chunks per thread when a 256-thread workgroup owns the row
static int block_bucket(int k) {
    const int nch = (k / 4 + 255) / 256;
    int b = 1;
    while (b < nch) b *= 2;
    return b;
}

template <typename T>
static void norm_quant_dispatch(const T *x, int64_t m, int k, const float *gain, float eps, int8_t *q,
                                float *s, int32_t *sumq, hipStream_t st, std::string *path) {
    const char *tn = sizeof(T) == 4 ? "f32" : "bf16";
    const int nvb = block_bucket(k);
    // a whole workgroup per row for few rows, and for rows of 4096 and more at any count (the
    // wave-per-row kernel holds 24 or 32 chunk slots per lane there: measured on MI355X at
    // 32768 x 5632 fp32, 183 against 191 us)
    if ((m < kFewRows || k >= 4096) && nvb <= 8) {
        switch (nvb) {
#define MMF_NQB(NV) case NV: launch_k(norm_quant_row_kernel<T, NV>, (unsigned)m, 256, 0, st, x, m, k, gain, eps, q, s, sumq); break;
            MMF_NQB(1) MMF_NQB(2) MMF_NQB(4) MMF_NQB(8)
#undef MMF_NQB
        }
        if (path) *path += std::string("norm_quant_row<") + tn + "," + std::to_string(nvb) + ">;";
        return;
    }
    if (m < kFewRows && k % 4 == 0) {
        launch_k(norm_quant_longrow_kernel<T>, (unsigned)m, 1024, 0, st, x, m, k, gain, eps, q, s, sumq);
        if (path) *path += std::string("norm_quant_longrow<") + tn + ">;";
        return;
    }
    const dim3 grid((unsigned)((m + 3) / 4)), block(256);
    const int nv = chunk_bucket(k, Chunk<T>::E);
    if (k % Chunk<T>::E != 0 || nv > kMaxCachedChunks) {
        launch_k(norm_quant_long_kernel<T>, grid, block, 0, st, x, m, k, gain, eps, q, s, sumq);
        if (path) *path += std::string("norm_quant_long<") + tn + ">;";
        return;
    }
    switch (nv) {
#define MMF_NQ(NV) case NV: launch_k(norm_quant_kernel<T, NV>, grid, block, 0, st, x, m, k, gain, eps, q, s, sumq); break;
        MMF_NQ(1) MMF_NQ(2) MMF_NQ(4) MMF_NQ(8) MMF_NQ(12) MMF_NQ(16) MMF_NQ(24) MMF_NQ(32)
#undef MMF_NQ
    }
    if (path) *path += std::string("norm_quant<") + tn + "," + std::to_string(nv) + ">;";
}

hipError_t launch_norm_quant(const void *x, ActType xt, int64_t m, int k, const float *gain, float eps,
                             int8_t *q, float *s, int32_t *sumq, hipStream_t stream, std::string *path) {
    if (m <= 0) return hipSuccess;
    if (xt == ACT_F32)
        norm_quant_dispatch(static_cast<const float *>(x), m, k, gain, eps, q, s, sumq, stream, path);
    else
        norm_quant_dispatch(static_cast<const uint16_t *>(x), m, k, gain, eps, q, s, sumq, stream, path);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------
// gnorm_quant: u = ((h * r_h) * g_norm_w) * SiLU(g), then the o_proj quantiser of u
// ----------------------------------------------------------------------------
template <typename TG, int NV>
__global__ __launch_bounds__(256) void gnorm_quant_kernel(const float *__restrict__ h, const TG *__restrict__ g,
                                                          int64_t m, int d, const float *__restrict__ gnw,
                                                          const float *__restrict__ ogain, float eps,
                                                          int8_t *__restrict__ q, float *__restrict__ s,
                                                          int32_t *__restrict__ sumq, float *__restrict__ u_out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= m) return;
    const int nch = d >> 2;
    const float *hr = h + row * (int64_t)d;
    const TG *gr = g + row * (int64_t)d;
    float u[NV][4], gs[NV][4];
    // all loads first, from a clamped chunk index (chunks past the row end are
    // masked below), so that no load waits behind another
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = min(lane + kWave * j, nch - 1);
        set4(u[j], load_f4(hr, c));
        set4(gs[j], load_act4(gr, 4 * (int64_t)c));
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) gs[j][e] = silu_fast(gs[j][e]);
        if (lane + kWave * j < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += (double)u[j][e] * (double)u[j][e];
    }
    const float rh = rms_factor(wave_sum(ss), d, eps);
    double su = 0.0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + kWave * j;
        float4 wv = (gnw && c < nch) ? *reinterpret_cast<const float4 *>(gnw + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f);
        const float we[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float y = u[j][e] * rh;
            if (gnw) y = y * we[e];
            y = y * gs[j][e];
            u[j][e] = y;
            if (c < nch) su += (double)y * (double)y;
        }
        if (u_out && c < nch)
            *reinterpret_cast<float4 *>(u_out + row * (int64_t)d + 4 * c) = make_float4(u[j][0], u[j][1], u[j][2], u[j][3]);
    }
    const float r = rms_factor(wave_sum(su), d, eps);
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + kWave * j;
        if (c < nch) {
            float4 gv = ogain ? *reinterpret_cast<const float4 *>(ogain + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f);
            const float ge[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float y = __fmul_rn(u[j][e], r);
                if (ogain) y = __fmul_rn(y, ge[e]);
                u[j][e] = y;
                amax = fmaxf(amax, fabsf(y));
            }
        }
    }
    const float sc = quant_scale(wave_max(amax));
    int tot = 0;
    uint32_t *qr = reinterpret_cast<uint32_t *>(q + row * (int64_t)d);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = lane + kWave * j;
        if (c < nch) {
            const int a0 = quant_code(u[j][0], sc), a1 = quant_code(u[j][1], sc);
            const int a2 = quant_code(u[j][2], sc), a3 = quant_code(u[j][3], sc);
            tot += a0 + a1 + a2 + a3;
            qr[c] = pack_codes4(a0, a1, a2, a3);
        }
    }
    tot = wave_sum_int(tot);
    if (lane == 0) {
        s[row] = sc;
        if (sumq) sumq[row] = tot;
    }
}

// Few rows (decode): one 256-thread workgroup per row (row_quant.hpp).
template <typename TG, int NV>
__global__ __launch_bounds__(256) void gnorm_quant_row_kernel(const float *__restrict__ h, const TG *__restrict__ g,
                                                              int64_t m, int d, const float *__restrict__ gnw,
                                                              const float *__restrict__ ogain, float eps,
                                                              int8_t *__restrict__ q, float *__restrict__ s,
                                                              int32_t *__restrict__ sumq, float *__restrict__ u_out) {
    __shared__ RowQuantLds sh;
    const int64_t row = blockIdx.x;
    row_gnorm_quant<TG, NV, false>(h + row * (int64_t)d, g + row * (int64_t)d, d, gnw, ogain, eps,
                                   q + row * (int64_t)d, s + row, sumq ? sumq + row : nullptr,
                                   u_out ? u_out + row * (int64_t)d : nullptr,
                                   sh);
}

template <typename TG>
static hipError_t gnorm_dispatch(const float *h, const TG *g, int64_t m, int d, const float *g_norm_w,
                                 const float *o_gain, float eps, int8_t *q, float *s, int32_t *sumq, float *u_out,
                                 hipStream_t stream, std::string *path) {
    const int nvb = block_bucket(d);
    if (m < kFewRows && nvb <= 8) {
        switch (nvb) {
#define MMF_GQB(NV) case NV: launch_k(gnorm_quant_row_kernel<TG, NV>, (unsigned)m, 256, 0, stream, h, g, m, d, g_norm_w, o_gain, eps, q, s, sumq, u_out); break;
            MMF_GQB(1) MMF_GQB(2) MMF_GQB(4) MMF_GQB(8)
#undef MMF_GQB
        }
        if (path) *path += "gnorm_quant_row<" + std::to_string(nvb) + ">;";
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((m + 3) / 4)), block(256);
    const int nv = chunk_bucket(d);
    switch (nv) {
#define MMF_GQ(NV) case NV: launch_k(gnorm_quant_kernel<TG, NV>, grid, block, 0, stream, h, g, m, d, g_norm_w, o_gain, eps, q, s, sumq, u_out); break;
        MMF_GQ(1) MMF_GQ(2) MMF_GQ(4) MMF_GQ(8) MMF_GQ(12) MMF_GQ(16) MMF_GQ(24) MMF_GQ(32)
#undef MMF_GQ
        default: return hipErrorInvalidValue;  // d > 8192 is rejected by the ABI layer
    }
    if (path) *path += "gnorm_quant<" + std::to_string(nv) + ">;";
    return hipGetLastError();
}

hipError_t launch_gnorm_quant(const float *h, const void *g, ActType g_type, int64_t m, int d, const float *g_norm_w,
                              const float *o_gain, float eps, int8_t *q, float *s, int32_t *sumq,
                              float *u_out, hipStream_t stream, std::string *path) {
    if (m <= 0) return hipSuccess;
    if (g_type == ACT_F32)
        return gnorm_dispatch(h, static_cast<const float *>(g), m, d, g_norm_w, o_gain, eps, q, s, sumq, u_out, stream, path);
    return gnorm_dispatch(h, static_cast<const uint16_t *>(g), m, d, g_norm_w, o_gain, eps, q, s, sumq, u_out, stream, path);
}

// ----------------------------------------------------------------------------
// Ternary packer: mu = (float)(sum |w| / (n k)) (binary64, fixed order), then
// t = clamp(rint(w * sw), -1, 1), sw = 1 / max(mu, 1e-5), 16 codes t+1 per word.
// ----------------------------------------------------------------------------
constexpr int kPackPartials = 512;

size_t pack_workspace_bytes() { return kPackPartials * sizeof(double); }

// Sum of |w| over one block's range of the weights (a multiple of 256 elements;
// the whole tensor a multiple of 16): 16-byte loads, four of them in flight per
// thread, four binary64 accumulators, then a fixed-order tree over the block.
__global__ __launch_bounds__(256) void abs_sum_partial_kernel(const float *__restrict__ w, int64_t count,
                                                              int64_t per_block, double *__restrict__ partial) {
    __shared__ double red[256];
    const int64_t lo = (int64_t)blockIdx.x * per_block;
    const int64_t hi = lo + per_block < count ? lo + per_block : count;
    const float4 *w4 = reinterpret_cast<const float4 *>(w);
    const int64_t hi4 = hi >> 2;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    auto add4 = [](double acc, float4 v) {
        return acc + (((double)fabsf(v.x) + (double)fabsf(v.y)) + ((double)fabsf(v.z) + (double)fabsf(v.w)));
    };
    int64_t i = (lo >> 2) + threadIdx.x;
    for (; i + 768 < hi4; i += 1024) {
        const float4 v0 = w4[i], v1 = w4[i + 256], v2 = w4[i + 512], v3 = w4[i + 768];
        a0 = add4(a0, v0);
        a1 = add4(a1, v1);
        a2 = add4(a2, v2);
        a3 = add4(a3, v3);
    }
    for (; i < hi4; i += 256) a0 = add4(a0, w4[i]);
    const double acc = (a0 + a1) + (a2 + a3);
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ w, int n, int k,
                                                   const double *__restrict__ partial, int nparts,
                                                   uint32_t *__restrict__ packed, float *__restrict__ mu) {
    __shared__ double red[256];
    double acc = 0.0;
    for (int i = threadIdx.x; i < nparts; i += 256) acc += partial[i];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    const float m = (float)(red[0] / ((double)n * (double)k));
    if (blockIdx.x == 0 && threadIdx.x == 0) *mu = m;
    const float sw = __fdiv_rn(1.0f, fmaxf(m, 1e-5f));
    const int kw = k >> 4;
    const int64_t word = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (word >= (int64_t)n * kw) return;
    const int64_t row = word / kw;
    const int wi = (int)(word % kw);
    const float4 *src = reinterpret_cast<const float4 *>(w + row * (int64_t)k + 16 * wi);
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 v = src[j];
        const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float p = rintf(__fmul_rn(e[b], sw));
            p = fminf(fmaxf(p, -1.0f), 1.0f);
            const uint32_t c = (uint32_t)((int)p + 1);
            // element 4j + b of the word: j-th code of byte b
            out |= c << (8 * b + 2 * j);
        }
    }
    packed[word] = out;
}

hipError_t launch_pack(const float *w, int n, int k, uint32_t *packed, float *mu, void *ws,
                       hipStream_t stream, std::string *path) {
    const int64_t count = (int64_t)n * k;
    int64_t per = (count + kPackPartials - 1) / kPackPartials;
    per = (per + 255) / 256 * 256;
    const int nparts = (int)((count + per - 1) / per);
    double *partial = static_cast<double *>(ws);
    launch_k(abs_sum_partial_kernel, nparts, 256, 0, stream, w, count, per, partial);
    const int64_t words = (int64_t)n * (k >> 4);
    launch_k(pack_kernel, (unsigned)((words + 255) / 256), 256, 0, stream, w, n, k, partial, nparts, packed, mu);
    if (path) *path += "abs_sum_partial;pack;";
    return hipGetLastError();
}

}  // namespace mmf
