// Derivative of FusedBitLinear with straight-through quantisers (gfx950).
//
// "MatMul-Free LLM 深度分析报告", list "可复用的模式与技巧": the ternary weight
// quantiser rounds in the forward pass and passes the gradient through unchanged
// in the backward pass (straight-through estimator); the activation quantiser is
// read the same way. The forward product is y = u^ W^T with the dequantised
// operands u^ = q / s (codes of the RMSNorm'd row) and W^ = t / sw, so
//   du = dy W^,   dW = dy^T u^,
// and the RMSNorm u = x r gain, r = (mean(x^2) + eps)^(-1/2), gives
//   dx_k = r gain_k du_k - (r^3 / K) x_k sum_j x_j gain_j du_j,
//   dgain_k = sum over rows of du_k x_k r.
//
// The two products run as hand-written bf16 GEMMs (k_gemm_bf16.hip); what is
// not a product -- fp32 -> bf16, the RMSNorm derivative and the gain's column
// sums -- is the kernels below.
#include "device_common.hpp"
#include "launch.hpp"

namespace mmf {

// fp32 -> bf16 (round to nearest even), 4 per thread
__global__ __launch_bounds__(256) void to_bf16_kernel(const float *__restrict__ x, int64_t n4, uint16_t *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 v = reinterpret_cast<const float4 *>(x)[i];
    reinterpret_cast<uint2 *>(out)[i] =
        make_uint2((uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                   (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16));
}

// The RMSNorm derivative for `rows` consecutive rows per workgroup (256
// threads; thread t owns the 4-element chunks t, t + 256, ... of a row):
// du = du_raw / sw, then per row the sums x.x (binary64) and x.(gain du) meet in
// LDS in one round, and dx = r gain du - (r^3 / K) x c. The gain's derivative is
// summed over the workgroup's rows in registers and written as one partial row.
template <typename TX, typename TD, int NV>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const TX *__restrict__ x, const float *__restrict__ du_raw,
                                                          const float *__restrict__ gain, const float *__restrict__ mu,
                                                          float eps, int64_t m, int k, int rows, TD *__restrict__ dx,
                                                          float *__restrict__ gpart) {
    __shared__ double red[2][2][4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nch = k >> 2;
    const float sw = __fdiv_rn(1.0f, fmaxf(*mu, 1e-5f));
    float gv[NV][4], gacc[NV][4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = min(tid + 256 * j, nch - 1);
        const float4 g = gain ? *reinterpret_cast<const float4 *>(gain + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f);
        gv[j][0] = g.x; gv[j][1] = g.y; gv[j][2] = g.z; gv[j][3] = g.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) gacc[j][e] = 0.0f;
    }
    const int64_t r0 = (int64_t)blockIdx.x * rows;
    const int64_t r1 = r0 + rows < m ? r0 + rows : m;
    for (int64_t row = r0; row < r1; ++row) {
        const int buf = (int)(row & 1);
        float xv[NV][4], dv[NV][4];
#pragma unroll
        for (int j = 0; j < NV; ++j) {  // straight-line loads; slots past the row end repeat the last chunk
            const int c = min(tid + 256 * j, nch - 1);
            const float4 a = load_act4(x + row * k, 4 * c);
            const float4 d = *reinterpret_cast<const float4 *>(du_raw + row * k + 4 * c);
            xv[j][0] = a.x; xv[j][1] = a.y; xv[j][2] = a.z; xv[j][3] = a.w;
            dv[j][0] = d.x; dv[j][1] = d.y; dv[j][2] = d.z; dv[j][3] = d.w;
        }
        double ss = 0.0, cs = 0.0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
            if (tid + 256 * j < nch)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dv[j][e] = __fdiv_rn(dv[j][e], sw);
                    ss += (double)xv[j][e] * (double)xv[j][e];
                    cs += (double)xv[j][e] * (double)(gv[j][e] * dv[j][e]);
                }
        ss = wave_sum(ss);
        cs = wave_sum(cs);
        if (lane == 0) {
            red[buf][0][wv] = ss;
            red[buf][1][wv] = cs;
        }
        __syncthreads();
        ss = (red[buf][0][0] + red[buf][0][1]) + (red[buf][0][2] + red[buf][0][3]);
        cs = (red[buf][1][0] + red[buf][1][1]) + (red[buf][1][2] + red[buf][1][3]);
        const float r = rms_factor(ss, k, eps);
        const float coef = (r * r * r) / (float)k;
        const float c = (float)cs;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int ch = tid + 256 * j;
            if (ch < nch) {
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[e] = r * gv[j][e] * dv[j][e] - coef * xv[j][e] * c;
                    gacc[j][e] += dv[j][e] * xv[j][e] * r;
                }
                if (dx) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) store_act(dx, row * k + 4 * ch + e, o[e]);
                }
            }
        }
    }
    if (gpart) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int ch = tid + 256 * j;
            if (ch < nch)
                *reinterpret_cast<float4 *>(gpart + (int64_t)blockIdx.x * k + 4 * ch) =
                    make_float4(gacc[j][0], gacc[j][1], gacc[j][2], gacc[j][3]);
        }
    }
}

// dgain[k] = sum of the partial rows, in two fixed-order levels: workgroup
// (x, y) sums the partial rows of split y for 64 columns (four row groups of 64
// threads meet in LDS) into part2[y]; then each column sums part2 over y.
constexpr int kGainSplits = 64;
__global__ __launch_bounds__(256) void gain_reduce_kernel(const float *__restrict__ part, int nblk, int k,
                                                          float *__restrict__ part2) {
    __shared__ float red[4][64];
    const int lane = threadIdx.x & 63, rg = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    const int per = (nblk + gridDim.y - 1) / gridDim.y;
    const int b0 = blockIdx.y * per, b1 = min(b0 + per, nblk);
    float acc = 0.0f;
    if (c < k)
        for (int b = b0 + rg; b < b1; b += 4) acc += part[(int64_t)b * k + c];
    red[rg][lane] = acc;
    __syncthreads();
    if (rg == 0 && c < k) part2[(int64_t)blockIdx.y * k + c] = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
}

__global__ __launch_bounds__(256) void gain_final_kernel(const float *__restrict__ part2, int splits, int k,
                                                         float *__restrict__ dgain) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= k) return;
    float acc = 0.0f;
    for (int y = 0; y < splits; ++y) acc += part2[(int64_t)y * k + c];
    dgain[c] = acc;
}

// ---------------------------------------------------------------------------
// The block's elementwise pieces (forward values kept for the derivative, and
// their derivatives); n4 = elements / 4, four per thread.
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ T act_from(float v);
template <> __device__ __forceinline__ float act_from<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t act_from<uint16_t>(float v) { return f32_to_bf16(v); }

// f = sigmoid(f^), x~ = (1 - f) SiLU(i^), g stored in the activation type: the
// same operations as the fused gate epilogue of the forward contraction
template <typename AT>
__global__ __launch_bounds__(256) void gates_keep_kernel(const float *__restrict__ ih, const float *__restrict__ fh,
                                                         const float *__restrict__ gh, int64_t n4, float *__restrict__ f,
                                                         float *__restrict__ xt, AT *__restrict__ g) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float4 a = reinterpret_cast<const float4 *>(ih)[i], b = reinterpret_cast<const float4 *>(fh)[i];
    const float4 c = reinterpret_cast<const float4 *>(gh)[i];
    const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w}, cv[4] = {c.x, c.y, c.z, c.w};
    float fo[4], xo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        fo[e] = sigmoid_fast(bv[e]);
        xo[e] = (1.0f - fo[e]) * silu_fast(av[e]);
        g[4 * i + e] = act_from<AT>(cv[e]);
    }
    reinterpret_cast<float4 *>(f)[i] = make_float4(fo[0], fo[1], fo[2], fo[3]);
    reinterpret_cast<float4 *>(xt)[i] = make_float4(xo[0], xo[1], xo[2], xo[3]);
}

// z = SiLU(a) * b for [a | b] rows of 2 inner, z stored in the activation type
// (the forward's GLU epilogue)
template <typename AT>
__global__ __launch_bounds__(256) void glu_keep_kernel(const float *__restrict__ ab, int64_t m, int inner,
                                                       AT *__restrict__ z) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= m * inner) return;
    const int64_t row = i / inner, c = i - row * inner;
    const float a = ab[row * 2 * inner + c], b = ab[row * 2 * inner + inner + c];
    z[i] = act_from<AT>(silu_fast(a) * b);
}

__device__ __forceinline__ float dsilu_f(float z) {
    const float sg = sigmoid_fast(z);
    return sg * (1.0f + z * (1.0f - sg));
}

// da = dz b SiLU'(a), db = dz SiLU(a)
__global__ __launch_bounds__(256) void glu_bwd_kernel(const float *__restrict__ dz, const float *__restrict__ ab,
                                                      int64_t m, int inner, float *__restrict__ dab) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= m * inner) return;
    const int64_t row = i / inner, c = i - row * inner;
    const float a = ab[row * 2 * inner + c], b = ab[row * 2 * inner + inner + c], g = dz[i];
    dab[row * 2 * inner + c] = g * b * dsilu_f(a);
    dab[row * 2 * inner + inner + c] = g * silu_fast(a);
}

// gate derivatives in place: dxt <- di^ = dxt (1 - f) SiLU'(i^), df <- df^ = (df - dxt SiLU(i^)) f (1 - f)
__global__ __launch_bounds__(256) void gates_bwd_kernel(float *__restrict__ dxt, float *__restrict__ df,
                                                        const float *__restrict__ ih, const float *__restrict__ f,
                                                        int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float x = dxt[i], fv = f[i], iv = ih[i];
    df[i] = (df[i] - x * silu_fast(iv)) * fv * (1.0f - fv);
    dxt[i] = x * (1.0f - fv) * dsilu_f(iv);
}

// out = a (type TA) + b + c + d (fp32; c, d may be null), in that order
template <typename TA>
__global__ __launch_bounds__(256) void sum_kernel(const TA *__restrict__ a, const float *__restrict__ b,
                                                  const float *__restrict__ c, const float *__restrict__ d, int64_t n,
                                                  float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float v = load_act(a, i) + b[i];
    if (c) v += c[i];
    if (d) v += d[i];
    out[i] = v;
}

// g_norm's derivative per row, u = (h r) w SiLU(g), r = (mean(h^2) + eps)^(-1/2):
// dn = du w SiLU(g); dg = du (h r) w SiLU'(g); dh = r dn - (r^3 / d) h (h . dn);
// the weight's derivative du (h r) SiLU(g) summed over the workgroup's rows.
// Same row scheme as rmsnorm_bwd_kernel.
template <typename TG, int NV>
__global__ __launch_bounds__(256) void gnorm_bwd_kernel(const float *__restrict__ h, const TG *__restrict__ g,
                                                        const float *__restrict__ du, const float *__restrict__ w,
                                                        float eps, int64_t m, int d, int rows, float *__restrict__ dh,
                                                        float *__restrict__ dg, float *__restrict__ wpart) {
    __shared__ double red[2][2][4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nch = d >> 2;
    float wvv[NV][4], wacc[NV][4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int c = min(tid + 256 * j, nch - 1);
        const float4 q = w ? *reinterpret_cast<const float4 *>(w + 4 * c) : make_float4(1.f, 1.f, 1.f, 1.f);
        wvv[j][0] = q.x; wvv[j][1] = q.y; wvv[j][2] = q.z; wvv[j][3] = q.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) wacc[j][e] = 0.0f;
    }
    const int64_t r0 = (int64_t)blockIdx.x * rows;
    const int64_t r1 = r0 + rows < m ? r0 + rows : m;
    for (int64_t row = r0; row < r1; ++row) {
        const int buf = (int)(row & 1);
        float hv[NV][4], gv[NV][4], uv[NV][4], dn[NV][4];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = min(tid + 256 * j, nch - 1);
            const float4 a = *reinterpret_cast<const float4 *>(h + row * d + 4 * c);
            const float4 b = load_act4(g + row * d, 4 * c);
            const float4 e = *reinterpret_cast<const float4 *>(du + row * d + 4 * c);
            hv[j][0] = a.x; hv[j][1] = a.y; hv[j][2] = a.z; hv[j][3] = a.w;
            gv[j][0] = b.x; gv[j][1] = b.y; gv[j][2] = b.z; gv[j][3] = b.w;
            uv[j][0] = e.x; uv[j][1] = e.y; uv[j][2] = e.z; uv[j][3] = e.w;
        }
        double ss = 0.0, cs = 0.0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dn[j][e] = uv[j][e] * wvv[j][e] * silu_fast(gv[j][e]);
                if (tid + 256 * j < nch) {
                    ss += (double)hv[j][e] * (double)hv[j][e];
                    cs += (double)hv[j][e] * (double)dn[j][e];
                }
            }
        ss = wave_sum(ss);
        cs = wave_sum(cs);
        if (lane == 0) {
            red[buf][0][wv] = ss;
            red[buf][1][wv] = cs;
        }
        __syncthreads();
        ss = (red[buf][0][0] + red[buf][0][1]) + (red[buf][0][2] + red[buf][0][3]);
        cs = (red[buf][1][0] + red[buf][1][1]) + (red[buf][1][2] + red[buf][1][3]);
        const float r = rms_factor(ss, d, eps);
        const float coef = (r * r * r) / (float)d;
        const float c = (float)cs;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int ch = tid + 256 * j;
            if (ch < nch) {
                float oh[4], og[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float nv = hv[j][e] * r;
                    oh[e] = r * dn[j][e] - coef * hv[j][e] * c;
                    og[e] = uv[j][e] * nv * wvv[j][e] * dsilu_f(gv[j][e]);
                    wacc[j][e] += uv[j][e] * nv * silu_fast(gv[j][e]);
                }
                *reinterpret_cast<float4 *>(dh + row * d + 4 * ch) = make_float4(oh[0], oh[1], oh[2], oh[3]);
                *reinterpret_cast<float4 *>(dg + row * d + 4 * ch) = make_float4(og[0], og[1], og[2], og[3]);
            }
        }
    }
    if (wpart) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int ch = tid + 256 * j;
            if (ch < nch)
                *reinterpret_cast<float4 *>(wpart + (int64_t)blockIdx.x * d + 4 * ch) =
                    make_float4(wacc[j][0], wacc[j][1], wacc[j][2], wacc[j][3]);
        }
    }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int rmsnorm_bwd_rows(int64_t m) {
    const int64_t target = 2048;  // workgroups
    int64_t r = (m + target - 1) / target;
    return (int)(r < 1 ? 1 : r);
}

static int nv_bucket(int k) {
    const int n = (k / 4 + 255) / 256;
    int b = 1;
    while (b < n) b *= 2;
    return b;
}

bool rmsnorm_bwd_supported(int k) { return k % 8 == 0 && nv_bucket(k) <= 8; }

hipError_t launch_to_bf16(const float *x, int64_t n, uint16_t *out, hipStream_t st) {
    const int64_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    launch_k(to_bf16_kernel, (unsigned)((n4 + 255) / 256), 256, 0, st, x, n4, out);
    return hipGetLastError();
}

template <typename TX, typename TD>
static void rms_bwd_t(const TX *x, const float *du_raw, const float *gain, const float *mu, float eps, int64_t m, int k,
                      TD *dx, float *gpart, hipStream_t st) {
    const int rows = rmsnorm_bwd_rows(m);
    const unsigned grid = (unsigned)((m + rows - 1) / rows);
    switch (nv_bucket(k)) {
#define MMF_RB(NV) case NV: launch_k(rmsnorm_bwd_kernel<TX, TD, NV>, grid, 256, 0, st, x, du_raw, gain, mu, eps, m, k, rows, dx, gpart); break;
        MMF_RB(1) MMF_RB(2) MMF_RB(4) MMF_RB(8)
#undef MMF_RB
    }
}

hipError_t launch_rmsnorm_bwd(const void *x, ActType xt, const float *du_raw, const float *gain, const float *mu,
                              float eps, int64_t m, int k, void *dx, ActType dxt, float *gpart, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    if (xt == ACT_F32) {
        if (dxt == ACT_F32) rms_bwd_t(static_cast<const float *>(x), du_raw, gain, mu, eps, m, k, static_cast<float *>(dx), gpart, st);
        else rms_bwd_t(static_cast<const float *>(x), du_raw, gain, mu, eps, m, k, static_cast<uint16_t *>(dx), gpart, st);
    } else {
        if (dxt == ACT_F32) rms_bwd_t(static_cast<const uint16_t *>(x), du_raw, gain, mu, eps, m, k, static_cast<float *>(dx), gpart, st);
        else rms_bwd_t(static_cast<const uint16_t *>(x), du_raw, gain, mu, eps, m, k, static_cast<uint16_t *>(dx), gpart, st);
    }
    return hipGetLastError();
}

static unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_gates_keep(const float *ih, const float *fh, const float *gh, int64_t n, float *f, float *xt, void *g,
                             ActType gt, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (gt == ACT_F32) launch_k(gates_keep_kernel<float>, blocks(n / 4), 256, 0, st, ih, fh, gh, n / 4, f, xt, static_cast<float *>(g));
    else launch_k(gates_keep_kernel<uint16_t>, blocks(n / 4), 256, 0, st, ih, fh, gh, n / 4, f, xt, static_cast<uint16_t *>(g));
    return hipGetLastError();
}

hipError_t launch_glu_keep(const float *ab, int64_t m, int inner, void *z, ActType zt, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    if (zt == ACT_F32) launch_k(glu_keep_kernel<float>, blocks(m * inner), 256, 0, st, ab, m, inner, static_cast<float *>(z));
    else launch_k(glu_keep_kernel<uint16_t>, blocks(m * inner), 256, 0, st, ab, m, inner, static_cast<uint16_t *>(z));
    return hipGetLastError();
}

hipError_t launch_glu_bwd(const float *dz, const float *ab, int64_t m, int inner, float *dab, hipStream_t st) {
    if (m > 0) launch_k(glu_bwd_kernel, blocks(m * inner), 256, 0, st, dz, ab, m, inner, dab);
    return hipGetLastError();
}

hipError_t launch_gates_bwd(float *dxt, float *df, const float *ih, const float *f, int64_t n, hipStream_t st) {
    if (n > 0) launch_k(gates_bwd_kernel, blocks(n), 256, 0, st, dxt, df, ih, f, n);
    return hipGetLastError();
}

hipError_t launch_sum(const void *a, ActType at, const float *b, const float *c, const float *d, int64_t n, float *out,
                      hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (at == ACT_F32) launch_k(sum_kernel<float>, blocks(n), 256, 0, st, static_cast<const float *>(a), b, c, d, n, out);
    else launch_k(sum_kernel<uint16_t>, blocks(n), 256, 0, st, static_cast<const uint16_t *>(a), b, c, d, n, out);
    return hipGetLastError();
}

template <typename TG>
static void gnorm_bwd_t(const float *h, const TG *g, const float *du, const float *w, float eps, int64_t m, int d,
                        float *dh, float *dg, float *wpart, hipStream_t st) {
    const int rows = rmsnorm_bwd_rows(m);
    const unsigned grid = (unsigned)((m + rows - 1) / rows);
    switch (nv_bucket(d)) {
#define MMF_GB(NV) case NV: launch_k(gnorm_bwd_kernel<TG, NV>, grid, 256, 0, st, h, g, du, w, eps, m, d, rows, dh, dg, wpart); break;
        MMF_GB(1) MMF_GB(2) MMF_GB(4) MMF_GB(8)
#undef MMF_GB
    }
}

hipError_t launch_gnorm_bwd(const float *h, const void *g, ActType gt, const float *du, const float *w, float eps,
                            int64_t m, int d, float *dh, float *dg, float *wpart, hipStream_t st) {
    if (m <= 0) return hipSuccess;
    if (gt == ACT_F32) gnorm_bwd_t(h, static_cast<const float *>(g), du, w, eps, m, d, dh, dg, wpart, st);
    else gnorm_bwd_t(h, static_cast<const uint16_t *>(g), du, w, eps, m, d, dh, dg, wpart, st);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t st) {
    if (n > 0) launch_k(zero_f32_kernel, (unsigned)((n + 255) / 256), 256, 0, st, p, n);
    return hipGetLastError();
}

int gain_reduce_splits(int nblk) { return nblk < kGainSplits ? (nblk > 0 ? nblk : 1) : kGainSplits; }

hipError_t launch_gain_reduce(const float *gpart, int nblk, int k, float *part2, float *dgain, hipStream_t st) {
    const int splits = gain_reduce_splits(nblk);
    launch_k(gain_reduce_kernel, dim3((unsigned)((k + 63) / 64), (unsigned)splits), 256, 0, st, gpart, nblk, k, part2);
    launch_k(gain_final_kernel, (unsigned)((k + 255) / 256), 256, 0, st, part2, splits, k, dgain);
    return hipGetLastError();
}

}  // namespace mmf
