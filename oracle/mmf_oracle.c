/*
 * CPU oracle for the HGRNBit layer forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
 * this file. It shares no code, header or constant generator with the HIP
 * library; it is written straight from the definitions it cites, as plain loops.
 *
 * Sources (web pages about the MatMul-free LM project):
 *   [R1] "MatMul-Free LLM 深度分析报告" (nightvoyager.top), section
 *        "核心价值提炼": table "创新之处" (ternary weight_quant, round to nearest
 *        {-1,0,+1}; HGRN recurrence) and list "可复用的模式与技巧" (RMSNorm fused
 *        with INT8 quantisation inside FusedBitLinear).
 *   [R3] "MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，剩下什麼" (hysenlabs.com),
 *        section "HGRNBitBlock 的結構": every FusedBitLinear carries an RMSNorm
 *        with eps = 1e-8.
 *   [R4] mooersco.com article, section 4.1 (a ternary GEMV is a conditional
 *        add / subtract per weight) and section 5.1 (branch-free form).
 * Readings where the pages are silent (absmax scale 127, the 1e-5 floors,
 * per-tensor mean-|W| weight scale, round-half-to-even) are the project's
 * stated problem, not the pages; each is named where it is used.
 *
 * Precision: the quantisers decide integers, so they run in the kernel's
 * precision (binary32, one rounding per *, /), with the sum of squares and the
 * reciprocal square root taken in binary64. Build with -ffp-contract=off and
 * no fast-math so that every binary32 operation is rounded on its own.
 * The integer contraction is exact (accumulated in int64, checked to fit int32).
 * The recurrence is binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Row-wise RMSNorm + absmax int8 quantiser ([R1] fused RMSNorm + INT8 quant;
 * [R3] eps on the RMSNorm).
 *   ss   = sum_k v_k^2                    (binary64, k in increasing order)
 *   r    = (float)(1 / sqrt(ss/K + eps))  (binary64, rounded once to binary32)
 *   y_k  = (v_k * r) * gain_k             (binary32; the gain product is skipped when gain is NULL)
 *   amax = max_k |y_k|
 *   s    = 127 / max(amax, 1e-5)          (binary32)
 *   q_k  = clamp(rint(y_k * s), -128, 127), rint = round half to even
 *   sumq = sum_k q_k
 * Returns 0, or -1 on bad arguments.
 */
int oracle_quant_rows(const float *v, int64_t m, int64_t k, const float *gain, float eps,
                      int8_t *q, float *s, int32_t *sumq)
{
    if (!v || !q || !s || !sumq || m < 0 || k <= 0) return -1;
    for (int64_t i = 0; i < m; ++i) {
        const float *row = v + i * k;
        double ss = 0.0;
        for (int64_t j = 0; j < k; ++j) ss += (double)row[j] * (double)row[j];
        float r = (float)(1.0 / sqrt(ss / (double)k + (double)eps));
        float amax = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            float y = row[j] * r;
            if (gain) y = y * gain[j];
            float a = fabsf(y);
            if (a > amax) amax = a;
        }
        float sc = 127.0f / fmaxf(amax, 1e-5f);
        int32_t total = 0;
        for (int64_t j = 0; j < k; ++j) {
            float y = row[j] * r;
            if (gain) y = y * gain[j];
            float p = rintf(y * sc);
            if (p > 127.0f) p = 127.0f;
            if (p < -128.0f) p = -128.0f;
            q[i * k + j] = (int8_t)p;
            total += (int32_t)p;
        }
        s[i] = sc;
        sumq[i] = total;
    }
    return 0;
}

/*
 * Ternary weight quantisation ([R1] weight_quant: round to nearest {-1,0,+1};
 * per-tensor mean-|W| scale is the stated problem's reading).
 *   mu = (float)(sum |W| / (N*K))       (binary64 sum in index order)
 *   sw = 1 / max(mu, 1e-5)              (binary32)
 *   t  = clamp(rint(W * sw), -1, 1)     (binary32 product, round half to even)
 */
int oracle_ternarize(const float *w, int64_t n, int64_t k, int8_t *t, float *mu)
{
    if (!w || !t || !mu || n <= 0 || k <= 0) return -1;
    const int64_t count = n * k;
    double acc = 0.0;
    for (int64_t i = 0; i < count; ++i) acc += fabs((double)w[i]);
    float m = (float)(acc / (double)count);
    float sw = 1.0f / fmaxf(m, 1e-5f);
    for (int64_t i = 0; i < count; ++i) {
        float p = rintf(w[i] * sw);
        if (p > 1.0f) p = 1.0f;
        if (p < -1.0f) p = -1.0f;
        t[i] = (int8_t)p;
    }
    *mu = m;
    return 0;
}

/*
 * 2-bit packing ([R4] section 5.1 suggests packing low-bit weights and
 * processing many per word). The code stored is c = t + 1 in {0,1,2}.
 * Word w of row n covers k = 16w .. 16w+15; ternary k = 16w + 4j + b sits at
 * bits [8b + 2j, 8b + 2j + 2) for j, b in 0..3. K must be a multiple of 16.
 */
int oracle_pack(const int8_t *t, int64_t n, int64_t k, uint32_t *words)
{
    if (!t || !words || n <= 0 || k <= 0 || (k % 16) != 0) return -1;
    const int64_t kw = k / 16;
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t w = 0; w < kw; ++w) {
            uint32_t word = 0;
            for (int j = 0; j < 4; ++j) {
                for (int b = 0; b < 4; ++b) {
                    int8_t tv = t[row * k + 16 * w + 4 * j + b];
                    if (tv < -1 || tv > 1) return -1;
                    uint32_t c = (uint32_t)(tv + 1);
                    word |= c << (8 * b + 2 * j);
                }
            }
            words[row * kw + w] = word;
        }
    }
    return 0;
}

/* Inverse of oracle_pack; returns -1 on a code 3 (not a valid ternary). */
int oracle_unpack(const uint32_t *words, int64_t n, int64_t k, int8_t *t)
{
    if (!t || !words || n <= 0 || k <= 0 || (k % 16) != 0) return -1;
    const int64_t kw = k / 16;
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t kk = 0; kk < k; ++kk) {
            int64_t w = kk / 16, j = (kk % 16) / 4, b = kk % 4;
            uint32_t c = (words[row * kw + w] >> (8 * b + 2 * j)) & 3u;
            if (c == 3u) return -1;
            t[row * k + kk] = (int8_t)((int)c - 1);
        }
    }
    return 0;
}

/*
 * Exact ternary contraction ([R4] section 4.1: per weight, add the input when
 * the weight is +1, subtract it when -1, skip it when 0):
 *   acc[i][o] = sum_k q[i][k] * t[o][k]
 * Accumulated in int64; returns -2 if a result does not fit int32.
 * Independent outputs are spread over OpenMP threads; each output is summed
 * in increasing k by one thread.
 */
int oracle_ternary_matmul(const int8_t *q, const int8_t *t, int64_t m, int64_t n, int64_t k,
                          int32_t *acc)
{
    if (!q || !t || !acc || m < 0 || n <= 0 || k <= 0) return -1;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t o = 0; o < n; ++o) {
            const int8_t *qi = q + i * k;
            const int8_t *to = t + o * k;
            int64_t sum = 0;
            for (int64_t kk = 0; kk < k; ++kk) {
                if (to[kk] == 1) sum += qi[kk];
                else if (to[kk] == -1) sum -= qi[kk];
            }
            if (sum > INT32_MAX || sum < INT32_MIN) bad = 1;
            acc[i * n + o] = (int32_t)sum;
        }
    }
    return bad ? -2 : 0;
}

/*
 * HGRN recurrence ([R1] table "创新之处": h_t = gate_t * h_{t-1} + x_t, elementwise,
 * O(T*D)), binary64, sequential in t for every (batch, channel):
 *   h[b][t][c] = f[b][t][c] * h[b][t-1][c] + x[b][t][c],  h[b][-1][c] = h0[b][c] (0 if h0 is NULL)
 */
int oracle_hgrn_scan(const double *x, const double *f, const double *h0, int64_t b, int64_t t,
                     int64_t d, double *h)
{
    if (!x || !f || !h || b < 0 || t < 0 || d <= 0) return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bi = 0; bi < b; ++bi) {
        for (int64_t c = 0; c < d; ++c) {
            double state = h0 ? h0[bi * d + c] : 0.0;
            for (int64_t s = 0; s < t; ++s) {
                int64_t idx = (bi * t + s) * d + c;
                state = f[idx] * state + x[idx];
                h[idx] = state;
            }
        }
    }
    return 0;
}

/*
 * Derivative of the recurrence above, binary64. A loss L sees h through
 * dL/dh[b][t][c] = dh and dL/dh_last[b][c] = dh_last (NULL: 0). With D_t the
 * whole derivative of L with respect to h_t (directly, and through h_{t+1},
 * which holds f_{t+1} * h_t):
 *   D_{T-1} = dh_{T-1} + dh_last,   D_t = dh_t + f_{t+1} * D_{t+1}
 *   dx_t = D_t,   df_t = D_t * h_{t-1},   dh0 = f_0 * D_0      (h_{-1} = h0 or 0)
 * taken for t = T-1 down to 0. dh0 may be NULL; with t = 0, dh0 = dh_last.
 */
int oracle_hgrn_scan_bwd(const double *f, const double *h, const double *h0, const double *dh,
                         const double *dh_last, int64_t b, int64_t t, int64_t d, double *dx, double *df,
                         double *dh0)
{
    if (b < 0 || t < 0 || d <= 0) return -1;
    if (t > 0 && (!f || !h || !dh || !dx || !df)) return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bi = 0; bi < b; ++bi) {
        for (int64_t c = 0; c < d; ++c) {
            double total = dh_last ? dh_last[bi * d + c] : 0.0;  /* D_{t+1} times nothing yet */
            for (int64_t s = t - 1; s >= 0; --s) {
                int64_t idx = (bi * t + s) * d + c;
                double f_next = (s + 1 < t) ? f[idx + d] : 1.0;
                double h_prev = (s > 0) ? h[idx - d] : (h0 ? h0[bi * d + c] : 0.0);
                total = dh[idx] + f_next * total;
                dx[idx] = total;
                df[idx] = total * h_prev;
            }
            if (dh0) dh0[bi * d + c] = (t > 0) ? f[(bi * t) * d + c] * total : total;
        }
    }
    return 0;
}

/* Number of OpenMP threads the parallel loops above use (1 without OpenMP). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
