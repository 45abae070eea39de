// Epilogues of the ternary contraction, shared by the prefill, decode and
// fused decode kernels: exact int32 sums -> dequantised values -> the fused
// elementwise step of the HGRNBit block (gates + recurrence step, residual,
// SiLU-gated MLP product).
#pragma once
#include "device_common.hpp"
#include "launch.hpp"

namespace mmf {

__device__ __forceinline__ float load_any(const void *p, ActType t, int64_t i) {
    return t == ACT_F32 ? static_cast<const float *>(p)[i] : bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
}
__device__ __forceinline__ void store_any(void *p, ActType t, int64_t i, float v) {
    if (t == ACT_F32)
        static_cast<float *>(p)[i] = v;
    else
        static_cast<uint16_t *>(p)[i] = f32_to_bf16(v);
}

__device__ __forceinline__ float weight_sw(const float *mu) { return __fdiv_rn(1.0f, fmaxf(*mu, 1e-5f)); }

// v[g] = exact sum t*q of output (m, c) for group g; dq[g] = 1 / (s * sw).
template <int EPI, int NG>
__device__ __forceinline__ void epilogue_vals(const ContractArgs &p, int64_t m, int c, const int32_t (&v)[NG],
                                              const float (&dq)[NG]) {
    float y[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        y[g] = (float)v[g] * dq[g];
        if (p.acc_probe) p.acc_probe[m * (int64_t)(NG * p.nc) + (int64_t)g * p.nc + c] = v[g];
    }
    const int64_t o = m * (int64_t)p.nc + c;
    if constexpr (EPI == EPI_LINEAR) {
        store_any(p.out0, p.out_type, o, y[0]);
    } else if constexpr (EPI == EPI_RESID) {
        const float r = load_any(p.res, p.res_type, o);
        store_any(p.out0, p.out_type, o, r + y[0]);
    } else if constexpr (EPI == EPI_GATES) {
        const float f = sigmoid_fast(y[1]);
        const float xt = (1.0f - f) * silu_fast(y[0]);
        static_cast<float *>(p.out0)[o] = f;
        static_cast<float *>(p.out1)[o] = xt;
        static_cast<float *>(p.out2)[o] = y[2];
    } else if constexpr (EPI == EPI_GATES_STEP) {
        const float f = sigmoid_fast(y[1]);
        const float xt = (1.0f - f) * silu_fast(y[0]);
        float *h = static_cast<float *>(p.out0);
        h[o] = f * h[o] + xt;
        static_cast<float *>(p.out1)[o] = y[2];
        if (p.out2) static_cast<float *>(p.out2)[o] = f;
        if (p.out3) static_cast<float *>(p.out3)[o] = xt;
    } else if constexpr (EPI == EPI_GLU) {
        static_cast<float *>(p.out0)[o] = silu_fast(y[0]) * y[1];
    }
}

// raw[g] = sum c*q of output (m, c) for group g (offset codes). Corrects by
// sum q, dequantises with 1 / (s * sw) and applies the epilogue.
template <int EPI, int NG>
__device__ __forceinline__ void epilogue(const ContractArgs &p, const float (&sw)[3], int64_t m, int c,
                                         const int32_t (&raw)[NG]) {
    int32_t v[NG];
    float dq[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        v[g] = raw[g] - p.sumq[g][m];
        dq[g] = __builtin_amdgcn_rcpf(p.s[g][m] * sw[g]);
    }
    epilogue_vals<EPI, NG>(p, m, c, v, dq);
}

}  // namespace mmf
