// Epilogues of the ternary contraction, shared by the prefill and decode
// kernels: exact int32 sums -> dequantised values -> the fused
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

// g / z output in its storage type, with the optional fp32 copy of the stored value
__device__ __forceinline__ void store_aux(const ContractArgs &p, void *dst, int64_t o, float v) {
    if (p.aux_type == ACT_F32) {
        static_cast<float *>(dst)[o] = v;
        if (p.aux_probe) p.aux_probe[o] = v;
    } else {
        const uint16_t b = f32_to_bf16(v);
        static_cast<uint16_t *>(dst)[o] = b;
        if (p.aux_probe) p.aux_probe[o] = bf16_to_f32(b);
    }
}

__device__ __forceinline__ float weight_sw(const float *mu) { return __fdiv_rn(1.0f, fmaxf(*mu, 1e-5f)); }

// v[g] = exact sum t*q of output (m, c) for group g; dq[g] = 1 / (s * sw).
// With PRE, `pre` already holds the residual (EPI_RESID) or the old state
// (EPI_GATES_STEP) of this output, loaded early by the caller.
template <int EPI, int NG, bool PRE = false>
__device__ __forceinline__ void epilogue_vals(const ContractArgs &p, int64_t m, int c, const int32_t (&v)[NG],
                                              const float (&dq)[NG], float pre = 0.0f) {
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
        const float r = PRE ? pre : load_any(p.res, p.res_type, o);
        store_any(p.out0, p.out_type, o, r + y[0]);
    } else if constexpr (EPI == EPI_GATES) {
        const float f = sigmoid_fast(y[1]);
        const float xt = (1.0f - f) * silu_fast(y[0]);
        static_cast<float *>(p.out0)[o] = f;
        static_cast<float *>(p.out1)[o] = xt;
        store_aux(p, p.out2, o, y[2]);
    } else if constexpr (EPI == EPI_GATES_STEP) {
        const float f = sigmoid_fast(y[1]);
        const float xt = (1.0f - f) * silu_fast(y[0]);
        float *h = static_cast<float *>(p.out0);
        // one fused multiply-add on the rounded x~, as the scan's step does: written out so that
        // every kernel instantiating this epilogue rounds the same way
        h[o] = __fmaf_rn(f, PRE ? pre : h[o], xt);
        store_aux(p, p.out1, o, y[2]);
        if (p.out2) static_cast<float *>(p.out2)[o] = f;
        if (p.out3) static_cast<float *>(p.out3)[o] = xt;
    } else if constexpr (EPI == EPI_GLU) {
        store_aux(p, p.out0, o, silu_fast(y[0]) * y[1]);
    }
}

}  // namespace mmf
