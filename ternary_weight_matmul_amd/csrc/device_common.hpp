// Device-side helpers shared by the gfx950 kernels of libmmf.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mmf {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---- activation element types -------------------------------------------------
// fp32 and bf16 (stored as raw uint16 bits). bf16 -> fp32 is exact; fp32 -> bf16
// rounds to nearest even (gfx950's v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float load_act(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_act(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void store_act(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void store_act(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

// Four consecutive elements starting at p[i] (i % 4 == 0).
__device__ __forceinline__ float4 load_act4(const float *p, int64_t i) {
    return *reinterpret_cast<const float4 *>(p + i);
}
__device__ __forceinline__ float4 load_act4(const uint16_t *p, int64_t i) {
    uint2 v = *reinterpret_cast<const uint2 *>(p + i);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}

// ---- LDS-DMA (global_load_lds_dwordx4) -----------------------------------------
// One 16-byte LDS-DMA load: lane L copies 16 bytes from src to LDS byte
// lds_base + 16 L (lds_base is wave-uniform). Written in asm so that the
// compiler's own wait insertion, which cannot tell which LDS bytes the load
// fills and so waits for it before any LDS read, leaves it alone; the kernel
// waits for it with an explicit vmcnt. The load has no register result, and
// M0 and the address registers are read when it issues. One wait state
// between the M0 write and the load.
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(src)
                 : "memory", "m0");
}

__device__ __forceinline__ void vmcnt_wait(int n) {
    // s_waitcnt with only the vector-memory counter constrained (expcnt 7, lgkmcnt 15 = no wait)
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
        case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
        case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
        case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// ---- wave reductions (wave64) -------------------------------------------------
// Within each row of 16 lanes: DPP quad permutes (xor 1, xor 2), half-row
// mirror and row mirror leave the row total in every lane of the row; the four
// row totals are then read out with readlane and combined in a fixed order.
// Every lane returns the same value.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) { return __int_as_float(dpp_i<CTRL>(__float_as_int(v))); }
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    return __hiloint2double(dpp_i<CTRL>(__double2hiint(v)), dpp_i<CTRL>(__double2loint(v)));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ double lane_d(double v, int lane) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                            __builtin_amdgcn_readlane(__double2loint(v), lane));
}

__device__ __forceinline__ double wave_sum(double v) {
    v += dpp_d<kDppXor1>(v);
    v += dpp_d<kDppXor2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    v += dpp_d<kDppMirror>(v);
    return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ __forceinline__ int wave_sum_int(int v) {
    v += dpp_i<kDppXor1>(v);
    v += dpp_i<kDppXor2>(v);
    v += dpp_i<kDppHalfMirror>(v);
    v += dpp_i<kDppMirror>(v);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// ---- activations ---------------------------------------------------------------
// sigmoid(z) = 1 / (1 + e^-z) with the hardware exp2 and reciprocal (about 2 ulp).
__device__ __forceinline__ float sigmoid_fast(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}
__device__ __forceinline__ float silu_fast(float z) { return z * sigmoid_fast(z); }

// ---- the row quantiser's binary32 decision steps ----------------------------------
// r = (float)(1 / sqrt(ss / k + eps)), binary64 inside.
__device__ __forceinline__ float rms_factor(double ss, int k, float eps) {
    return (float)(1.0 / sqrt(ss / (double)k + (double)eps));
}
// s = 127 / max(amax, 1e-5), a correctly rounded binary32 division.
__device__ __forceinline__ float quant_scale(float amax) {
    return __fdiv_rn(127.0f, fmaxf(amax, 1e-5f));
}
__device__ __forceinline__ int quant_code(float y, float s) {
    float p = rintf(__fmul_rn(y, s));
    p = fminf(fmaxf(p, -128.0f), 127.0f);
    return (int)p;
}
__device__ __forceinline__ uint32_t pack_codes4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// ---- ternary words ----------------------------------------------------------------
// A word holds 16 offset codes c = t + 1; (w >> 2j) & 0x03030303 gives the four
// codes of k = 4j .. 4j+3 as int8 lanes, so one word is one 16-byte MFMA operand.
__device__ __forceinline__ i32x4 decode_word(uint32_t w) {
    i32x4 r;
    r[0] = (int32_t)(w & 0x03030303u);
    r[1] = (int32_t)((w >> 2) & 0x03030303u);
    r[2] = (int32_t)((w >> 4) & 0x03030303u);
    r[3] = (int32_t)((w >> 6) & 0x03030303u);
    return r;
}

}  // namespace mmf
