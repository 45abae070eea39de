// Decode step of one HGRNBit block as one persistent kernel on one XCD (gfx950).
//
// A decode step ("MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，剩下什麼", section
// "HGRNBitBlock 的結構"; recurrence step from "MatMul-Free LLM 深度分析报告", table
// "创新之处") is eight dependent phases: quantise x -> i/f/g contraction with the
// gate and state update -> g_norm + quantise -> o_proj + residual -> quantise ->
// gate_proj + SiLU product -> quantise -> down_proj + residual. With a handful
// of rows every phase is short, so as separate kernels the step pays a kernel
// boundary (about 1.9 us on MI355X) eight times. A barrier across all eight
// XCDs costs more than that (arrivals, cache write-back and invalidation all go
// through memory); a barrier among the workgroups of ONE XCD, which share its
// L2, costs well under 1 us. So the whole step runs as one kernel on the 32
// CUs of XCD 0. The hardware deals a launch's workgroups to the XCDs
// round-robin by index, starting from an XCD that depends on earlier
// dispatches (checked once per device by the host: round-robin from any
// start); a workgroup reads its XCD from the XCC_ID hardware register, those
// on XCD 0 do the work with rank index / 8 (0..31 under that dealing) and the
// others return at once. One XCD streams the packed weights at about 1.3 TB/s.
//
// Coherence inside the launch: a workgroup's stores are complete (waitcnt)
// before it arrives at a barrier, and data that another workgroup wrote in an
// earlier phase of the launch is read with non-temporal loads, which do not
// return a cache line that may still hold an older copy.
//
// The arithmetic is that of the separate kernels: the row quantisers are the
// same functions (row_quant.hpp), the contractions sum exactly in int32 and
// share the epilogue (epilogue.hpp), so both paths give the same bits.
#include "device_common.hpp"
#include "launch.hpp"
#include "epilogue.hpp"
#include "row_quant.hpp"

#include <mutex>

namespace mmf {

constexpr int kXcdGroups = 32;                    // workgroups doing the work (the CUs of one XCD)
constexpr int kDecWaves = 16;                     // waves per workgroup
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kPartBytes = kDecWaves * 3 * 256 * 4;  // per-wave partial sums, up to three groups
constexpr long kSpinLimit = 1L << 20;             // about a second of polling (each poll reaches memory)

// Barrier state: arrivals, generation and expired spins, each on its own
// 256-byte line. Zero when the library loads; the arrival count stays a
// multiple of kXcdGroups (a power of two) between barriers.
__device__ unsigned g_xsync[3 * 64];

__device__ __forceinline__ unsigned ld_relaxed(const unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// XCD this workgroup runs on (hardware register XCC_ID, low four bits).
__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xF; }

// Barrier among the kXcdGroups working workgroups.
__device__ __forceinline__ void xcd_barrier() {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned *cnt = g_xsync, *gen = g_xsync + 64;
        const unsigned g0 = ld_relaxed(gen);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);  // the generation is read before this arrival counts
        asm volatile("" ::: "memory");
        const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (((old + 1) & (kXcdGroups - 1)) == 0) {
            __hip_atomic_fetch_add(gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            long spins = 0;
            while (ld_relaxed(gen) == g0) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins > kSpinLimit) {
                    __hip_atomic_fetch_add(g_xsync + 128, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
    }
    __syncthreads();
}

template <typename T>
__device__ __forceinline__ T ld_nt(const T *p) { return __builtin_nontemporal_load(p); }

// The epilogue's extra operand of output (r, c): old state, residual input or
// residual x1 (written in an earlier phase: non-temporal).
struct NoPre {
    __device__ float operator()(int64_t) const { return 0.0f; }
};
template <typename PT, bool NT>
struct PreFrom {
    const PT *p;
    __device__ float operator()(int64_t o) const {
        if constexpr (NT) return to_float(ld_nt(p + o));
        else return to_float(p[o]);
    }
    static __device__ float to_float(float v) { return v; }
    static __device__ float to_float(uint16_t v) { return bf16_to_f32(v); }
};

// One contraction phase: out[r][c] = epilogue(sum_k t[c][k] q[r][k]) for the
// rows r < b and the nc channels (NG groups). The codes of rows 0..15 are
// staged in LDS once (row stride K + 16 bytes: 16-byte reads of 16 rows fall in
// different banks). Blocks of 16 channels are dealt to the workgroups; four
// waves work on a block, wave q taking the 256-k chunks q, q + 4, ... (CPW at
// most), every weight load issued before its MFMAs; the four waves' partial
// sums meet in LDS and the block's 256 outputs take one thread each.
template <int NG, int EPI, int CPW, typename Pre>
__device__ __forceinline__ void gemv_phase(const ContractArgs &c, const uint32_t *const (&W)[3], const float *const (&mu)[3],
                                           const int8_t *codes, const float *s, const int32_t *sumq, int K, int b,
                                           int wg, char *lds_a, int32_t *part, const Pre &pre) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nc = c.nc;
    const int KW = K >> 4, nchunk = K >> 8;
    const int stride = K + 16;
    // stage the codes of rows 0..15 (rows past b repeat row b-1)
    const int per_row = K >> 4;  // 16-byte pieces per row
    for (int i = tid; i < 16 * per_row; i += kDecThreads) {
        const int r = i / per_row, p16 = i - r * per_row;
        const int rs = r < b ? r : b - 1;
        const i32x4 v = ld_nt(reinterpret_cast<const i32x4 *>(codes + (int64_t)rs * K) + p16);
        *reinterpret_cast<i32x4 *>(lds_a + r * stride + 16 * p16) = v;
    }
    __syncthreads();
    float sw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sw[g] = weight_sw(mu[g]);
    const int nblk = (nc + 15) >> 4;
    const int slot = wave >> 2, q = wave & 3;
    const int lc = lane & 15, lg = lane >> 4;
    const int t4 = (wave & 3) * 64 + lane;  // output of the block this thread finishes
    const int er = t4 >> 4, ec = t4 & 15;
    for (int first = wg; first < nblk; first += 4 * kXcdGroups) {
        const int blk = first + slot * kXcdGroups;
        const bool has = blk < nblk;
        const int ch = min(blk * 16 + lc, nc - 1);
        i32x4 acc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g] = i32x4{};
        if (has) {
            uint4 wv[NG][CPW];
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                const int cc = q + 4 * j;
                if (cc < nchunk)
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        wv[g][j] = *reinterpret_cast<const uint4 *>(W[g] + (int64_t)ch * KW + 16 * cc + 4 * lg);
            }
            const char *arow = lds_a + lc * stride + 64 * lg;
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                const int cc = q + 4 * j;
                if (cc < nchunk) {
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const i32x4 af = *reinterpret_cast<const i32x4 *>(arow + 256 * cc + 16 * qq);
#pragma unroll
                        for (int g = 0; g < NG; ++g) {
                            const uint32_t word = qq == 0 ? wv[g][j].x : qq == 1 ? wv[g][j].y : qq == 2 ? wv[g][j].z : wv[g][j].w;
                            acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, decode_word(word), acc[g], 0, 0, 0);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) part[(wave * NG + g) * 256 + (4 * lg + i) * 16 + lc] = acc[g][i];
        __syncthreads();
        const int oc = blk * 16 + ec;
        if (has && er < b && oc < nc) {
            int32_t v[NG];
            float dq[NG];
            const float srow = ld_nt(s + er);
            const int32_t sqrow = ld_nt(sumq + er);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                int32_t sum = 0;
#pragma unroll
                for (int w = 0; w < 4; ++w) sum += part[((slot * 4 + w) * NG + g) * 256 + er * 16 + ec];
                v[g] = sum - sqrow;
                dq[g] = __builtin_amdgcn_rcpf(srow * sw[g]);
            }
            epilogue_vals<EPI, NG, true>(c, er, oc, v, dq, pre((int64_t)er * nc + oc));
        }
        __syncthreads();
    }
}

template <typename T, int NVX, int NVZ, int CPWD, int CPWI>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(const DecodeStepArgs a) {
    if (xcc_id() != 0) return;  // only the workgroups of XCD 0 take part
    const int wg = blockIdx.x >> 3;
    extern __shared__ __attribute__((aligned(16))) char dyn[];
    __shared__ RowQuantLds sh;
    const int d = a.d, inner = a.inner, b = a.b;
    const int maxk = d > inner ? d : inner;
    char *lds_a = dyn;
    int32_t *part = reinterpret_cast<int32_t *>(dyn + 16 * (maxk + 16));
    const T *x = static_cast<const T *>(a.x);
    const ActType at = sizeof(T) == 4 ? ACT_F32 : ACT_BF16;

    // 1. RMSNorm + quantise x (one row per workgroup)
    if (wg < b)
        row_quant<T, NVX, false>(x + (int64_t)wg * d, d, a.gain_x, a.eps, a.codes + (int64_t)wg * d, a.s + wg,
                                 a.sumq + wg, sh);
    xcd_barrier();
    // 2. i/f/g: f = sigmoid, x~ = (1 - f) SiLU(i), h = f h + x~ (in place), g stored
    {
        ContractArgs c{};
        c.nc = d;
        c.out0 = a.h; c.out1 = a.g; c.out_type = ACT_F32; c.aux_type = at;
        const uint32_t *W[3] = {a.w_ifg[0], a.w_ifg[1], a.w_ifg[2]};
        const float *mu[3] = {a.mu_ifg[0], a.mu_ifg[1], a.mu_ifg[2]};
        gemv_phase<3, EPI_GATES_STEP, CPWD>(c, W, mu, a.codes, a.s, a.sumq, d, b, wg, lds_a, part,
                                            PreFrom<float, false>{a.h});
    }
    xcd_barrier();
    // 3. g_norm gate + o_proj's quantiser
    if (wg < b)
        row_gnorm_quant<T, NVX, true>(a.h + (int64_t)wg * d, static_cast<const T *>(a.g) + (int64_t)wg * d, d,
                                      a.g_norm_w, a.gain_o, a.eps, a.codes + (int64_t)wg * d, a.s + wg, a.sumq + wg,
                                      nullptr, sh);
    xcd_barrier();
    // 4. o_proj + residual: x1 = x + o (fp32)
    {
        ContractArgs c{};
        c.nc = d;
        c.out0 = a.x1; c.out_type = ACT_F32;
        const uint32_t *W[3] = {a.w_o, a.w_o, a.w_o};
        const float *mu[3] = {a.mu_o, a.mu_o, a.mu_o};
        gemv_phase<1, EPI_RESID, CPWD>(c, W, mu, a.codes, a.s, a.sumq, d, b, wg, lds_a, part, PreFrom<T, false>{x});
    }
    xcd_barrier();
    // 5. quantise x1
    if (wg < b)
        row_quant<float, NVX, true>(a.x1 + (int64_t)wg * d, d, a.gain_gate, a.eps, a.codes + (int64_t)wg * d,
                                    a.s + wg, a.sumq + wg, sh);
    xcd_barrier();
    // 6. gate_proj: z = SiLU(first half) * second half
    {
        ContractArgs c{};
        c.nc = inner;
        c.out0 = a.z; c.aux_type = at;
        const uint32_t *W[3] = {a.w_gate, a.w_gate + (int64_t)inner * (d >> 4), a.w_gate};
        const float *mu[3] = {a.mu_gate, a.mu_gate, a.mu_gate};
        gemv_phase<2, EPI_GLU, CPWD>(c, W, mu, a.codes, a.s, a.sumq, d, b, wg, lds_a, part, NoPre{});
    }
    xcd_barrier();
    // 7. quantise z
    if (wg < b)
        row_quant<T, NVZ, true>(static_cast<const T *>(a.z) + (int64_t)wg * inner, inner, a.gain_down, a.eps,
                                a.codes + (int64_t)wg * inner, a.s + wg, a.sumq + wg, sh);
    xcd_barrier();
    // 8. down_proj + residual: out = x1 + down (activation dtype)
    {
        ContractArgs c{};
        c.nc = d;
        c.out0 = a.out; c.out_type = at;
        const uint32_t *W[3] = {a.w_down, a.w_down, a.w_down};
        const float *mu[3] = {a.mu_down, a.mu_down, a.mu_down};
        gemv_phase<1, EPI_RESID, CPWI>(c, W, mu, a.codes, a.s, a.sumq, inner, b, wg, lds_a, part,
                                       PreFrom<float, true>{a.x1});
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// XCD of each workgroup of a probe launch (the placement check below)
constexpr int kXccMapGroups = 2048;
__device__ unsigned g_xccmap[kXccMapGroups];

__global__ void xcc_map_kernel(unsigned *out) {
    if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

// Whether workgroup i of a launch runs on XCD (i + o) % 8 for one start o,
// checked once per device (synchronously: never while the stream is being
// captured; until the check has run the separate kernels are used).
static bool xcd_layout_ok(hipStream_t st, std::string *why) {
    static std::mutex mu;
    static int state[64];  // 0 unknown, 1 yes, 2 no
    static std::string seen[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    std::lock_guard<std::mutex> lock(mu);
    if (state[dev]) {
        *why = seen[dev];
        return state[dev] == 1;
    }
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
        *why = "capturing";
        return false;
    }
    (void)hipGetLastError();
    bool ok = false;
    std::string note;
    unsigned *buf = nullptr;
    hipError_t e = hipGetSymbolAddress(reinterpret_cast<void **>(&buf), HIP_SYMBOL(g_xccmap));
    if (e == hipSuccess) {
        xcc_map_kernel<<<kXccMapGroups, 64, 0, st>>>(buf);
        unsigned host[kXccMapGroups];
        e = hipMemcpyAsync(host, buf, sizeof host, hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e == hipSuccess) {
            int bad = -1;
            for (int i = 0; i < kXccMapGroups; ++i)
                if (host[i] != (host[0] + i) % 8 && bad < 0) bad = i;
            ok = bad < 0;
            note = "xcc";
            for (int i = 0; i < 8; ++i) note += char('0' + (host[i] & 15));
            if (bad >= 0) note += ",first-mismatch@" + std::to_string(bad);
        }
    }
    if (e != hipSuccess) note = std::string("check:") + hipGetErrorName(e);
    seen[dev] = note;
    *why = note;
    state[dev] = ok ? 1 : 2;
    return ok;
}

struct DecodeVariant {
    int nvx, nvz, cpwd, cpwi;  // 256-thread chunks of a d row / inner row; 256-k chunks per wave for K = d / inner
    const void *f32, *bf16;
};

#define MMF_DEC_VARIANT(A, B, C, D)                                                                \
    {A, B, C, D, reinterpret_cast<const void *>(&decode_step_kernel<float, A, B, C, D>),            \
     reinterpret_cast<const void *>(&decode_step_kernel<uint16_t, A, B, C, D>)}
static const DecodeVariant kDecodeVariants[] = {
    MMF_DEC_VARIANT(1, 1, 1, 1), MMF_DEC_VARIANT(1, 2, 1, 2), MMF_DEC_VARIANT(1, 3, 1, 3),
    MMF_DEC_VARIANT(2, 6, 2, 6), MMF_DEC_VARIANT(3, 7, 3, 7),
};
#undef MMF_DEC_VARIANT

static const DecodeVariant *pick_variant(int d, int inner) {
    const int nvx = (d / 4 + 255) / 256, nvz = (inner / 4 + 255) / 256;
    const int cpwd = (d / 256 + 3) / 4, cpwi = (inner / 256 + 3) / 4;
    for (const auto &v : kDecodeVariants)
        if (v.nvx >= nvx && v.nvz >= nvz && v.cpwd >= cpwd && v.cpwi >= cpwi) return &v;
    return nullptr;
}

static size_t decode_lds_bytes(int d, int inner) {
    const int maxk = d > inner ? d : inner;
    return (size_t)16 * (maxk + 16) + kPartBytes;
}

bool decode_step_supported(int64_t b, int d, int inner) {
    return b >= 1 && b <= 16 && d % 256 == 0 && inner % 256 == 0 && pick_variant(d, inner) != nullptr &&
           decode_lds_bytes(d, inner) <= 160 * 1024;
}

hipError_t launch_decode_step(const DecodeStepArgs &a, hipStream_t st, std::string *path, bool *launched) {
    *launched = false;
    // a call that does not launch says why in the path string (no silent fallback)
    auto skip = [&](const char *why) {
        if (path) *path += std::string("decode_step_xcd_skipped(") + why + ");";
        return hipSuccess;
    };
    if (!decode_step_supported(a.b, a.d, a.inner)) return skip("shape");
    std::string why;
    if (!xcd_layout_ok(st, &why)) return skip(("placement:" + why).c_str());
    const DecodeVariant *v = pick_variant(a.d, a.inner);
    const void *fn = a.act == ACT_F32 ? v->f32 : v->bf16;
    const size_t lds = decode_lds_bytes(a.d, a.inner);
    hipError_t e = hipSuccess;
    {
        // dynamic LDS above the default limit is allowed per kernel, up to what its
        // static LDS leaves of the 160 KB; raised when a larger shape needs more
        constexpr int kNumFns = 2 * sizeof kDecodeVariants / sizeof kDecodeVariants[0];
        static std::mutex mu;
        static const void *fns[kNumFns];
        static size_t allowed[kNumFns];
        std::lock_guard<std::mutex> lock(mu);
        int slot = -1;
        for (int i = 0; i < kNumFns && slot < 0; ++i)
            if (fns[i] == fn || !fns[i]) slot = i;
        if (slot < 0) return hipErrorUnknown;
        if (!fns[slot] || allowed[slot] < lds) {
            hipFuncAttributes attr{};
            if ((e = hipFuncGetAttributes(&attr, fn)) != hipSuccess) return e;
            if (attr.sharedSizeBytes + lds > (size_t)160 * 1024) return skip("lds");
            if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
                return e;
            fns[slot] = fn;
            allowed[slot] = lds;
        }
    }
    // an ordinary launch: a cooperative one costs about 20 us more on MI355X.
    // The 32 working workgroups need 32 CUs at once; each needs most of a CU's
    // LDS, so XCD 0 holds exactly them while no other kernel runs there. Every
    // barrier wait is bounded: a violated assumption shows as an expired wait
    // (decode_step_expired_spins), never as a hang.
    DecodeStepArgs args = a;
    void *params[] = {&args};
    e = hipLaunchKernel(fn, dim3(8 * kXcdGroups), dim3(kDecThreads), params, lds, st);
    if (e == hipSuccess) {
        *launched = true;
        if (path) *path += "decode_step_xcd;";
    }
    return e;
}

hipError_t decode_step_expired_spins(unsigned *count) {
    return hipMemcpyFromSymbol(count, HIP_SYMBOL(g_xsync), sizeof(unsigned), 128 * sizeof(unsigned),
                               hipMemcpyDeviceToHost);
}

}  // namespace mmf
