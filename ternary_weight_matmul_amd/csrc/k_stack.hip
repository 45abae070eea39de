// Decode step of a whole stack of HGRNBit blocks as one persistent kernel (gfx950).
//
// One token per sequence through every block of the stack ("MatMul-Free LM：把
// 矩陣乘法從語言模型裡拿掉之後，剩下什麼", section "HGRNBitBlock 的結構": the blocks
// are stacked, each i/f/g/o FusedBitLinear plus g_norm plus the SiLU-gated MLP;
// the step-wise recurrence from "MatMul-Free LLM 深度分析报告", table "创新之处" and
// list "可复用的模式与技巧", fused_recurrent for generation). A block's step is
// eight dependent phases: quantise x -> i/f/g contraction with the gates and
// the state update -> g_norm + quantise -> o_proj + residual -> quantise ->
// gate_proj + SiLU product -> quantise -> down_proj + residual. Here all of
// them, for every block, run in one launch: the phases are separated by
// barriers across the whole grid. A barrier is split into an arrival and a
// wait; between the two halves of the barrier that ends a contraction, every
// wave issues the loads of its packed weights for the next contraction, so
// they stream in during that barrier and the quantiser phase after it.
//
// The launch is cooperative: all workgroups (64, one CU each) are resident
// together, or the launch fails, so a barrier cannot wait for a workgroup that
// was never scheduled. Every wait is still bounded: a wait that expires
// raises the launch's abort word and a library-wide count
// (stack_decode_expired_waits), every workgroup then leaves at its next
// barrier, and each writes NaN over the whole output, so an expired wait
// never yields a plausible result.
//
// Coherence across the XCDs (each has its own L2): a workgroup's stores are
// complete before it arrives (waitcnt in every wave, then a workgroup
// barrier), the arrival is a release at device scope (the L2 writes back its
// dirty lines), and after the wait an acquire at device scope invalidates
// the stale lines; the arrival counters are device-scope atomics in groups of
// 32 workgroups so no single counter takes every arrival.
//
// The arithmetic is that of the per-block kernels: the row quantisers are the
// same functions (row_quant.hpp), the contractions sum exactly in int32 and
// share the epilogue (epilogue.hpp), so the stack step gives the bits of a
// chain of per-block decode steps.
#include "device_common.hpp"
#include "launch.hpp"
#include "epilogue.hpp"
#include "row_quant.hpp"
#include "stack.hpp"

#include <atomic>
#include <mutex>

namespace mmf {

constexpr int kStkWaves = 8;
constexpr int kStkThreads = kStkWaves * 64;
constexpr int kStkPartBytes = kStkWaves * 3 * 256 * 4;  // per-wave partial sums, up to three groups
constexpr int kStkGroup = 32;                            // workgroups per arrival counter
constexpr long kStkSpinLimit = 1L << 21;                 // polls before a wait is given up (about a second)
// Workgroups of a launch: 8 per XCD on MI355X. A barrier's cost grows with the
// arrivals (measured with release and acquire: 1.9 / 3.0 / 3.9 / 5.8 us at 32 /
// 64 / 128 / 256 workgroups), and the 1.3B stack step was fastest at 64 (60 / 64
// us per layer at batch 1 / 16, against 80 with a workgroup on every CU): fewer
// workgroups stream the weights more slowly, more wait longer at each barrier.
constexpr int kStkGrid = 64;
// 16-channel blocks per workgroup and round in the contractions (i/f/g and
// o_proj, gate_proj, down_proj). More blocks per workgroup (every contraction
// of the 1.3B block in one round at 64 workgroups) held more weight registers
// across the quantiser phases than a 512-thread workgroup has: the kernel
// spilled to scratch in every such geometry tried.
constexpr int kSlotsD = 1, kSlotsG = 2, kSlotsI = 1;

// Barrier words, each on its own 256-byte line (zeroed before every launch).
enum { BAR_GROUPS = 0, BAR_TOP = 16 * 64, BAR_GEN = 17 * 64, BAR_ABORT = 18 * 64 };

// Waits that expired in any launch since the library was loaded.
__device__ unsigned g_stack_expired;

__device__ __forceinline__ unsigned ld_agent(const unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier across the grid in two halves, so that loads which do not depend on
// it can be issued between them: barrier_arrive (every wave's stores complete,
// then thread 0 counts the workgroup in, with release at device scope) and
// barrier_wait (thread 0 polls the generation word, then acquires at device
// scope). Thread 0 keeps the generation it has passed in *gen_local.
// barrier_wait returns false (in every thread) once the launch is aborted.
__device__ __forceinline__ void barrier_arrive(unsigned *bar, int nwg, unsigned gen_local) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const int wg = blockIdx.x, grp = wg / kStkGroup, ngrp = (nwg + kStkGroup - 1) / kStkGroup;
        const int gsize = min(kStkGroup, nwg - grp * kStkGroup);
        // release: this workgroup's stores (complete in L2) are written back before the arrival counts
        const unsigned old = __hip_atomic_fetch_add(bar + BAR_GROUPS + 64 * grp, 1u, __ATOMIC_RELEASE,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1 == (unsigned)gsize) {
            // last of its group: reset the group counter, then count the group
            __hip_atomic_store(bar + BAR_GROUPS + 64 * grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const unsigned top = __hip_atomic_fetch_add(bar + BAR_TOP, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            if (top + 1 == (unsigned)ngrp) {
                __hip_atomic_store(bar + BAR_TOP, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(bar + BAR_GEN, gen_local + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

__device__ __forceinline__ bool barrier_wait(unsigned *bar, unsigned *gen_local, int *flag) {
    if (threadIdx.x == 0) {
        const unsigned g0 = *gen_local;
        int ok = 1;
        long spins = 0;
        while (true) {
            if (ld_agent(bar + BAR_GEN) != g0) break;
            if (ld_agent(bar + BAR_ABORT)) { ok = 0; break; }
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kStkSpinLimit) {
                __hip_atomic_fetch_add(&g_stack_expired, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(bar + BAR_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // lines older than the other workgroups' stores are dropped
        *gen_local = g0 + 1;
        *flag = ok;
    }
    __syncthreads();
    return *flag != 0;
}

// The packed-weight words a wave contracts in one round of a contraction
// phase: NG groups x CPW 256-k chunks of its 16-channel block.
template <int NG, int CPW>
struct WeightRegs {
    uint4 w[NG][CPW];
};

// Geometry of a contraction phase: SLOTS 16-channel blocks per workgroup and
// round, WPB = kStkWaves / SLOTS waves per block, wave q of a block taking the
// 256-k chunks q, q + WPB, ... (CPW at most).
template <int SLOTS>
struct PhaseGeom {
    static constexpr int WPB = kStkWaves / SLOTS;
    int slot, q, lc, lg;
    __device__ PhaseGeom() {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        slot = wave / WPB;
        q = wave % WPB;
        lc = lane & 15;
        lg = lane >> 4;
    }
};

// Issue the weight loads of this wave for the round of a contraction phase
// that workgroup position wg takes (block wg * SLOTS + slot; wg + round * nwg
// in later rounds); nothing is loaded for a block past the end.
template <int NG, int CPW, int SLOTS>
__device__ __forceinline__ void load_weights(WeightRegs<NG, CPW> &r, const uint32_t *const (&W)[3], int nc, int K,
                                             int wg) {
    const PhaseGeom<SLOTS> gm;
    const int blk = wg * SLOTS + gm.slot;
    constexpr int WPB = PhaseGeom<SLOTS>::WPB;
    const int nblk = (nc + 15) >> 4, nchunk = K >> 8, KW = K >> 4;
    if (blk >= nblk) return;
    const int ch = min(blk * 16 + gm.lc, nc - 1);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const int cc = gm.q + WPB * j;
        if (cc < nchunk)
#pragma unroll
            for (int g = 0; g < NG; ++g)
                r.w[g][j] = *reinterpret_cast<const uint4 *>(W[g] + (int64_t)ch * KW + 16 * cc + 4 * gm.lg);
    }
}

// The epilogue's extra operand of output (r, c): old state or residual.
struct NoPre {
    __device__ float operator()(int64_t) const { return 0.0f; }
};
template <typename PT>
struct PreFrom {
    const PT *p;
    __device__ float operator()(int64_t o) const { return load_act(p, o); }
};

// One contraction phase: out[r][c] = epilogue(sum_k t[c][k] q[r][k]) for the
// rows r < b and the nc channels (NG groups). The codes of rows 0..15 are
// staged in LDS once (row stride K + 16 bytes, so 16-byte reads of the 16
// rows fall in different banks); each wave's MFMAs read their activation
// fragments from there; the block's waves meet in LDS and the block's 256
// outputs are finished by its waves' threads. `pre` holds the weights of the
// first round, loaded before the barrier that opened the phase.
template <int NG, int EPI, int SLOTS, int CPW, typename Pre>
__device__ __forceinline__ void gemv_phase(const ContractArgs &c, const uint32_t *const (&W)[3],
                                           const float *const (&mu)[3], const int8_t *codes, const float *s,
                                           const int32_t *sumq, int K, int b, int wg, int nwg, char *lds_a,
                                           int32_t *part, const Pre &pre, WeightRegs<NG, CPW> &first) {
    constexpr int WPB = PhaseGeom<SLOTS>::WPB;
    const PhaseGeom<SLOTS> gm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nc = c.nc, nchunk = K >> 8, stride = K + 16;
    const int nblk = (nc + 15) >> 4;
    if (wg * SLOTS >= nblk) return;  // no block for this workgroup (uniform)
    // stage the codes of rows 0..15 (rows past b repeat row b-1)
    const int per_row = K >> 4;  // 16-byte pieces per row
    for (int i = tid; i < 16 * per_row; i += kStkThreads) {
        const int r = i / per_row, p16 = i - r * per_row;
        const int rs = r < b ? r : b - 1;
        const i32x4 v = reinterpret_cast<const i32x4 *>(codes + (int64_t)rs * K)[p16];
        *reinterpret_cast<i32x4 *>(lds_a + r * stride + 16 * p16) = v;
    }
    float sw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sw[g] = weight_sw(mu[g]);
    __syncthreads();
    bool first_round = true;
    for (int base = wg * SLOTS; base < nblk; base += nwg * SLOTS) {
        const int blk = base + gm.slot;
        const bool has = blk < nblk;
        WeightRegs<NG, CPW> r;
        if (first_round) r = first;
        else load_weights<NG, CPW, SLOTS>(r, W, nc, K, base / SLOTS);  // base = (wg + round * nwg) * SLOTS
        first_round = false;
        i32x4 acc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g] = i32x4{};
        if (has) {
            const char *arow = lds_a + gm.lc * stride + 64 * gm.lg;
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                const int cc = gm.q + WPB * j;
                if (cc < nchunk) {
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const i32x4 af = *reinterpret_cast<const i32x4 *>(arow + 256 * cc + 16 * qq);
#pragma unroll
                        for (int g = 0; g < NG; ++g) {
                            const uint4 wv = r.w[g][j];
                            const uint32_t word = qq == 0 ? wv.x : qq == 1 ? wv.y : qq == 2 ? wv.z : wv.w;
                            acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, decode_word(word), acc[g], 0, 0, 0);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) part[(wave * NG + g) * 256 + (4 * gm.lg + i) * 16 + gm.lc] = acc[g][i];
        __syncthreads();
        for (int o = gm.q * 64 + lane; o < 256; o += 64 * WPB) {
            const int er = o >> 4, ec = o & 15;
            const int oc = blk * 16 + ec;
            if (has && er < b && oc < nc) {
                int32_t v[NG];
                float dq[NG];
                const float srow = s[er];
                const int32_t sqrow = sumq[er];
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    int32_t sum = 0;
#pragma unroll
                    for (int w = 0; w < WPB; ++w) sum += part[((gm.slot * WPB + w) * NG + g) * 256 + er * 16 + ec];
                    v[g] = sum - sqrow;
                    dq[g] = __builtin_amdgcn_rcpf(srow * sw[g]);
                }
                epilogue_vals<EPI, NG, true>(c, er, oc, v, dq, pre((int64_t)er * nc + oc));
            }
        }
        __syncthreads();
    }
}

// Every workgroup of an aborted launch writes NaN over the whole output.
template <typename T>
__device__ void poison_output(T *out, int64_t n) {
    const uint32_t nan = 0x7FC00000u;
    for (int64_t i = threadIdx.x; i < n; i += kStkThreads) {
        if constexpr (sizeof(T) == 4) reinterpret_cast<uint32_t *>(out)[i] = nan;
        else reinterpret_cast<uint16_t *>(out)[i] = (uint16_t)(nan >> 16);
    }
}

// Phase geometry of the four contractions: i/f/g and o_proj kSlotsD 16-channel
// blocks per workgroup, gate_proj kSlotsG, down_proj kSlotsI, the waves of a
// workgroup split evenly between its blocks. CDA, CDH, CIA: 256-k chunks per
// wave for K = d in i/f/g and o_proj, K = d in gate_proj and K = inner in
// down_proj. The
// weights of a contraction are loaded between the two halves of the barrier
// that ends the contraction before it, so they arrive during the quantiser
// phase in between.
template <typename T, int NVX, int NVZ, int CDA, int CDH, int CIA>
__global__ __launch_bounds__(kStkThreads) void stack_decode_kernel(const StackArgs a) {
    extern __shared__ __attribute__((aligned(16))) char dyn[];
    __shared__ RowQuantLds sh;
    __shared__ int flag;
    unsigned gen_local = 0;
    const int wg = blockIdx.x, nwg = gridDim.x;
    const int d = a.d, inner = a.inner, b = a.b;
    const int maxk = d > inner ? d : inner;
    char *lds_a = dyn;
    int32_t *part = reinterpret_cast<int32_t *>(dyn + 16 * (maxk + 16));
    const ActType at = sizeof(T) == 4 ? ACT_F32 : ACT_BF16;
    T *out_final = static_cast<T *>(a.out);
    auto wait = [&]() {
        if (barrier_wait(a.bar, &gen_local, &flag)) return true;
        poison_output(out_final, (int64_t)b * d);
        return false;
    };
    auto arrive = [&]() { barrier_arrive(a.bar, nwg, gen_local); };

    WeightRegs<3, CDA> wifg;
    {
        const StackLayer &L0 = a.layers[0];
        const uint32_t *W[3] = {L0.w[0], L0.w[1], L0.w[2]};
        load_weights<3, CDA, kSlotsD>(wifg, W, d, d, wg);
    }
    for (int l = 0; l < a.n_layers; ++l) {
        const StackLayer &L = a.layers[l];
        const T *x = l == 0 ? static_cast<const T *>(a.x) : static_cast<const T *>(a.act[(l - 1) & 1]);
        T *out = l == a.n_layers - 1 ? out_final : static_cast<T *>(a.act[l & 1]);
        const float eps = L.eps;
        const int8_t *codes = a.codes;
        const uint32_t *Wifg[3] = {L.w[0], L.w[1], L.w[2]};
        const float *Mifg[3] = {L.mu[0], L.mu[1], L.mu[2]};
        const uint32_t *Wo[3] = {L.w[3], L.w[3], L.w[3]};
        const float *Mo[3] = {L.mu[3], L.mu[3], L.mu[3]};
        const uint32_t *Wg[3] = {L.w[4], L.w[4] + (int64_t)inner * (d >> 4), L.w[4]};
        const float *Mg[3] = {L.mu[4], L.mu[4], L.mu[4]};
        const uint32_t *Wd[3] = {L.w[5], L.w[5], L.w[5]};
        const float *Md[3] = {L.mu[5], L.mu[5], L.mu[5]};

        // 1. RMSNorm + quantise x (one row per workgroup)
        if (wg < b)
            row_quant<T, NVX, false>(x + (int64_t)wg * d, d, L.gain[0], eps, a.codes + (int64_t)wg * d, a.s + wg,
                                     a.sumq + wg, sh);
        arrive();
        if (!wait()) return;
        // 2. i/f/g: f = sigmoid, x~ = (1 - f) SiLU(i), h = f h + x~ (in place), g kept in fp32
        {
            ContractArgs c{};
            c.nc = d;
            c.out0 = L.h; c.out1 = a.g; c.out_type = ACT_F32; c.aux_type = ACT_F32;
            gemv_phase<3, EPI_GATES_STEP, kSlotsD, CDA>(c, Wifg, Mifg, codes, a.s, a.sumq, d, b, wg, nwg, lds_a, part,
                                                   PreFrom<float>{L.h}, wifg);
        }
        arrive();
        WeightRegs<1, CDA> wo;
        load_weights<1, CDA, kSlotsD>(wo, Wo, d, d, wg);
        if (!wait()) return;
        // 3. g_norm gate + o_proj's quantiser
        if (wg < b)
            row_gnorm_quant<float, NVX, false>(L.h + (int64_t)wg * d, a.g + (int64_t)wg * d, d, L.g_norm_w,
                                               L.gain[3], eps, a.codes + (int64_t)wg * d, a.s + wg, a.sumq + wg,
                                               nullptr, sh);
        arrive();
        if (!wait()) return;
        // 4. o_proj + residual: x1 = x + o (fp32)
        {
            ContractArgs c{};
            c.nc = d;
            c.out0 = a.x1; c.out_type = ACT_F32;
            gemv_phase<1, EPI_RESID, kSlotsD, CDA>(c, Wo, Mo, codes, a.s, a.sumq, d, b, wg, nwg, lds_a, part,
                                              PreFrom<T>{x}, wo);
        }
        arrive();
        WeightRegs<2, CDH> wgt;
        load_weights<2, CDH, kSlotsG>(wgt, Wg, inner, d, wg);
        if (!wait()) return;
        // 5. quantise x1
        if (wg < b)
            row_quant<float, NVX, false>(a.x1 + (int64_t)wg * d, d, L.gain[4], eps, a.codes + (int64_t)wg * d,
                                         a.s + wg, a.sumq + wg, sh);
        arrive();
        if (!wait()) return;
        // 6. gate_proj: z = SiLU(first half) * second half, z kept in fp32
        {
            ContractArgs c{};
            c.nc = inner;
            c.out0 = a.z; c.aux_type = ACT_F32;
            gemv_phase<2, EPI_GLU, kSlotsG, CDH>(c, Wg, Mg, codes, a.s, a.sumq, d, b, wg, nwg, lds_a, part, NoPre{},
                                           wgt);
        }
        arrive();
        WeightRegs<1, CIA> wdn;
        load_weights<1, CIA, kSlotsI>(wdn, Wd, d, inner, wg);
        if (!wait()) return;
        // 7. quantise z
        if (wg < b)
            row_quant<float, NVZ, false>(a.z + (int64_t)wg * inner, inner, L.gain[5], eps,
                                         a.codes + (int64_t)wg * inner, a.s + wg, a.sumq + wg, sh);
        arrive();
        if (!wait()) return;
        // 8. down_proj + residual: out = x1 + down (activation dtype)
        {
            ContractArgs c{};
            c.nc = d;
            c.out0 = out; c.out_type = at;
            gemv_phase<1, EPI_RESID, kSlotsI, CIA>(c, Wd, Md, codes, a.s, a.sumq, inner, b, wg, nwg, lds_a, part,
                                              PreFrom<float>{a.x1}, wdn);
        }
        if (l + 1 < a.n_layers) {
            arrive();
            const StackLayer &N = a.layers[l + 1];
            const uint32_t *W[3] = {N.w[0], N.w[1], N.w[2]};
            load_weights<3, CDA, kSlotsD>(wifg, W, d, d, wg);
            if (!wait()) return;
        }
    }
}

__global__ void stack_barrier_reset(unsigned *bar) {
    for (int i = threadIdx.x; i < kStackBarWords; i += blockDim.x) bar[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct StackVariant {
    int nvx, nvz, cda, cdh, cia;
    const void *f32, *bf16;
};

#define MMF_STK_VARIANT(A, B, C, D, E)                                                                    \
    {A, B, C, D, E, reinterpret_cast<const void *>(&stack_decode_kernel<float, A, B, C, D, E>),           \
     reinterpret_cast<const void *>(&stack_decode_kernel<uint16_t, A, B, C, D, E>)}
// 370M (d 1024, inner 2816), 1.3B (d 2048, inner 5632) and 2.7B (d 2560, inner 6912) shapes
static const StackVariant kStackVariants[] = {
    MMF_STK_VARIANT(1, 3, 1, 1, 2),
    MMF_STK_VARIANT(2, 6, 1, 2, 3),
    MMF_STK_VARIANT(3, 7, 2, 3, 4),
};
#undef MMF_STK_VARIANT

static const StackVariant *pick_stack_variant(int d, int inner) {
    const int nvx = (d / 4 + 255) / 256, nvz = (inner / 4 + 255) / 256;
    const int nd = d / 256, ni = inner / 256;
    constexpr int wd = kStkWaves / kSlotsD, wgp = kStkWaves / kSlotsG, wi = kStkWaves / kSlotsI;
    const int cda = (nd + wd - 1) / wd, cdh = (nd + wgp - 1) / wgp, cia = (ni + wi - 1) / wi;
    for (const auto &v : kStackVariants)
        if (v.nvx >= nvx && v.nvz >= nvz && v.cda >= cda && v.cdh >= cdh && v.cia >= cia) return &v;
    return nullptr;
}

size_t stack_decode_lds_bytes(int d, int inner) {
    const int maxk = d > inner ? d : inner;
    return (size_t)16 * (maxk + 16) + kStkPartBytes;
}

const char *stack_decode_unsupported(int64_t b, int d, int inner) {
    if (b < 1 || b > 16) return "b must be in 1..16";
    if (d % 256 || inner % 256) return "d and inner must be multiples of 256";
    if (!pick_stack_variant(d, inner)) return "no kernel variant for this width";
    if (stack_decode_lds_bytes(d, inner) + 1024 > (size_t)160 * 1024) return "codes staging exceeds LDS";
    return nullptr;
}

hipError_t launch_stack_decode(const StackArgs &a, hipStream_t st, std::string *path) {
    const StackVariant *v = pick_stack_variant(a.d, a.inner);
    if (!v) return hipErrorInvalidValue;
    const void *fn = a.act_type == ACT_F32 ? v->f32 : v->bf16;
    const size_t lds = stack_decode_lds_bytes(a.d, a.inner);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static int ncu[64];
    static std::atomic<bool> raised[64][2 * sizeof kStackVariants / sizeof kStackVariants[0]];
    const int vi = (int)(v - kStackVariants) * 2 + (a.act_type == ACT_F32 ? 0 : 1);
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (!raised[dev][vi].load(std::memory_order_acquire)) {
        // the kernel's dynamic LDS limit goes to all that its static LDS leaves of a CU's 160 KB,
        // once per device, so every width the variant serves can launch
        std::lock_guard<std::mutex> lock(mu);
        hipFuncAttributes attr{};
        if ((e = hipFuncGetAttributes(&attr, fn)) != hipSuccess) return e;
        const int limit = 160 * 1024 - (int)attr.sharedSizeBytes;
        if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, limit)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&ncu[dev], hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        raised[dev][vi].store(true, std::memory_order_release);
    }
    int per_cu = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kStkThreads, lds)) != hipSuccess) return e;
    if (per_cu < 1) return hipErrorCooperativeLaunchTooLarge;
    const int nwg = ncu[dev] < kStkGrid ? ncu[dev] : kStkGrid;
    if (nwg < a.b) return hipErrorInvalidConfiguration;  // the quantiser phases take a row per workgroup
    launch_k(stack_barrier_reset, dim3(1), dim3(256), 0, st, a.bar);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    StackArgs args = a;
    void *params[] = {&args};
    e = hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(kStkThreads), params, (unsigned)lds, st);
    if (e == hipSuccess && path) *path += "stack_decode;";
    return e;
}

hipError_t stack_decode_expired_waits(unsigned *count) {
    return hipMemcpyFromSymbol(count, HIP_SYMBOL(g_stack_expired), sizeof(unsigned), 0, hipMemcpyDeviceToHost);
}

}  // namespace mmf
