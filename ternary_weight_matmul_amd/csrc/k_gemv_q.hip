// Decode contraction with its input quantiser in the same launch (gfx950).
//
// A decode step of the HGRNBit block ("MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，
// 剩下什麼", section "HGRNBitBlock 的結構") quantises a few rows (one per sequence)
// before each of its four ternary contractions: x before i/f/g, the g_norm
// gate output before o_proj, x1 before gate_proj and z before down_proj
// ("MatMul-Free LLM 深度分析报告", list "可复用的模式与技巧": the RMSNorm and the
// activation quantiser belong to the same fused step). As separate kernels a
// quantiser and its contraction pay a kernel boundary (about 2 us in a HIP
// graph on MI355X) and the contraction's weight loads start only after it.
//
// Here one launch does both. Workgroups 0..b-1 each quantise one row (the
// 256-thread quantisers of row_quant.hpp, so the bits equal those of the
// separate quantiser kernels) and publish it: codes, scale and code sum go out
// with device-scope stores, which write through to memory, and a device-scope
// counter counts the rows. The other workgroups, one per 16 output channels,
// issue their weight and epilogue-operand loads at once, wait (bounded) until
// the counter reaches b, then read the codes with device-scope loads (which do
// not return an older cached copy; the XCDs' L2 caches are not coherent with
// each other) and finish as the decode GEMV does. Workgroups are dispatched in
// index order, so the quantising ones run before anyone waits for them.
//
// The counter pair (rows published, workgroups finished) is library state on
// the device: the last workgroup to finish returns both to zero, so the next
// launch starts from zero. Calls on one stream therefore never interfere;
// each stream gets its own pair (kHSlots streams per device at most).
#include "device_common.hpp"
#include "launch.hpp"
#include "epilogue.hpp"
#include "row_quant.hpp"

#include <mutex>
#include <type_traits>
#include <unordered_map>

namespace mmf {

constexpr int kHSlots = 64;               // counter pairs: one per stream
constexpr long kHSpinLimit = 1L << 20;    // about a second of polling
constexpr unsigned kBufferRsrcWord3 = 0x00020000u;  // raw buffer descriptor, gfx9 data format
constexpr int kSc1 = 16;                  // buffer-load cache policy: device scope

// slot s: rows published at [64 s], workgroups finished at [64 s + 32];
// waits that gave up at [64 kHSlots]
__device__ unsigned g_handoff[64 * kHSlots + 64];

struct QuantContractArgs {
    ContractArgs c;      // contraction: B, mu, m (= b rows), nc, k, outputs, residual
    const void *x;       // QK_ROW: rows to quantise [b][k]; QK_GNORM: h [b][k] fp32
    const void *g;       // QK_GNORM: g [b][k]
    const float *gain;   // quantiser gain (RMSNorm weight) or null
    const float *gnw;    // QK_GNORM: g_norm weight or null
    float eps;
    int8_t *codes;       // handoff: codes [b][k], scale [b], code sum [b]
    float *s;
    int32_t *sumq;
    int slot;
    int nslices;         // 256-k slices of a row
};

__device__ __forceinline__ unsigned ld_dev(const unsigned *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NG, int EPI, int QK, typename XT, typename GT, typename RT, int NVQ, int SPW>
__global__ __launch_bounds__(1024) void tgemv_q_kernel(const QuantContractArgs a) {
    const ContractArgs &p = a.c;
    extern __shared__ int32_t part[];  // [waves][NG][256]
    __shared__ RowQuantLds sh;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int b = (int)p.m, K = p.k, KW = K >> 4;
    unsigned *done = g_handoff + 64 * a.slot, *fin = done + 32;

    if ((int)blockIdx.x < b) {
        // ---- quantiser workgroup: row r, published with device-scope stores
        const int r = blockIdx.x;
        if constexpr (QK == QK_GNORM) {
            static_assert(std::is_same<XT, float>::value, "g_norm reads the fp32 state");
            row_gnorm_quant<GT, NVQ, false, true>(static_cast<const float *>(a.x) + (int64_t)r * K,
                                                  static_cast<const GT *>(a.g) + (int64_t)r * K, K, a.gnw, a.gain,
                                                  a.eps, a.codes + (int64_t)r * K, a.s + r, a.sumq + r, nullptr, sh);
        } else {
            row_quant<XT, NVQ, false, true>(static_cast<const XT *>(a.x) + (int64_t)r * K, K, a.gain, a.eps,
                                            a.codes + (int64_t)r * K, a.s + r, a.sumq + r, sh);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        // ---- contraction workgroup: 16 output channels
        const int lc = lane & 15, lg = lane >> 4;
        const int n0 = ((int)blockIdx.x - b) * 16;
        const int gn = min(n0 + lc, p.nc - 1);  // columns past nc load a valid row; never stored
        // weights of this wave's slices (straight-line: slices past the row load the last one, unused)
        uint4 bw[SPW][NG];
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int sl = min(wave + nw * j, a.nslices - 1);
#pragma unroll
            for (int g = 0; g < NG; ++g)
                bw[j][g] = *reinterpret_cast<const uint4 *>(p.B[g] + (int64_t)gn * KW + sl * 16 + lg * 4);
        }
        float sw[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) sw[g] = weight_sw(p.mu[g]);
        // the epilogue operand of this thread's output (row er, channel n0 + ec)
        constexpr bool PRE = EPI == EPI_RESID || EPI == EPI_GATES_STEP;
        const int er = tid >> 4, ec = tid & 15;
        float pre = 0.0f;
        if (PRE && tid < 256) {
            const RT *src = static_cast<const RT *>(EPI == EPI_RESID ? p.res : p.out0);
            pre = load_act(src, (int64_t)min(er, b - 1) * p.nc + min(n0 + ec, p.nc - 1));
        }
        // wait for the b rows
        if (tid == 0) {
            long spins = 0;
            while (ld_dev(done) < (unsigned)b) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins > kHSpinLimit) {
                    __hip_atomic_fetch_add(g_handoff + 64 * kHSlots, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
        __syncthreads();
        // codes of row lc (rows past b read row b - 1, never stored), device scope
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(a.codes, 0, b * K, kBufferRsrcWord3);
        const int arow = min(lc, b - 1) * K;
        i32x4 af[SPW][4];
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int sl = min(wave + nw * j, a.nslices - 1);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                af[j][q] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rsrc, arow + 16 * (sl * 16 + lg * 4 + q), 0, kSc1));
        }
        float srow = 0.0f;
        int32_t sqrow = 0;
        if (tid < 256 && er < b) {
            srow = __uint_as_float(ld_dev(reinterpret_cast<const unsigned *>(a.s) + er));
            sqrow = (int32_t)ld_dev(reinterpret_cast<const unsigned *>(a.sumq) + er);
        }
        i32x4 acc[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g] = i32x4{};
#pragma unroll
        for (int j = 0; j < SPW; ++j)
            if (wave + nw * j < a.nslices)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int g = 0; g < NG; ++g) {
                        const uint32_t word = q == 0 ? bw[j][g].x : q == 1 ? bw[j][g].y : q == 2 ? bw[j][g].z : bw[j][g].w;
                        acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[j][q], decode_word(word), acc[g], 0, 0, 0);
                    }
        int32_t *mine = part + wave * NG * 256;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) mine[g * 256 + (4 * lg + i) * 16 + lc] = acc[g][i];
        __syncthreads();
        if (tid < 256 && er < b && n0 + ec < p.nc) {
            int32_t v[NG];
            float dq[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                int32_t sum = 0;
                for (int w = 0; w < nw; ++w) sum += part[(w * NG + g) * 256 + er * 16 + ec];
                v[g] = sum - sqrow;
                dq[g] = __builtin_amdgcn_rcpf(srow * sw[g]);
            }
            epilogue_vals<EPI, NG, true>(p, er, n0 + ec, v, dq, pre);
        }
    }
    // the last workgroup to finish returns the counters to zero for the next launch
    __syncthreads();
    if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(fin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == gridDim.x - 1) {
            __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(fin, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static const char *q_epi_name(int epi) {
    switch (epi) {
        case EPI_GATES_STEP: return "gates_step";
        case EPI_RESID: return "resid";
        case EPI_GLU: return "glu";
    }
    return "?";
}

// 256-thread chunks per row the quantiser registers must hold
static int q_pick_nv(int k, int qk) {
    const int need = (k + 1023) / 1024;
    const int opts[3] = {2, 3, 7};
    const int nopt = qk == QK_GNORM ? 2 : 3;
    for (int i = 0; i < nopt; ++i)
        if (need <= opts[i]) return opts[i];
    return 0;
}

static int q_waves(int nslices) { return nslices < 4 ? 4 : nslices > 16 ? 16 : nslices; }

bool quant_contract_supported(int64_t b, int nc, int k, EpiKind epi, int qk, ActType xt, ActType gt) {
    (void)xt;
    (void)gt;
    if (b < 1 || b > 16 || nc < 1 || k < 256 || k % 256) return false;
    if (epi != EPI_GATES_STEP && epi != EPI_RESID && epi != EPI_GLU) return false;
    if (q_pick_nv(k, qk) == 0) return false;
    if ((qk == QK_GNORM || epi != EPI_RESID) && k > 3072) return false;  // one slice per wave for K = d
    return (k >> 8) <= 32;
}

// The counter pair of a stream (kHSlots per process; -1 once they are taken).
static int handoff_slot(hipStream_t st) {
    static std::mutex mu;
    static std::unordered_map<hipStream_t, int> slots;
    std::lock_guard<std::mutex> lock(mu);
    auto it = slots.find(st);
    if (it != slots.end()) return it->second;
    if ((int)slots.size() >= kHSlots) return -1;
    const int s = (int)slots.size();
    slots.emplace(st, s);
    return s;
}

template <int NG, int EPI, int QK, typename XT, typename GT, typename RT, int NVQ, int SPW>
static hipError_t run_q(const QuantContractArgs &a, hipStream_t st) {
    const int nw = q_waves(a.nslices);
    const size_t lds = (size_t)nw * NG * 256 * sizeof(int32_t);
    const unsigned grid = (unsigned)(a.c.m + (a.c.nc + 15) / 16);
    tgemv_q_kernel<NG, EPI, QK, XT, GT, RT, NVQ, SPW><<<grid, nw * 64, lds, st>>>(a);
    return hipGetLastError();
}

template <int NG, int EPI, int QK, typename XT, typename GT, typename RT>
static hipError_t run_q_nv(const QuantContractArgs &a, int nv, int spw, hipStream_t st) {
    if constexpr (QK == QK_GNORM || EPI != EPI_RESID) {
        // K = d: at most 3072, one slice per wave
        if (spw != 1 || nv == 7) return hipErrorInvalidValue;
        return nv == 2 ? run_q<NG, EPI, QK, XT, GT, RT, 2, 1>(a, st) : run_q<NG, EPI, QK, XT, GT, RT, 3, 1>(a, st);
    } else {
        switch (nv * 2 + spw) {
            case 2 * 2 + 1: return run_q<NG, EPI, QK, XT, GT, RT, 2, 1>(a, st);
            case 3 * 2 + 1: return run_q<NG, EPI, QK, XT, GT, RT, 3, 1>(a, st);
            case 7 * 2 + 1: return run_q<NG, EPI, QK, XT, GT, RT, 7, 1>(a, st);
            case 7 * 2 + 2: return run_q<NG, EPI, QK, XT, GT, RT, 7, 2>(a, st);
        }
        return hipErrorInvalidValue;
    }
}

hipError_t launch_quant_contract(const ContractArgs &c, EpiKind epi, int qk, const void *x, ActType xt,
                                 const void *g, ActType gt, const float *gain, const float *gnw, float eps,
                                 int8_t *codes, float *s, int32_t *sumq, hipStream_t st, std::string *path) {
    if (!quant_contract_supported(c.m, c.nc, c.k, epi, qk, xt, gt)) return hipErrorInvalidValue;
    QuantContractArgs a{};
    a.c = c;
    a.x = x; a.g = g; a.gain = gain; a.gnw = gnw; a.eps = eps;
    a.codes = codes; a.s = s; a.sumq = sumq;
    a.nslices = c.k >> 8;
    a.slot = handoff_slot(st);
    if (a.slot < 0) return hipErrorInvalidValue;
    const int nv = q_pick_nv(c.k, qk);
    const int spw = a.nslices > 16 ? 2 : 1;
    if (path) *path += std::string("tgemv_q<") + (qk == QK_GNORM ? "gnorm_resid" : q_epi_name(epi)) + ">;";
    const bool xf = xt == ACT_F32, gf = gt == ACT_F32;
    switch (epi) {
        case EPI_GATES_STEP:  // quantised x, state in place
            if (qk != QK_ROW) return hipErrorInvalidValue;
            return xf ? run_q_nv<3, EPI_GATES_STEP, QK_ROW, float, float, float>(a, nv, spw, st)
                      : run_q_nv<3, EPI_GATES_STEP, QK_ROW, uint16_t, uint16_t, float>(a, nv, spw, st);
        case EPI_GLU:  // quantised x1 (fp32)
            if (qk != QK_ROW || !xf) return hipErrorInvalidValue;
            return run_q_nv<2, EPI_GLU, QK_ROW, float, float, float>(a, nv, spw, st);
        case EPI_RESID:
            if (qk == QK_GNORM) {  // g_norm gate of (h, g) + o_proj, residual x in g's type
                if (!xf || c.res_type != gt) return hipErrorInvalidValue;
                return gf ? run_q_nv<1, EPI_RESID, QK_GNORM, float, float, float>(a, nv, spw, st)
                          : run_q_nv<1, EPI_RESID, QK_GNORM, float, uint16_t, uint16_t>(a, nv, spw, st);
            }
            // quantised z + down_proj, residual x1 (fp32)
            if (c.res_type != ACT_F32) return hipErrorInvalidValue;
            return xf ? run_q_nv<1, EPI_RESID, QK_ROW, float, float, float>(a, nv, spw, st)
                      : run_q_nv<1, EPI_RESID, QK_ROW, uint16_t, uint16_t, float>(a, nv, spw, st);
        default:
            return hipErrorInvalidValue;
    }
}

hipError_t quant_contract_expired_waits(unsigned *count) {
    return hipMemcpyFromSymbol(count, HIP_SYMBOL(g_handoff), sizeof(unsigned), 64 * kHSlots * sizeof(unsigned),
                               hipMemcpyDeviceToHost);
}

}  // namespace mmf
