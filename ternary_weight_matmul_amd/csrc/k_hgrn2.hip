// The HGRN recurrence with an expanded state (HGRN2), fp32 (gfx950).
//
// "MatMul-Free LLM 深度分析报告" (section "核心价值提炼", table "创新之处" and list
// "关键设计决策") names HGRN2 as the gated linear recurrence that replaces
// attention and prints its elementwise form h_t = g_t * h_{t-1} + x_t. The
// expanded state widens each head's state from e channels to an e x e matrix:
//     S_t[a][c] = f_t[a] * S_{t-1}[a][c] + (1 - f_t[a]) * i_t[c]
//     y_t[c]    = sum_a o_t[a] * S_t[a][c]
// (a, c index the head's e channels; the forget gate acts on the rows).
//
// Columns of the state are independent of each other, so a workgroup owns one
// (sequence, head, block of BC columns) and keeps its E x BC block of the
// state in registers for the whole sequence: thread (ta, tc) holds rows
// ta*RA .. ta*RA+RA-1 and columns tc*RC .. tc*RC+RC-1, with ta the lane's low
// four bits, so the sum over rows of the readout is a DPP reduction within a
// row of 16 lanes (every lane ends with the row total; fixed order). Per token
// a thread does 3 RA*RC multiply-adds and 4 RC DPP adds: the recurrence is
// bound by the vector ALU (about 5 e^2 flops per token and head against 16 e
// bytes of HBM traffic). The gates of TT tokens are staged through LDS with
// coalesced loads issued one chunk ahead; the outputs of a chunk leave as
// 16-byte stores. The state block enters and leaves through LDS as 16-byte
// row pieces, so a decode step (one token) streams the state at full width.
// Workgroups that share a (sequence, head) are dealt to the same XCD, so its f
// and o rows come from that XCD's L2 after the first reader.
#include "device_common.hpp"
#include "launch.hpp"

namespace mmf {

template <int E>
struct H2Shape {
    static constexpr int BC = E < 32 ? E : 32;  // state columns per workgroup
    static constexpr int RA = E / 16;           // rows per thread
    static constexpr int RC = BC / 16;          // columns per thread
    static constexpr int TT = 16;               // tokens per LDS chunk
    static constexpr int GATE_FL = 2 * TT * E;  // f and o of a chunk (floats)
    static constexpr int STATE_FL = E * BC;     // the state block (floats)
    static constexpr int STAGE_FL = GATE_FL > STATE_FL ? GATE_FL : STATE_FL;
    static constexpr int G4 = TT * E / 4;       // float4s of one gate per chunk
    static constexpr int I4 = TT * BC / 4;      // float4s of i per chunk
    static constexpr int GL = (G4 + 255) / 256; // float4 slots per thread per gate
    static constexpr int IL = (I4 + 255) / 256;
    static constexpr int S4 = E * BC / 4;       // float4s of the state block
    static constexpr int SL = (S4 + 255) / 256;
};

template <int E>
__global__ __launch_bounds__(256) void hgrn2_scan_kernel(const float *__restrict__ f, const float *__restrict__ xi,
                                                         const float *__restrict__ o, const float *s0, float *y,
                                                         float *s_last, int64_t t, int64_t d, int heads) {
    using Sh = H2Shape<E>;
    constexpr int BC = Sh::BC, RA = Sh::RA, RC = Sh::RC, TT = Sh::TT;
    constexpr int CBK = E / BC;
    __shared__ __attribute__((aligned(16))) float stage[Sh::STAGE_FL];  // f, o of a chunk; the state block
    __shared__ __attribute__((aligned(16))) float si[TT * BC];
    __shared__ __attribute__((aligned(16))) float sy[TT * BC];

    // workgroup -> (pair, column block); with a grid of whole XCD rounds, the
    // CBK workgroups of a pair get consecutive slots of one XCD
    const int G = gridDim.x, g = blockIdx.x;
    const int lin = (G & 7) == 0 ? (g & 7) * (G >> 3) + (g >> 3) : g;
    const int pair = lin / CBK, cblk = lin - pair * CBK;
    const int64_t bi = pair / heads;
    const int head = pair - (int)bi * heads;
    const int tid = threadIdx.x, ta = tid & 15, tc = tid >> 4;
    const int64_t col0 = (int64_t)head * E;         // first channel of the head
    const int64_t ccol0 = col0 + (int64_t)cblk * BC; // first channel of the column block
    const int64_t row_base = bi * t * d;             // element (bi, 0, 0)
    const int64_t sbase = ((int64_t)pair * E) * E + (int64_t)cblk * BC;  // state (pair, 0, cblk*BC)

    // ---- the state block: coalesced rows of BC floats through LDS
    float S[RA][RC];
#pragma unroll
    for (int j = 0; j < Sh::SL; ++j) {
        const int q = tid + 256 * j;
        if (q < Sh::S4) {
            const int a = q / (BC / 4), c4 = q - a * (BC / 4);
            const float4 v = s0 ? *reinterpret_cast<const float4 *>(s0 + sbase + (int64_t)a * E + 4 * c4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<float4 *>(stage + a * BC + 4 * c4) = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RA; ++r)
#pragma unroll
        for (int c = 0; c < RC; ++c) S[r][c] = stage[(ta * RA + r) * BC + tc * RC + c];
    __syncthreads();

    // ---- chunks of TT tokens: loads of chunk n+1 in flight while chunk n runs
    float4 pf[Sh::GL], po[Sh::GL], pi[Sh::IL];
    auto fetch = [&](int64_t t0) {
#pragma unroll
        for (int j = 0; j < Sh::GL; ++j) {
            const int q = tid + 256 * j;
            const int k = q / (E / 4), c4 = q - k * (E / 4);
            const int64_t tk = t0 + k < t ? t0 + k : t - 1;  // rows past t: any valid row, unused
            const int64_t off = row_base + tk * d + col0 + 4 * c4;
            if (q < Sh::G4) {
                pf[j] = *reinterpret_cast<const float4 *>(f + off);
                po[j] = *reinterpret_cast<const float4 *>(o + off);
            }
        }
#pragma unroll
        for (int j = 0; j < Sh::IL; ++j) {
            const int q = tid + 256 * j;
            const int k = q / (BC / 4), c4 = q - k * (BC / 4);
            const int64_t tk = t0 + k < t ? t0 + k : t - 1;
            if (q < Sh::I4) pi[j] = *reinterpret_cast<const float4 *>(xi + row_base + tk * d + ccol0 + 4 * c4);
        }
    };
    auto park = [&]() {
#pragma unroll
        for (int j = 0; j < Sh::GL; ++j) {
            const int q = tid + 256 * j;
            if (q < Sh::G4) {
                *reinterpret_cast<float4 *>(stage + 4 * q) = pf[j];
                *reinterpret_cast<float4 *>(stage + TT * E + 4 * q) = po[j];
            }
        }
#pragma unroll
        for (int j = 0; j < Sh::IL; ++j) {
            const int q = tid + 256 * j;
            if (q < Sh::I4) *reinterpret_cast<float4 *>(si + 4 * q) = pi[j];
        }
    };

    if (t > 0) {
        fetch(0);
        park();
        __syncthreads();
    }
    for (int64_t t0 = 0; t0 < t; t0 += TT) {
        const int nk = t - t0 < TT ? (int)(t - t0) : TT;
        const bool more = t0 + TT < t;
        if (more) fetch(t0 + TT);
        for (int k = 0; k < nk; ++k) {
            float fa[RA], oa[RA], vc[RC];
#pragma unroll
            for (int r = 0; r < RA; ++r) {
                fa[r] = stage[k * E + ta * RA + r];
                oa[r] = stage[TT * E + k * E + ta * RA + r];
            }
#pragma unroll
            for (int c = 0; c < RC; ++c) vc[c] = si[k * BC + tc * RC + c];
            float part[RC];
#pragma unroll
            for (int c = 0; c < RC; ++c) part[c] = 0.0f;
#pragma unroll
            for (int r = 0; r < RA; ++r) {
                const float kr = 1.0f - fa[r];
#pragma unroll
                for (int c = 0; c < RC; ++c) {
                    S[r][c] = fmaf(fa[r], S[r][c], kr * vc[c]);
                    part[c] = fmaf(oa[r], S[r][c], part[c]);
                }
            }
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                float v = part[c];
                v += dpp_f<kDppXor1>(v);
                v += dpp_f<kDppXor2>(v);
                v += dpp_f<kDppHalfMirror>(v);
                v += dpp_f<kDppMirror>(v);
                part[c] = v;
            }
            if (ta == 0) {
#pragma unroll
                for (int c = 0; c < RC; ++c) sy[k * BC + tc * RC + c] = part[c];
            }
        }
        __syncthreads();  // sy complete; stage and si no longer read
        for (int q = tid; q < nk * (BC / 4); q += 256) {
            const int k = q / (BC / 4), c4 = q - k * (BC / 4);
            *reinterpret_cast<float4 *>(y + row_base + (t0 + k) * d + ccol0 + 4 * c4) =
                *reinterpret_cast<const float4 *>(sy + 4 * q);
        }
        if (more) park();
        __syncthreads();  // the next chunk is in LDS; sy free again
    }

    // ---- the state block out, through LDS
    if (s_last) {
#pragma unroll
        for (int r = 0; r < RA; ++r)
#pragma unroll
            for (int c = 0; c < RC; ++c) stage[(ta * RA + r) * BC + tc * RC + c] = S[r][c];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < Sh::SL; ++j) {
            const int q = tid + 256 * j;
            if (q < Sh::S4) {
                const int a = q / (BC / 4), c4 = q - a * (BC / 4);
                *reinterpret_cast<float4 *>(s_last + sbase + (int64_t)a * E + 4 * c4) =
                    *reinterpret_cast<const float4 *>(stage + a * BC + 4 * c4);
            }
        }
    }
}

hipError_t launch_hgrn2_scan(const float *f, const float *i, const float *o, const float *s0, float *y,
                             float *s_last, int64_t b, int64_t t, int64_t d, int e, hipStream_t st,
                             const char **name) {
    const int heads = (int)(d / e);
    const int64_t pairs = b * heads;
    const int cbk = e < 32 ? 1 : e / 32;
    const unsigned grid = (unsigned)(pairs * cbk);
    if (grid == 0) return hipSuccess;
    switch (e) {
        case 16: launch_k(hgrn2_scan_kernel<16>, grid, 256, 0, st, f, i, o, s0, y, s_last, t, d, heads); break;
        case 32: launch_k(hgrn2_scan_kernel<32>, grid, 256, 0, st, f, i, o, s0, y, s_last, t, d, heads); break;
        case 64: launch_k(hgrn2_scan_kernel<64>, grid, 256, 0, st, f, i, o, s0, y, s_last, t, d, heads); break;
        case 128: launch_k(hgrn2_scan_kernel<128>, grid, 256, 0, st, f, i, o, s0, y, s_last, t, d, heads); break;
        default: return hipErrorInvalidValue;
    }
    if (name) *name = e == 16 ? "hgrn2_scan<16>" : e == 32 ? "hgrn2_scan<32>" : e == 64 ? "hgrn2_scan<64>"
                                                                                     : "hgrn2_scan<128>";
    return hipGetLastError();
}

}  // namespace mmf
