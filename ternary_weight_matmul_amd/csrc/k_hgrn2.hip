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
// four bits. The sum over rows of the readout runs as a DPP sum over each quad
// of lanes per token and a sum of the four quads' partials, in LDS, once per
// chunk of tokens (fixed order). Per token a thread does 3 RA*RC vector
// operations (S - v, then f (S - v) + v, then the readout's multiply-add) and
// 2 DPP adds per column: the recurrence is bound by the vector ALU (about
// 5 e^2 flops per token and head against 16 e bytes of HBM traffic). The
// gates of TT tokens are staged through LDS with
// coalesced loads issued one chunk ahead; the outputs of a chunk leave as
// 16-byte stores. The state block goes straight between HBM and registers as
// one RC-float piece per row and thread (16 bytes for heads of 64 and 128).
// Workgroups that share a (sequence, head) are dealt to the same XCD, so its f
// and o rows come from that XCD's L2 after the first reader.
#include "device_common.hpp"
#include "launch.hpp"

namespace mmf {

template <int N>
using fvec = float __attribute__((ext_vector_type(N)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <int E>
struct H2Shape {
    static constexpr int BC = E < 64 ? E : 64;  // state columns per workgroup
    static constexpr int TA = 16;               // lanes that share a column (a DPP row)
    static constexpr int RA = E / TA;           // rows per thread
    static constexpr int RC = BC * TA / 256;    // columns per thread
    static constexpr int TT = 16;               // tokens per LDS chunk
    static constexpr int GATE_FL = 2 * TT * E;  // f and o of a chunk (floats)
    static constexpr int G4 = TT * E / 4;       // float4s of one gate per chunk
    static constexpr int I4 = TT * BC / 4;      // float4s of i per chunk
    static constexpr int GL = (G4 + 255) / 256; // float4 slots per thread per gate
    static constexpr int IL = (I4 + 255) / 256;
    static_assert(TA * RA == E && RC * (256 / TA) == BC, "256 threads tile the E x BC block");
};

template <int E>
__global__ __launch_bounds__(256) void hgrn2_scan_kernel(const float *__restrict__ f, const float *__restrict__ xi,
                                                         const float *__restrict__ o, const float *s0, float *y,
                                                         float *s_last, int64_t t, int64_t d, int heads) {
    using Sh = H2Shape<E>;
    constexpr int BC = Sh::BC, RA = Sh::RA, RC = Sh::RC, TT = Sh::TT, TA = Sh::TA;
    constexpr int CBK = E / BC;
    __shared__ __attribute__((aligned(16))) float stage[Sh::GATE_FL];  // f and o of a chunk
    __shared__ __attribute__((aligned(16))) float si[TT * BC];
    constexpr int NQ = TA / 4;  // quads of lanes per column
    __shared__ __attribute__((aligned(16))) float sq[TT * NQ * BC];  // per-quad sums of the readout

    // workgroup -> (pair, column block); with a grid of whole XCD rounds, the
    // CBK workgroups of a pair get consecutive slots of one XCD
    const int G = gridDim.x, g = blockIdx.x;
    const int lin = (G & 7) == 0 ? (g & 7) * (G >> 3) + (g >> 3) : g;
    const int pair = lin / CBK, cblk = lin - pair * CBK;
    const int64_t bi = pair / heads;
    const int head = pair - (int)bi * heads;
    const int tid = threadIdx.x, ta = tid & (TA - 1), tc = tid / TA;
    const int64_t col0 = (int64_t)head * E;         // first channel of the head
    const int64_t ccol0 = col0 + (int64_t)cblk * BC; // first channel of the column block
    const int64_t row_base = bi * t * d;             // element (bi, 0, 0)
    const int64_t sbase = ((int64_t)pair * E) * E + (int64_t)cblk * BC;  // state (pair, 0, cblk*BC)

    // ---- chunks of TT tokens: loads of chunk n+1 in flight while chunk n runs
    // (a gate of a chunk is at most 512 float4s and i at most 256, so a thread
    // holds at most two slots of each gate and one of i, in named registers;
    // slots past a gate's float4 count -- only when it is not a multiple of 256
    // -- load a clamped, valid element and are never parked)
    static_assert(Sh::GL <= 2 && Sh::IL == 1, "prefetch slots");
    float4 pf0, pf1, po0, po1, pi0;
    auto gate_off = [&](int64_t t0, int j) __attribute__((always_inline)) {
        const int q = min(tid + 256 * j, Sh::G4 - 1);
        const int k = q / (E / 4), c4 = q - k * (E / 4);
        const int64_t tk = t0 + k < t ? t0 + k : t - 1;  // rows past t: any valid row, unused
        return row_base + tk * d + col0 + 4 * c4;
    };
    auto fetch = [&](int64_t t0) __attribute__((always_inline)) {
        const int64_t off0 = gate_off(t0, 0);
        pf0 = *reinterpret_cast<const float4 *>(f + off0);
        po0 = *reinterpret_cast<const float4 *>(o + off0);
        if constexpr (Sh::GL == 2) {
            const int64_t off1 = gate_off(t0, 1);
            pf1 = *reinterpret_cast<const float4 *>(f + off1);
            po1 = *reinterpret_cast<const float4 *>(o + off1);
        }
        const int q = min(tid, Sh::I4 - 1);
        const int k = q / (BC / 4), c4 = q - k * (BC / 4);
        const int64_t tk = t0 + k < t ? t0 + k : t - 1;
        pi0 = *reinterpret_cast<const float4 *>(xi + row_base + tk * d + ccol0 + 4 * c4);
    };
    auto park = [&]() __attribute__((always_inline)) {
        if (Sh::G4 % 256 == 0 || tid < Sh::G4) {
            *reinterpret_cast<float4 *>(stage + 4 * tid) = pf0;
            *reinterpret_cast<float4 *>(stage + TT * E + 4 * tid) = po0;
        }
        if constexpr (Sh::GL == 2) {
            const int q = tid + 256;
            if (Sh::G4 % 256 == 0 || q < Sh::G4) {
                *reinterpret_cast<float4 *>(stage + 4 * q) = pf1;
                *reinterpret_cast<float4 *>(stage + TT * E + 4 * q) = po1;
            }
        }
        if (Sh::I4 % 256 == 0 || tid < Sh::I4) *reinterpret_cast<float4 *>(si + 4 * tid) = pi0;
    };

    if (t > 0) fetch(0);

    // ---- the state block, straight into registers: each of a thread's RA rows is
    // one RC-float vector (one load instruction of a wave covers 16 rows x 4 RC
    // contiguous floats); these loads are in flight with the first chunk's
    float S[RA][RC];
    {
        fvec<RC> sv[RA];
        if (s0) {  // one uniform branch around all the loads: no wait between them
#pragma unroll
            for (int r = 0; r < RA; ++r)
                sv[r] = *reinterpret_cast<const fvec<RC> *>(s0 + sbase + (int64_t)(ta * RA + r) * E + tc * RC);
        } else {
#pragma unroll
            for (int r = 0; r < RA; ++r) sv[r] = fvec<RC>{};
        }
#pragma unroll
        for (int r = 0; r < RA; ++r)
#pragma unroll
            for (int c = 0; c < RC; ++c) S[r][c] = sv[r][c];
    }

    // one token: S <- f (S - v) + v (= f S + (1 - f) v), y = sum over rows of o S
    auto token = [&](int k) __attribute__((always_inline)) {
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
        for (int r = 0; r < RA; ++r)
#pragma unroll
            for (int c = 0; c < RC; ++c) {
                S[r][c] = fmaf(fa[r], S[r][c] - vc[c], vc[c]);
                part[c] = fmaf(oa[r], S[r][c], part[c]);
            }
        // sums over each quad of lanes (DPP); the quads meet when the chunk is written
        fvec<RC> qs;
#pragma unroll
        for (int c = 0; c < RC; ++c) {
            float v = part[c];
            v += dpp_f<kDppXor1>(v);
            v += dpp_f<kDppXor2>(v);
            qs[c] = v;
        }
        if ((ta & 3) == 0) *reinterpret_cast<fvec<RC> *>(sq + (k * NQ + (ta >> 2)) * BC + tc * RC) = qs;
    };

    if (t > 0) park();
    // every load so far (the state, the first chunk) has landed before the loop:
    // otherwise the loop's first use of the state would have to wait for the
    // prefetch issued in front of it too
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt, lgkmcnt unconstrained
    __syncthreads();
    for (int64_t t0 = 0; t0 < t; t0 += TT) {
        const int nk = t - t0 < TT ? (int)(t - t0) : TT;
        const bool more = t0 + TT < t;
        if (more) fetch(t0 + TT);
        if (nk == TT) {
#pragma unroll
            for (int k = 0; k < TT; ++k) token(k);
        } else {
            for (int k = 0; k < nk; ++k) token(k);
        }
        __syncthreads();  // sq complete; stage and si no longer read
        for (int q = tid; q < nk * (BC / 4); q += 256) {
            const int k = q / (BC / 4), c4 = q - k * (BC / 4);
            const float *pq = sq + k * NQ * BC + 4 * c4;
            float4 acc = *reinterpret_cast<const float4 *>(pq);
#pragma unroll
            for (int qd = 1; qd < NQ; ++qd) {
                const float4 v = *reinterpret_cast<const float4 *>(pq + qd * BC);
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
            *reinterpret_cast<float4 *>(y + row_base + (t0 + k) * d + ccol0 + 4 * c4) = acc;
        }
        if (more) park();
        __syncthreads();  // the next chunk is in LDS; sq free again
    }

    // ---- the state block out, as it came in
    if (s_last) {
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            fvec<RC> v;
#pragma unroll
            for (int c = 0; c < RC; ++c) v[c] = S[r][c];
            *reinterpret_cast<fvec<RC> *>(s_last + sbase + (int64_t)(ta * RA + r) * E + tc * RC) = v;
        }
    }
}

// ----------------------------------------------------------------------------
// Chunked form (the pages name a step-wise and a chunked implementation of the
// recurrence). Over a chunk of C tokens starting from the state S0:
//   Q~[t][a]  = o_t[a] * prod_{r<=t} f_r[a]             (decay from the chunk start)
//   K^[s][a]  = (1 - f_s[a]) * prod_{s<r<C} f_r[a]      (decay to the chunk end)
//   A[t][s]   = sum_a o_t[a] (1 - f_s[a]) prod_{s<r<=t} f_r[a]   (s <= t, else 0)
//   Y  = Q~ S0 + A V                  (C x BC: the chunk's outputs)
//   S1 = diag(prod_{r<C} f_r) S0 + K^T V
// (V = the chunk's input rows of the block's columns). When every gate of the
// chunk is at least 2^-6, 1 / prod_{r<=s} f_r stays below 2^96 and A is the
// product Q~ K~^T with K~[s][a] = (1 - f_s[a]) / prod_{r<=s} f_r[a] (and
// K^ = K~ * prod_{r<C} f_r); a chunk with a smaller gate takes A as sums of
// running products of the gates and K^ as suffix products, with no division.
// The products run on fp32 MFMA (v_mfma_f32_16x16x4_f32); wave w owns the
// block's columns 16w .. 16w+15 and holds their E x 16 slice of the state as
// E/16 accumulator tiles, which serve as the B operand of Q~ S0 as they are.
//
// The loop is pipelined over three chunks, with two synchronisations per
// chunk (a barrier, and the workgroup's vote on small gates, a block-wide OR
// that also orders LDS): while the waves read out chunk k (Y and the state
// update, the only steps that need the state), they form chunk k+1's A, and
// between the two the decays of chunk k+2 (Q~, K~, the total decay) are
// prepared from its gates, which were parked in LDS during the same iteration. Gates load into registers one
// iteration before they are parked. Tokens past the sequence end act as
// f = 1, o = 0, i = 0.
//
// The gates, the input and the outputs move through buffer resources that
// span the workgroup's sequence: rows past its end read as zeros and are not
// written. So every iteration issues the same loads and stores whatever its
// chunk (the prefetches past the last chunk read nothing), and each wait for
// a prefetch counts only what was issued after it, never this chunk's output
// stores. A sequence's rows must span less than 2^31 bytes.
constexpr float kChunkMinGate = 0.015625f;  // 2^-6
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw 32-bit buffer access, range-checked

template <int E>
struct H2Chunk {
    static constexpr int C = 16;          // tokens per chunk
    static constexpr int BC = 64;         // state columns per workgroup: 4 waves x 16
    static constexpr int AT = E / 16;     // 16-row tiles of a wave's state slice
    static constexpr int RA = E / 16;     // rows per thread in the direct A sums (16 threads per s)
    static constexpr int G4 = C * E / 4;  // float4s of one gate per chunk
    static constexpr int I4 = C * BC / 4; // float4s of i per chunk
    static constexpr int GL = (G4 + 255) / 256;
    // LDS row strides chosen so that the MFMA operand reads (16 lanes along one index, 4 lane
    // groups along the other) spread over the banks
    static constexpr int QS = C + 1;       // Q~, K~ / K^ and A stored transposed: [a][t], [s][t]
    static constexpr int VS = BC + 16;     // V [t][column]
    static_assert(E == 64 || E == 128, "chunked form: heads of 64 or 128");
    static_assert(I4 == 256 && GL <= 2, "prefetch slots");
};

template <int E>
__global__ __launch_bounds__(256, 2) void hgrn2_chunk_kernel(const float *__restrict__ f, const float *__restrict__ xi,
                                                          const float *__restrict__ o, const float *s0, float *y,
                                                          float *s_last, int64_t t, int64_t d, int heads) {
    using Sh = H2Chunk<E>;
    constexpr int C = Sh::C, BC = Sh::BC, AT = Sh::AT, RA = Sh::RA, CBK = E / BC;
    constexpr int QS = Sh::QS, VS = Sh::VS;
    __shared__ __attribute__((aligned(16))) float sf[C * E];      // f of the chunk being prepared, [t][a]
    __shared__ __attribute__((aligned(16))) float so[C * E];      // o of that chunk, [t][a]
    __shared__ __attribute__((aligned(16))) float sv[C * VS];     // i of the chunk being read out, [t][column]
    __shared__ __attribute__((aligned(16))) float sq[2][E * QS];  // Q~, [a][t]
    __shared__ __attribute__((aligned(16))) float skt[2][E * QS]; // K~ or K^, [a][t]
    __shared__ __attribute__((aligned(16))) float sa[2][C * QS];  // A, [s][t]
    __shared__ float sdec[2][E];                                   // prod f over the chunk
    __shared__ __attribute__((aligned(16))) float spart[4][C * C]; // the waves' partial A tiles, [t][s]

    const int G = gridDim.x, g = blockIdx.x;
    const int lin = (G & 7) == 0 ? (g & 7) * (G >> 3) + (g >> 3) : g;
    const int pair = lin / CBK, cblk = lin - pair * CBK;
    const int64_t bi = pair / heads;
    const int head = pair - (int)bi * heads;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
    const int64_t col0 = (int64_t)head * E;
    const int64_t ccol0 = col0 + (int64_t)cblk * BC;
    const int64_t row_base = bi * t * d;
    const int64_t sbase = ((int64_t)pair * E) * E + (int64_t)cblk * BC + 16 * wave;  // state (pair, 0, wave's first column)
    const int64_t nch = (t + C - 1) / C;
    auto tokens = [&](int64_t c) __attribute__((always_inline)) { return t - c * C < C ? (int)(t - c * C) : C; };

    // ---- gate and input traffic: loads into registers, parked in LDS an iteration later;
    // byte offsets within the sequence, rows past its end read as zeros
    const int seq_bytes = (int)(t * d * 4);
    const auto rf = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(f + row_base), 0, seq_bytes, kBufferWord3);
    const auto ro = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(o + row_base), 0, seq_bytes, kBufferWord3);
    const auto ri = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(xi + row_base), 0, seq_bytes, kBufferWord3);
    const auto ry = __builtin_amdgcn_make_buffer_rsrc(y + row_base, 0, seq_bytes, kBufferWord3);
    const int row_bytes = (int)d * 4;
    auto ld4 = [](__amdgpu_buffer_rsrc_t r, int off) __attribute__((always_inline)) {
        return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    };
    float4 pf0, pf1, po0, po1, pi0;
    auto fetch_gates = [&](int64_t c) __attribute__((always_inline)) {
        // chunks past the last read as zeros; the offset stays in int range for any c the loop reaches
        const int crow = (int)(c < nch ? c : nch) * C;
        {
            const int k = tid / (E / 4), c4 = tid - k * (E / 4);
            const int off = (crow + k) * row_bytes + (int)(col0 + 4 * c4) * 4;
            pf0 = ld4(rf, off);
            po0 = ld4(ro, off);
        }
        if constexpr (Sh::GL == 2) {
            const int q = tid + 256, k = q / (E / 4), c4 = q - k * (E / 4);
            const int off = (crow + k) * row_bytes + (int)(col0 + 4 * c4) * 4;
            pf1 = ld4(rf, off);
            po1 = ld4(ro, off);
        }
    };
    auto fetch_input = [&](int64_t c) __attribute__((always_inline)) {
        const int crow = (int)(c < nch ? c : nch) * C;
        const int k = tid / (BC / 4), c4 = tid - k * (BC / 4);
        pi0 = ld4(ri, (crow + k) * row_bytes + (int)(ccol0 + 4 * c4) * 4);
    };
    // tokens at or past `nk` of the chunk become f = 1, o = 0, i = 0 (selected per
    // component: a select of whole float4 values would go through memory)
    auto or4 = [](bool in, float4 v, float w) __attribute__((always_inline)) {
        return make_float4(in ? v.x : w, in ? v.y : w, in ? v.z : w, in ? v.w : w);
    };
    auto park_gates = [&](int nk) __attribute__((always_inline)) {
        {
            const bool in = tid / (E / 4) < nk;
            *reinterpret_cast<float4 *>(sf + 4 * tid) = or4(in, pf0, 1.0f);
            *reinterpret_cast<float4 *>(so + 4 * tid) = or4(in, po0, 0.0f);
        }
        if constexpr (Sh::GL == 2) {
            const int q = tid + 256;
            const bool in = q / (E / 4) < nk;
            *reinterpret_cast<float4 *>(sf + 4 * q) = or4(in, pf1, 1.0f);
            *reinterpret_cast<float4 *>(so + 4 * q) = or4(in, po1, 0.0f);
        }
    };
    auto park_input = [&](int nk) __attribute__((always_inline)) {
        *reinterpret_cast<float4 *>(sv + (tid / (BC / 4)) * VS + 4 * (tid % (BC / 4))) =
            or4(tid / (BC / 4) < nk, pi0, 0.0f);
    };

    // ---- decays of the parked chunk, one thread per row a: Q~, K~ (into skt) and the total
    // decay; returns whether a gate is below the floor that keeps 1 / prod f in range
    auto prepare = [&](int bf) __attribute__((always_inline)) {
        bool tiny = false;
        if (tid < E) {
            const int a = tid;
            float p = 1.0f;
#pragma unroll
            for (int k = 0; k < C; ++k) {
                const float fk = sf[k * E + a];
                tiny |= fk < kChunkMinGate;
                p *= fk;
                sq[bf][a * QS + k] = so[k * E + a] * p;
                skt[bf][a * QS + k] = (1.0f - fk) * __builtin_amdgcn_rcpf(p);
            }
            sdec[bf][a] = p;
        }
        return tiny;
    };
    // A = Q~ K~^T on MFMA, the E rows split over the four waves; each wave's partial tile,
    // entries with s > t dropped, goes to spart
    auto a_partial = [&](int bf) __attribute__((always_inline)) {
        f32x4v pa = {0.f, 0.f, 0.f, 0.f};
        float qa[E / 16], kb[E / 16];
#pragma unroll
        for (int q = 0; q < E / 16; ++q) {
            const int row = wave * (E / 4) + 4 * q + lg;
            qa[q] = sq[bf][row * QS + l16];
            kb[q] = skt[bf][row * QS + l16];
        }
#pragma unroll
        for (int q = 0; q < E / 16; ++q) pa = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[q], kb[q], pa, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) spart[wave][(4 * lg + j) * 16 + l16] = pa[j];  // [t][s]
    };
    // the partial tiles summed in a fixed order, s > t set to 0
    auto a_reduce = [&](int bf) __attribute__((always_inline)) {
        const int tI = tid >> 4, sI = tid & 15;
        const float v =
            ((spart[0][tI * 16 + sI] + spart[1][tI * 16 + sI]) + spart[2][tI * 16 + sI]) + spart[3][tI * 16 + sI];
        sa[bf][sI * QS + tI] = sI <= tI ? v : 0.0f;
    };
    // a chunk with a small gate: A[t][s] from running products of its gates (thread (s, ac)
    // sums rows ac*RA .. ac*RA+RA-1, the 16 ac meet by DPP) and K^ as suffix products, both
    // from the gates still parked in sf / so
    auto a_direct = [&](int bf) __attribute__((always_inline)) {
        const int sI = tid >> 4, ac = tid & 15;
        float dk[RA];
#pragma unroll
        for (int r = 0; r < RA; ++r) dk[r] = 1.0f - sf[sI * E + ac * RA + r];
#pragma unroll
        for (int k = 0; k < C; ++k) {
            float pk = 0.0f;
#pragma unroll
            for (int r = 0; r < RA; ++r) {
                if (k > sI) dk[r] *= sf[k * E + ac * RA + r];
                pk = fmaf(so[k * E + ac * RA + r], dk[r], pk);
            }
            pk = k >= sI ? pk : 0.0f;
            pk += dpp_f<kDppXor1>(pk);
            pk += dpp_f<kDppXor2>(pk);
            pk += dpp_f<kDppHalfMirror>(pk);
            pk += dpp_f<kDppMirror>(pk);
            if (ac == 0) sa[bf][sI * QS + k] = pk;
        }
        if (tid < E) {
            float suf = 1.0f;
#pragma unroll
            for (int k = C - 1; k >= 0; --k) {
                const float fk = sf[k * E + tid];
                skt[bf][tid * QS + k] = (1.0f - fk) * suf;
                suf *= fk;
            }
        }
    };

    // the wave's state slice in accumulator layout, column 16 wave + l16: st[i][j] holds row
    // 16i + lg + 4j. The update's output row m = 4 lg + j of tile i is taken to be state row
    // 16i + (m >> 2) + 4 (m & 3) (the order of its K~/K^ operand rows), so that for Q~ S0 the
    // register st[i][j] is the B operand of the K step whose lane group lg is row 16i + 4j + lg
    float st[AT][4];
    // ---- Y = Q~ S0 + A V for the wave's 16 columns, then S1 = diag(decay) S0 + K^T V
    auto read_out = [&](int bf, bool direct, int64_t t0) __attribute__((always_inline)) {
        f32x4v y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < AT; ++i)
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
                y0 = __builtin_amdgcn_mfma_f32_16x16x4f32(sq[bf][(16 * i + 4 * j + lg) * QS + l16], st[i][j], y0, 0, 0,
                                                          0);
                y1 = __builtin_amdgcn_mfma_f32_16x16x4f32(sq[bf][(16 * i + 4 * j + 4 + lg) * QS + l16], st[i][j + 1],
                                                          y1, 0, 0, 0);
            }
#pragma unroll
        for (int q = 0; q < C / 4; q += 2) {
            y0 = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[bf][(4 * q + lg) * QS + l16],
                                                      sv[(4 * q + lg) * VS + 16 * wave + l16], y0, 0, 0, 0);
            y1 = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[bf][(4 * q + 4 + lg) * QS + l16],
                                                      sv[(4 * q + 4 + lg) * VS + 16 * wave + l16], y1, 0, 0, 0);
        }
        const f32x4v yacc = y0 + y1;
        // S1 = diag(decay) S0 + K^T V; K^ = K~ * total decay (skt holds K^ itself in a direct chunk)
        float kv[C / 4], ka[AT][C / 4];
        const int prow = (l16 >> 2) + 4 * (l16 & 3);  // state row of operand row l16 within a tile
#pragma unroll
        for (int i = 0; i < AT; ++i) {
            const float ks = direct ? 1.0f : sdec[bf][16 * i + prow];
#pragma unroll
            for (int q = 0; q < C / 4; ++q) ka[i][q] = skt[bf][(16 * i + prow) * QS + 4 * q + lg] * ks;
        }
#pragma unroll
        for (int q = 0; q < C / 4; ++q) kv[q] = sv[(4 * q + lg) * VS + 16 * wave + l16];
        f32x4v acc[AT];
#pragma unroll
        for (int i = 0; i < AT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = st[i][j] * sdec[bf][16 * i + lg + 4 * j];
#pragma unroll
        for (int q = 0; q < C / 4; ++q)
#pragma unroll
            for (int i = 0; i < AT; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[i][q], kv[q], acc[i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < AT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) st[i][j] = acc[i][j];
        // the chunk's outputs: row 4 lg + j, column 16 wave + l16 (rows past the end are dropped)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yacc[j]), ry,
                                                  ((int)t0 + 4 * lg + j) * row_bytes + (int)(ccol0 + 16 * wave + l16) * 4,
                                                  0, 0);
    };

    if (nch > 0) {
        fetch_gates(0);
        fetch_input(0);
    }
    if (s0) {
#pragma unroll
        for (int i = 0; i < AT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) st[i][j] = s0[sbase + (int64_t)(16 * i + lg + 4 * j) * E + l16];
    } else {
#pragma unroll
        for (int i = 0; i < AT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) st[i][j] = 0.0f;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the state and the first chunk have landed

    // prologue: chunk 0 parked and prepared; its A, chunk 1 parked and prepared, chunk 0's input
    // parked. `direct0` / `direct1` say how chunks k and k+1 were prepared
    bool direct0 = false, direct1 = false;
    if (nch > 0) {
        park_gates(tokens(0));
        fetch_gates(1);
        __syncthreads();
        direct1 = __syncthreads_or(prepare(0));
        if (direct1) a_direct(0);
        else a_partial(0);
        if (nch > 1) {
            if (direct1) __syncthreads();  // the direct sums read chunk 0's gates in sf / so
            park_gates(tokens(1));
        }
        fetch_gates(2);
        __syncthreads();
        if (!direct1) a_reduce(0);
        park_input(tokens(0));
        fetch_input(1);
        const bool tiny = nch > 1 ? prepare(1) : false;
        direct0 = direct1;
        direct1 = __syncthreads_or(tiny);
        // vmcnt(0), once: the loop is entered with nothing in flight, so the waits in its body
        // count only the loop's own loads and stores
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    // iteration k: A of chunk k+1 and chunk k+2 parked, chunk k read out; then chunk k+1's A
    // summed and its input parked, chunk k+2 prepared. Every iteration issues the same loads
    // and stores; only LDS and MFMA work depends on which chunks exist
    for (int64_t k = 0; k < nch; ++k) {
        const bool has1 = k + 1 < nch, has2 = k + 2 < nch;
        if (has1) {
            if (direct1) a_direct((int)((k + 1) & 1));
            else a_partial((int)((k + 1) & 1));
        }
        if (has2) {
            if (has1 && direct1) __syncthreads();  // the direct sums read chunk k+1's gates in sf / so
            park_gates(tokens(k + 2));
        }
        fetch_gates(k + 3);
        read_out((int)(k & 1), direct0, k * C);
        __syncthreads();  // spart, the parked gates; every read of chunk k's buffers and of sv done
        if (has1) {
            if (!direct1) a_reduce((int)((k + 1) & 1));
            park_input(tokens(k + 1));
        }
        fetch_input(k + 2);
        const bool tiny = has2 ? prepare((int)((k + 2) & 1)) : false;
        const bool direct2 = __syncthreads_or(tiny);  // chunk k+1's A and V, chunk k+2's decays in LDS
        direct0 = direct1;
        direct1 = direct2;
    }

    if (s_last) {
#pragma unroll
        for (int i = 0; i < AT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s_last[sbase + (int64_t)(16 * i + lg + 4 * j) * E + l16] = st[i][j];
    }
}

int64_t hgrn2_workgroups(int64_t b, int64_t d, int e) {
    const int bc = e == 16 ? H2Shape<16>::BC : e == 32 ? H2Shape<32>::BC : e == 64 ? H2Shape<64>::BC
                                                                                 : H2Shape<128>::BC;
    return b * (d / e) * (e / bc);
}

hipError_t launch_hgrn2_scan(const float *f, const float *i, const float *o, const float *s0, float *y,
                             float *s_last, int64_t b, int64_t t, int64_t d, int e, bool chunk, hipStream_t st,
                             const char **name) {
    const int heads = (int)(d / e);
    const unsigned grid = (unsigned)hgrn2_workgroups(b, d, e);
    if (grid == 0) return hipSuccess;
    if (chunk) {
        switch (e) {
            case 64: launch_k(hgrn2_chunk_kernel<64>, grid, 256, 0, st, f, i, o, s0, y, s_last, t, d, heads); break;
            case 128: launch_k(hgrn2_chunk_kernel<128>, grid, 256, 0, st, f, i, o, s0, y, s_last, t, d, heads); break;
            default: return hipErrorInvalidValue;
        }
        if (name) *name = e == 64 ? "hgrn2_chunk<64>" : "hgrn2_chunk<128>";
        return hipGetLastError();
    }
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
