// HGRN recurrence h_t = f_t * h_{t-1} + x_t per (batch, channel), fp32 (gfx950).
//
// The recurrence and its two implementations -- step-wise and chunked -- are
// those of the MatMul-free LM ("MatMul-Free LLM 深度分析报告", section
// "核心价值提炼", table "创新之处" and list "可复用的模式与技巧").
//
// The scan is HBM-bound: 12 bytes per (b, t, c) (read x and f, write h).
// Channels are contiguous, so one lane per channel gives fully coalesced
// 256-byte wave accesses at every step; loads of a block of U steps are issued
// before the dependent chain of that block runs.
//  * recurrent: one lane runs the whole sequence of its channel.
//  * tiled (single pass, chunked): a workgroup of W waves owns 64 channels of
//    one sequence and walks it in chunks of W*S steps. Wave w reduces its S
//    steps of the chunk to the pair (A = prod f, B = h started from 0); the W
//    pairs meet in LDS; each wave folds the pairs before its own into the
//    chunk's carry, h_in = A*h_in + B, and re-runs its S steps from there. The
//    loads of the next P chunks are in flight during a chunk's arithmetic and
//    every element is read once, with streaming (non-temporal) loads and
//    stores: 12 bytes per (b, t, c). Used when there are enough (sequence,
//    64-channel) groups to occupy the GPU.
//  * two-pass chunked: t is split into C chunks. Pass 1 reduces each chunk but
//    the last to its pair; pass 2 lane (b, j, c) folds the pairs of chunks < j
//    into its carry and re-runs chunk j from it. C lanes per channel fill the
//    GPU when b*d is small; the price is re-reading the first C-1 chunks.
#include "device_common.hpp"
#include "launch.hpp"

#include <atomic>

namespace mmf {

constexpr int kScanU = 8;

// Runs steps [t0, t1) of one channel from state h (strided by d), writing h
// when out != nullptr. Returns the state after step t1-1.
__device__ __forceinline__ float scan_run(const float *x, const float *f, float *out, int64_t d, int64_t t0,
                                          int64_t t1, float h) {
    int64_t t = t0;
    for (; t + kScanU <= t1; t += kScanU) {
        float xa[kScanU], fa[kScanU];
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            xa[u] = x[(t + u) * d];
            fa[u] = f[(t + u) * d];
        }
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            h = fa[u] * h + xa[u];
            if (out) out[(t + u) * d] = h;
        }
    }
    for (; t < t1; ++t) {
        h = f[t * d] * h + x[t * d];
        if (out) out[t * d] = h;
    }
    return h;
}

__global__ __launch_bounds__(256) void scan_recurrent_kernel(const float *x, const float *f, const float *h0,
                                                             float *h, float *h_last, int64_t b, int64_t t,
                                                             int64_t d) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= b * d) return;
    const int64_t bi = gid / d, c = gid % d;
    const int64_t base = bi * t * d + c;
    float state = h0 ? h0[gid] : 0.0f;
    state = scan_run(x + base, f + base, h + base, d, 0, t, state);
    if (h_last) h_last[gid] = state;
}

// Pass 1: pair (prod f, h from 0) of chunk j < C-1.
__global__ __launch_bounds__(256) void scan_chunk_reduce_kernel(const float *__restrict__ x,
                                                                const float *__restrict__ f, int64_t b,
                                                                int64_t t, int64_t d, int chunks, int64_t clen,
                                                                float2 *__restrict__ agg) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_b = (int64_t)(chunks - 1) * d;
    if (gid >= b * per_b) return;
    const int64_t bi = gid / per_b;
    const int64_t j = (gid % per_b) / d;
    const int64_t c = gid % d;
    const int64_t t0 = j * clen;
    const int64_t t1 = t0 + clen < t ? t0 + clen : t;
    const float *xp = x + bi * t * d + c;
    const float *fp = f + bi * t * d + c;
    float a = 1.0f, hb = 0.0f;
    int64_t s = t0;
    for (; s + kScanU <= t1; s += kScanU) {
        float xa[kScanU], fa[kScanU];
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            xa[u] = xp[(s + u) * d];
            fa[u] = fp[(s + u) * d];
        }
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            hb = fa[u] * hb + xa[u];
            a = a * fa[u];
        }
    }
    for (; s < t1; ++s) {
        const float fv = fp[s * d];
        hb = fv * hb + xp[s * d];
        a = a * fv;
    }
    agg[(bi * (chunks - 1) + j) * d + c] = make_float2(a, hb);
}

// Pass 2: carry into chunk j, then chunk j itself.
__global__ __launch_bounds__(256) void scan_chunk_apply_kernel(const float *x, const float *f, const float *h0,
                                                               float *h, float *h_last, int64_t b, int64_t t,
                                                               int64_t d, int chunks, int64_t clen,
                                                               const float2 *__restrict__ agg) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_b = (int64_t)chunks * d;
    if (gid >= b * per_b) return;
    const int64_t bi = gid / per_b;
    const int j = (int)((gid % per_b) / d);
    const int64_t c = gid % d;
    float state = h0 ? h0[bi * d + c] : 0.0f;
    const float2 *ag = agg + bi * (int64_t)(chunks - 1) * d + c;
    for (int jj = 0; jj < j; ++jj) {
        const float2 p = ag[(int64_t)jj * d];
        state = p.x * state + p.y;
    }
    const int64_t t0 = (int64_t)j * clen;
    const int64_t t1 = t0 + clen < t ? t0 + clen : t;
    const int64_t base = bi * t * d + c;
    state = scan_run(x + base, f + base, h + base, d, t0, t1, state);
    if (h_last && j == chunks - 1) h_last[bi * d + c] = state;
}

// Every element of x, f and h is touched once; with NT the accesses are
// marked non-temporal (worth it once the three tensors outgrow the 256 MB
// memory-side cache, where a normal access could still hit).
template <bool NT>
__device__ __forceinline__ float ld_stream(const float *p) { return NT ? __builtin_nontemporal_load(p) : *p; }
template <bool NT>
__device__ __forceinline__ void st_stream(float *p, float v) {
    if (NT) __builtin_nontemporal_store(v, p); else *p = v;
}

// CW channels per workgroup (64, or 32 when the (sequence, channel-group) pairs
// are too few to fill the GPU at 64): with 32, the two half-waves share their
// wave's S steps of a chunk, SL = S / 2 each, and the 2W segments of a chunk
// fold in time order (wave, half).
template <int W, int S, int P, bool NT, int CW = 64>
__global__ __launch_bounds__(W * 64) void scan_tiled_kernel(const float *x, const float *f, const float *h0,
                                                            float *h, float *h_last, int64_t t, int64_t d,
                                                            int64_t groups) {
    constexpr int CH = W * S;    // steps per chunk; P chunks of loads run ahead of the arithmetic
    constexpr int HS = 64 / CW;  // lanes per channel, each with SL consecutive steps of its wave's S
    constexpr int SL = S / HS;
    static_assert(CW * HS == 64 && SL * HS == S, "a wave covers CW channels x S steps");
    __shared__ float2 pairs[2][W][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lc = lane % CW, hs = lane / CW;
    const int64_t bi = blockIdx.x / groups;
    const int64_t c = (blockIdx.x % groups) * CW + lc;
    const bool live = c < d;
    const int64_t cl = live ? c : d - 1;  // loads of idle lanes stay in bounds
    const float *xp = x + bi * t * d + cl;
    const float *fp = f + bi * t * d + cl;
    float *hp = h + bi * t * d + c;
    float carry = (h0 && live) ? h0[bi * d + c] : 0.0f;
    const int64_t nchunks = (t + CH - 1) / CH;
    float fa[P + 1][SL], xa[P + 1][SL];  // [0] = current chunk, [1..P] = chunks in flight
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int s = 0; s < SL; ++s) {
            const int64_t ts = min((int64_t)(p * CH + w * S + hs * SL + s), t - 1);
            fa[p][s] = ld_stream<NT>(fp + ts * d);
            xa[p][s] = ld_stream<NT>(xp + ts * d);
        }
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = ch * CH + w * S + hs * SL;
        if (ch + P < nchunks) {
#pragma unroll
            for (int s = 0; s < SL; ++s) {
                const int64_t ts = min(t0 + P * CH + s, t - 1);
                fa[P][s] = ld_stream<NT>(fp + ts * d);
                xa[P][s] = ld_stream<NT>(xp + ts * d);
            }
        }
        // steps past the end act as the identity (f = 1, x = 0)
        float a = 1.0f, bb = 0.0f;
#pragma unroll
        for (int s = 0; s < SL; ++s) {
            const bool in = t0 + s < t;
            fa[0][s] = in ? fa[0][s] : 1.0f;
            xa[0][s] = in ? xa[0][s] : 0.0f;
            bb = fa[0][s] * bb + xa[0][s];
            a = a * fa[0][s];
        }
        pairs[ch & 1][w][lane] = make_float2(a, bb);
        __syncthreads();
        // fold: the state entering this lane's segment, and the state after the whole chunk
        float hin = carry, cn = carry;
#pragma unroll
        for (int v = 0; v < W; ++v)
#pragma unroll
            for (int u = 0; u < HS; ++u) {
                if (v == w && u == hs) hin = cn;
                const float2 pr = pairs[ch & 1][v][u * CW + lc];
                cn = pr.x * cn + pr.y;
            }
        float hv = hin;
#pragma unroll
        for (int s = 0; s < SL; ++s) {
            hv = fa[0][s] * hv + xa[0][s];
            if (live && t0 + s < t) st_stream<NT>(hp + (t0 + s) * d, hv);
        }
        carry = cn;
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int s = 0; s < SL; ++s) {
                fa[p][s] = fa[p + 1][s];
                xa[p][s] = xa[p + 1][s];
            }
    }
    if (h_last && live && hs == 0) h_last[bi * d + c] = carry;
}

// ----------------------------------------------------------------------------
// Backward of the recurrence (reverse time)
// ----------------------------------------------------------------------------
// With d_t the whole derivative of the loss with respect to h_t (through h_t
// itself and through every later step):
//   d_t = dh_t + f_{t+1} d_{t+1},   d_{T-1} = dh_{T-1} + dh_last
//   dx_t = d_t,   df_t = d_t h_{t-1},   dh0 = f_0 d_0      (h_{-1} = h0 or 0)
// which is the forward recurrence run from t = T-1 down, with f shifted by one
// step (f_T taken as 1) and the carry starting at dh_last; chunk carries
// compose as the same (prod f, partial) pairs. 20 bytes per (b, t, c): read
// dh, f and h, write dx and df. dx may be dh (every element is read before it
// is written, by the same lane).
__global__ __launch_bounds__(256) void scan_bwd_recurrent_kernel(const float *f, const float *h, const float *h0,
                                                                 const float *dh, const float *dh_last, float *dx,
                                                                 float *df, float *dh0, int64_t b, int64_t t,
                                                                 int64_t d) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= b * d) return;
    const int64_t bi = gid / d, c = gid % d;
    const int64_t base = bi * t * d + c;
    const float *fp = f + base, *hp = h + base, *gp = dh + base;
    float *xo = dx + base, *fo = df + base;
    const float hinit = h0 ? h0[gid] : 0.0f;
    float carry = dh_last ? dh_last[gid] : 0.0f;
    float fnext = 1.0f;  // f_{s+1} of the step s being taken
    int64_t s = t - 1;
    for (; s + 1 >= kScanU; s -= kScanU) {  // steps s, s-1, ..., s-U+1
        float ga[kScanU], fa[kScanU], ha[kScanU];
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int64_t ts = s - u;
            ga[u] = gp[ts * d];
            fa[u] = fp[ts * d];
            const float hv = hp[(ts > 0 ? ts - 1 : 0) * d];
            ha[u] = ts > 0 ? hv : hinit;
        }
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
            const int64_t ts = s - u;
            carry = fnext * carry + ga[u];
            xo[ts * d] = carry;
            fo[ts * d] = carry * ha[u];
            fnext = fa[u];
        }
    }
    for (; s >= 0; --s) {
        const float g = gp[s * d], fv = fp[s * d];
        const float hm = s > 0 ? hp[(s - 1) * d] : hinit;
        carry = fnext * carry + g;
        xo[s * d] = carry;
        fo[s * d] = carry * hm;
        fnext = fv;
    }
    if (dh0) dh0[gid] = fnext * carry;
}

// Tiled backward: the forward tiled kernel's scheme walked from the last chunk
// to the first. Wave w of a chunk owns its steps w*S .. w*S+S-1 and takes them
// from the last; the carry enters the chunk's last wave first, so wave w folds
// the pairs of the waves after it.
template <int W, int S, int P, bool NT>
__global__ __launch_bounds__(W * 64) void scan_bwd_tiled_kernel(const float *f, const float *h, const float *h0,
                                                                const float *dh, const float *dh_last, float *dx,
                                                                float *df, float *dh0, int64_t t, int64_t d,
                                                                int64_t groups) {
    constexpr int CH = W * S;
    __shared__ float2 pairs[2][W][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t bi = blockIdx.x / groups;
    const int64_t c = (blockIdx.x % groups) * 64 + lane;
    const bool live = c < d;
    const int64_t cl = live ? c : d - 1;  // loads of idle lanes stay in bounds
    const float *fp = f + bi * t * d + cl;
    const float *hp = h + bi * t * d + cl;
    const float *gp = dh + bi * t * d + cl;
    float *xo = dx + bi * t * d + c;
    float *fo = df + bi * t * d + c;
    const float hinit = (h0 && live) ? h0[bi * d + c] : 0.0f;
    float carry = (dh_last && live) ? dh_last[bi * d + c] : 0.0f;
    const int64_t nchunks = (t + CH - 1) / CH;
    // per step ts of a slot: dh_ts, f_{ts+1} and h_{ts-1} (indices clamped;
    // the values that fall outside [0, t) are replaced where they are used)
    float ga[P + 1][S], fa[P + 1][S], ha[P + 1][S];
    auto load = [&](int slot, int64_t ck) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int64_t ts = ck * CH + w * S + s;
            const int64_t tg = min(ts, t - 1), tf = min(ts + 1, t - 1);
            const int64_t th = ts > 0 ? min(ts - 1, t - 1) : 0;
            ga[slot][s] = ld_stream<NT>(gp + tg * d);
            fa[slot][s] = ld_stream<NT>(fp + tf * d);
            ha[slot][s] = ld_stream<NT>(hp + th * d);
        }
    };
#pragma unroll
    for (int p = 0; p < P; ++p) load(p, nchunks - 1 - p >= 0 ? nchunks - 1 - p : 0);
    for (int64_t k = 0; k < nchunks; ++k) {
        const int64_t ck = nchunks - 1 - k;
        const int64_t t0 = ck * CH + w * S;
        if (k + P < nchunks) load(P, ck - P);
        // this wave's steps, last first: steps past the end act as the identity
        float a = 1.0f, bb = 0.0f;
#pragma unroll
        for (int s = S - 1; s >= 0; --s) {
            const int64_t ts = t0 + s;
            fa[0][s] = ts + 1 < t ? fa[0][s] : 1.0f;
            ga[0][s] = ts < t ? ga[0][s] : 0.0f;
            ha[0][s] = ts > 0 ? ha[0][s] : hinit;
            bb = fa[0][s] * bb + ga[0][s];
            a = a * fa[0][s];
        }
        pairs[k & 1][w][lane] = make_float2(a, bb);
        __syncthreads();
        // fold from the chunk's last wave: the carry entering wave w, and after the chunk
        float hin = carry, cn = carry;
#pragma unroll
        for (int v = W - 1; v >= 0; --v) {
            if (v == w) hin = cn;
            const float2 pr = pairs[k & 1][v][lane];
            cn = pr.x * cn + pr.y;
        }
        float gs = hin;
#pragma unroll
        for (int s = S - 1; s >= 0; --s) {
            const int64_t ts = t0 + s;
            gs = fa[0][s] * gs + ga[0][s];
            if (live && ts < t) {
                st_stream<NT>(xo + ts * d, gs);
                st_stream<NT>(fo + ts * d, gs * ha[0][s]);
            }
        }
        carry = cn;
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int s = 0; s < S; ++s) {
                ga[p][s] = ga[p + 1][s];
                fa[p][s] = fa[p + 1][s];
                ha[p][s] = ha[p + 1][s];
            }
    }
    if (dh0 && live && w == 0) dh0[bi * d + c] = fp[0] * carry;
}

__global__ void copy_state_kernel(const float *h0, float *h_last, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) h_last[i] = h0 ? h0[i] : 0.0f;
}

size_t scan_workspace_bytes(int64_t b, int64_t d, int chunks) {
    return chunks > 1 ? (size_t)b * (size_t)(chunks - 1) * (size_t)d * sizeof(float2) : 0;
}

constexpr int64_t kTiledMinGroups = 128;     // (sequence, 64-channel) groups that occupy the GPU
constexpr int64_t kTiledManyGroups = 512;    // from here 4-wave workgroups (more chunks in flight)
constexpr int64_t kStreamBytes = 256ll << 20;  // x, f and h together beyond the memory-side cache

// Plan: 1 = recurrent, kScanTiled = single-pass tiled, c >= 2 = two-pass with c
// chunks. Recurrent for explicit requests, t = 1, and (auto) short sequences;
// tiled when there are enough channel groups; otherwise two passes with enough
// chunks for ~128k lanes, each chunk at least 64 steps.
int scan_pick_chunks(int64_t b, int64_t t, int64_t d, int mode) {
    if (mode == 1 || t <= 1) return 1;
    if (b * ((d + 63) / 64) >= kTiledMinGroups) return (mode == 0 && t < 64) ? 1 : kScanTiled;
    const int64_t lanes = b * d;
    int64_t c = (131072 + lanes - 1) / lanes;
    if (mode == 2 && c < 2) c = 2;
    const int64_t max_c = t / 64 > 1 ? t / 64 : (mode == 2 ? t : 1);
    if (c > max_c) c = max_c;
    if (c > 256) c = 256;
    if (c < 1) c = 1;
    if (mode == 2 && c < 2 && t >= 2) c = 2;
    return (int)c;
}

int scan_bwd_pick(int64_t t, int mode) {
    if (mode == 1 || t <= 1 || (mode == 0 && t < 64)) return 1;
    return kScanTiled;
}

hipError_t launch_scan_bwd(const float *f, const float *h, const float *h0, const float *dh, const float *dh_last,
                           float *dx, float *df, float *dh0, int64_t b, int64_t t, int64_t d, int plan,
                           hipStream_t stream, std::string *path) {
    if (b <= 0) return hipSuccess;
    if (t == 0) {
        // h_last is h0: its derivative passes straight through
        if (dh0) launch_k(copy_state_kernel, (unsigned)((b * d + 255) / 256), 256, 0, stream, dh_last, dh0, b * d);
        if (path) *path += "scan_bwd_empty;";
        return hipGetLastError();
    }
    if (plan == kScanTiled) {
        const int64_t groups = (d + 63) / 64;
        const unsigned grid = (unsigned)(b * groups);
        const bool nt = 20 * b * t * d > kStreamBytes;
        const bool many = b * groups >= kTiledManyGroups;
        // measured on MI355X: 4-wave workgroups of 4 steps per wave with 6 chunks
        // ahead once the groups fill the GPU (71 % of 8 TB/s at 16 x 2048 x 2048,
        // 63 % with 8 steps and 3 ahead)
        if (many && nt)
            launch_k(scan_bwd_tiled_kernel<4, 4, 6, true>, grid, 256, 0, stream, f, h, h0, dh, dh_last, dx, df, dh0, t, d, groups);
        else if (many)
            launch_k(scan_bwd_tiled_kernel<4, 4, 6, false>, grid, 256, 0, stream, f, h, h0, dh, dh_last, dx, df, dh0, t, d, groups);
        else if (nt)
            launch_k(scan_bwd_tiled_kernel<16, 8, 1, true>, grid, 1024, 0, stream, f, h, h0, dh, dh_last, dx, df, dh0, t, d, groups);
        else
            launch_k(scan_bwd_tiled_kernel<16, 8, 1, false>, grid, 1024, 0, stream, f, h, h0, dh, dh_last, dx, df, dh0, t, d, groups);
        if (path) *path += std::string("scan_bwd_tiled<") + (many ? "4w" : "16w") + (nt ? ",nt" : "") + ">;";
        return hipGetLastError();
    }
    launch_k(scan_bwd_recurrent_kernel, (unsigned)((b * d + 255) / 256), 256, 0, stream, f, h, h0, dh, dh_last, dx, df,
                                                                                   dh0, b, t, d);
    if (path) *path += "scan_bwd_recurrent;";
    return hipGetLastError();
}

// Compute units of the current device (cached per device).
static int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_scan(const float *x, const float *f, const float *h0, float *h, float *h_last, int64_t b,
                       int64_t t, int64_t d, int chunks, void *ws, hipStream_t stream, std::string *path) {
    if (b <= 0) return hipSuccess;
    if (t == 0) {
        if (h_last) launch_k(copy_state_kernel, (unsigned)((b * d + 255) / 256), 256, 0, stream, h0, h_last, b * d);
        if (path) *path += "scan_empty;";
        return hipGetLastError();
    }
    if (chunks == kScanTiled) {
        // geometry measured on MI355X: 16-wave workgroups (8 steps each, one chunk
        // ahead) while (sequence, channel-group) pairs are few; 4-wave
        // workgroups with 2 chunks ahead once they fill the GPU (72 % of 8 TB/s
        // at 16 x 2048 x 2048 against 69 % with 4 ahead)
        // fewer pairs than that, but twice as many 32-channel pairs still no more than
        // one workgroup per CU: groups of 32 channels, 16 steps per wave (the 370M
        // prefill, 8 x 2048 x 1024: 68.7 -> 51.3 us; at 4 x 4096 x 2560 the 320
        // workgroups took two rounds on 256 CUs and were slower, 130 -> 140 us)
        const bool nt = 12 * b * t * d > kStreamBytes;
        const bool many = b * ((d + 63) / 64) >= kTiledManyGroups;
        const bool half = !many && b * ((d + 31) / 32) <= cu_count();
        const int64_t groups = half ? (d + 31) / 32 : (d + 63) / 64;
        const unsigned grid = (unsigned)(b * groups);
        if (many && nt) launch_k(scan_tiled_kernel<4, 8, 2, true>, grid, 256, 0, stream, x, f, h0, h, h_last, t, d, groups);
        else if (many) launch_k(scan_tiled_kernel<4, 8, 2, false>, grid, 256, 0, stream, x, f, h0, h, h_last, t, d, groups);
        else if (half && nt) launch_k(scan_tiled_kernel<16, 16, 1, true, 32>, grid, 1024, 0, stream, x, f, h0, h, h_last, t, d, groups);
        else if (half) launch_k(scan_tiled_kernel<16, 16, 1, false, 32>, grid, 1024, 0, stream, x, f, h0, h, h_last, t, d, groups);
        else if (nt) launch_k(scan_tiled_kernel<16, 8, 1, true>, grid, 1024, 0, stream, x, f, h0, h, h_last, t, d, groups);
        else launch_k(scan_tiled_kernel<16, 8, 1, false>, grid, 1024, 0, stream, x, f, h0, h, h_last, t, d, groups);
        if (path) *path += std::string("scan_tiled<") + (many ? "4w" : half ? "16w,32c" : "16w") + (nt ? ",nt" : "") + ">;";
        return hipGetLastError();
    }
    if (chunks <= 1) {
        launch_k(scan_recurrent_kernel, (unsigned)((b * d + 255) / 256), 256, 0, stream, x, f, h0, h, h_last, b, t, d);
        if (path) *path += "scan_recurrent;";
        return hipGetLastError();
    }
    const int64_t clen = (t + chunks - 1) / chunks;
    const int c_eff = (int)((t + clen - 1) / clen);
    float2 *agg = static_cast<float2 *>(ws);
    if (c_eff > 1) {
        const int64_t n1 = b * (int64_t)(c_eff - 1) * d;
        launch_k(scan_chunk_reduce_kernel, (unsigned)((n1 + 255) / 256), 256, 0, stream, x, f, b, t, d, c_eff, clen, agg);
    }
    const int64_t n2 = b * (int64_t)c_eff * d;
    launch_k(scan_chunk_apply_kernel, (unsigned)((n2 + 255) / 256), 256, 0, stream, x, f, h0, h, h_last, b, t, d, c_eff,
                                                                              clen, agg);
    if (path) *path += "scan_chunk(" + std::to_string(c_eff) + "x" + std::to_string(clen) + ");";
    return hipGetLastError();
}

}  // namespace mmf
