// C ABI of libmmf (declared in include/mmf.h): argument validation, workspace
// carving and the order of kernel launches for a FusedBitLinear, the HGRN
// scan and one HGRNBit block ("MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，
// 剩下什麼", section "HGRNBitBlock 的結構").
//
// Validation happens on the host before any HIP call; errors set a
// thread-local message. Each call records the kernel variants it launched
// (mmf_last_path), so a caller can see which path ran: the same page, section
// "什麼情況下這個工具是錯的選擇", names a silent fallback to a slow path as a
// failure mode.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>
#include <cstring>
#include <atomic>
#include <mutex>

#include "mmf.h"
#include "launch.hpp"
#include "stack.hpp"
#include "ceiling.hpp"

using namespace mmf;

namespace {

thread_local std::string g_err;
thread_local std::string g_path;

mmf_status fail(mmf_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

mmf_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MMF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    g_err.clear();
    return MMF_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- optional per-launch timing (mmf_timing_enable) ----------------------------
struct TimingRec {
    std::string kernel;
    int64_t m;
    int n, k;
    hipEvent_t start, stop;
};
thread_local bool g_timing = false;
std::atomic<int> g_decode_mode{0};  // mmf_set_decode_kernel
thread_local std::vector<TimingRec> g_recs;
thread_local std::vector<hipEvent_t> g_events;
thread_local size_t g_events_used = 0;

hipEvent_t timing_event() {
    if (g_events_used == g_events.size()) {
        hipEvent_t e = nullptr;
        // without the system-scope fence an event costs the stream far less, so
        // the interval between a kernel's two events stays close to the kernel
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
        g_events.push_back(e);
    }
    return g_events[g_events_used++];
}

// The events bracket the launch on its stream: an interval runs from the point
// the stream reaches the first record to the point it reaches the second.
template <class F>
hipError_t timed(const std::string &kernel, int64_t m, int n, int k, hipStream_t st, F &&launch) {
    if (!g_timing) return launch();
    hipEvent_t a = timing_event(), b = timing_event();
    if (!a || !b) return hipErrorOutOfMemory;
    hipError_t e = hipEventRecord(a, st);
    if (e != hipSuccess) return e;
    if ((e = launch()) != hipSuccess) return e;
    if ((e = hipEventRecord(b, st)) != hipSuccess) return e;
    g_recs.push_back(TimingRec{kernel, m, n, k, a, b});
    return hipSuccess;
}

// The quantisers feed a contraction over the same m rows; when that
// contraction sums the codes itself, the quantiser does not.
hipError_t t_norm_quant(const void *x, ActType xt, int64_t m, int k, const float *gain, float eps, int8_t *q,
                        float *s, int32_t *sumq, hipStream_t st, std::string *path) {
    if (m <= 0) return hipSuccess;
    if (contract_sums_codes(m)) sumq = nullptr;
    return timed(xt == ACT_F32 ? "norm_quant<f32>" : "norm_quant<bf16>", m, k, k, st,
                 [&] { return launch_norm_quant(x, xt, m, k, gain, eps, q, s, sumq, st, path); });
}

hipError_t t_gnorm_quant(const float *h, const void *g, ActType gt, int64_t m, int d, const float *gw, const float *og,
                         float eps, int8_t *q, float *s, int32_t *sumq, float *u, hipStream_t st, std::string *path) {
    if (m <= 0) return hipSuccess;
    if (contract_sums_codes(m)) sumq = nullptr;
    return timed(gt == ACT_F32 ? "gnorm_quant<f32>" : "gnorm_quant<bf16>", m, d, d, st,
                 [&] { return launch_gnorm_quant(h, g, gt, m, d, gw, og, eps, q, s, sumq, u, st, path); });
}

hipError_t t_contract(const ContractArgs &a, EpiKind epi, int ng, bool shared, hipStream_t st, std::string *path) {
    if (a.m <= 0 || a.nc <= 0) return hipSuccess;
    return timed(contract_variant(a.m, a.k, epi, shared), a.m, ng * a.nc, a.k, st,
                 [&] { return launch_contract(a, epi, ng, shared, st, path); });
}

hipError_t t_scan(const float *x, const float *f, const float *h0, float *h, float *hl, int64_t b, int64_t t,
                  int64_t d, int chunks, void *ws, hipStream_t st, std::string *path) {
    return timed(chunks == kScanTiled ? "scan_tiled" : chunks > 1 ? "scan_chunk" : "scan_recurrent", b * t, (int)d,
                 (int)d, st,
                 [&] { return launch_scan(x, f, h0, h, hl, b, t, d, chunks, ws, st, path); });
}

constexpr int kMaxK = 65536;       // |sum t*q| <= 128*k stays exact in binary32
constexpr int kMaxNormRow = 8192;  // g_norm keeps a row in registers

// Carves 256-byte aligned buffers out of a workspace; with base == nullptr it
// only measures.
struct Carver {
    char *base;
    size_t off = 0;
    explicit Carver(void *b) : base(static_cast<char *>(b)) {}
    template <typename T>
    T *take(size_t count) {
        off = (off + 255) & ~size_t(255);
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

mmf_status check_weight(const mmf_ternary_weight *w, const char *name) {
    if (!w) return fail(MMF_ERR_INVALID_ARG, "%s: weight is NULL", name);
    if (!w->packed || !w->mu) return fail(MMF_ERR_INVALID_ARG, "%s: packed or mu is NULL", name);
    if (w->n <= 0 || w->k <= 0) return fail(MMF_ERR_INVALID_ARG, "%s: n=%d k=%d must be positive", name, w->n, w->k);
    if (w->k % 16) return fail(MMF_ERR_UNSUPPORTED, "%s: k=%d is not a multiple of 16", name, w->k);
    if (w->k > kMaxK) return fail(MMF_ERR_UNSUPPORTED, "%s: k=%d exceeds %d", name, w->k, kMaxK);
    if (!aligned16(w->packed) || (w->norm_w && !aligned16(w->norm_w)))
        return fail(MMF_ERR_INVALID_ARG, "%s: packed / norm_w must be 16-byte aligned", name);
    return MMF_OK;
}

bool valid_dtype(mmf_dtype t) { return t == MMF_F32 || t == MMF_BF16; }
ActType act(mmf_dtype t) { return t == MMF_F32 ? ACT_F32 : ACT_BF16; }

// ---------------------------------------------------------------- bitlinear --
struct BitlinearWs {
    int8_t *codes;
    float *s;
    int32_t *sumq;
};

size_t bitlinear_plan(Carver &c, int64_t m, int k, BitlinearWs *o) {
    BitlinearWs w;
    w.codes = c.take<int8_t>((size_t)m * k);
    w.s = c.take<float>((size_t)m);
    w.sumq = c.take<int32_t>((size_t)m);
    if (o) *o = w;
    return c.off;
}

// -------------------------------------------------------------------- layer --
struct LayerWs {
    int8_t *codes_x[3];
    float *s_x[3];
    int32_t *sq_x[3];
    float *f, *xt, *h, *x1;
    float *g, *z;  // fp32, whatever the activation dtype
    int8_t *codes_b;
    float *s_b;
    int32_t *sq_b;
    void *scan;
};

bool shared_ifg(const mmf_layer_weights *w) {
    return w->i.norm_w == w->f.norm_w && w->f.norm_w == w->g.norm_w;
}

size_t layer_plan(Carver &c, const mmf_layer_weights *w, int64_t b, int64_t t, int chunks, LayerWs *o) {
    const int64_t m = b * t;
    const size_t d = (size_t)w->d, inner = (size_t)w->inner;
    const int nq = shared_ifg(w) ? 1 : 3;
    LayerWs L{};
    for (int q = 0; q < nq; ++q) {
        L.codes_x[q] = c.take<int8_t>(m * d);
        L.s_x[q] = c.take<float>(m);
        L.sq_x[q] = c.take<int32_t>(m);
    }
    for (int q = nq; q < 3; ++q) {
        L.codes_x[q] = L.codes_x[0];
        L.s_x[q] = L.s_x[0];
        L.sq_x[q] = L.sq_x[0];
    }
    L.f = c.take<float>(m * d);
    L.xt = c.take<float>(m * d);
    L.g = c.take<float>(m * d);
    L.h = c.take<float>(m * d);
    L.x1 = c.take<float>(m * d);
    L.z = c.take<float>(m * inner);
    L.codes_b = c.take<int8_t>(m * (d > inner ? d : inner));
    L.s_b = c.take<float>(m);
    L.sq_b = c.take<int32_t>(m);
    L.scan = c.take<char>(scan_workspace_bytes(b, w->d, chunks));
    if (o) *o = L;
    return c.off;
}

mmf_status check_layer(const mmf_layer_weights *w) {
    if (!w) return fail(MMF_ERR_INVALID_ARG, "layer weights are NULL");
    const int d = w->d, inner = w->inner;
    if (d <= 0 || inner <= 0) return fail(MMF_ERR_INVALID_ARG, "d=%d inner=%d must be positive", d, inner);
    if (d % 16 || inner % 16) return fail(MMF_ERR_UNSUPPORTED, "d=%d and inner=%d must be multiples of 16", d, inner);
    if (d > kMaxNormRow) return fail(MMF_ERR_UNSUPPORTED, "d=%d exceeds %d", d, kMaxNormRow);
    if (!(w->eps >= 0.0f)) return fail(MMF_ERR_INVALID_ARG, "eps must be >= 0");
    const struct { const mmf_ternary_weight *p; const char *name; int n, k; } ws[] = {
        {&w->i, "i_proj", d, d}, {&w->f, "f_proj", d, d}, {&w->g, "g_proj", d, d},
        {&w->o, "o_proj", d, d}, {&w->gate, "gate_proj", 2 * inner, d}, {&w->down, "down_proj", d, inner}};
    for (const auto &e : ws) {
        mmf_status st = check_weight(e.p, e.name);
        if (st != MMF_OK) return st;
        if (e.p->n != e.n || e.p->k != e.k)
            return fail(MMF_ERR_INVALID_ARG, "%s: shape [%d][%d], expected [%d][%d]", e.name, e.p->n, e.p->k, e.n, e.k);
    }
    if (w->g_norm_w && !aligned16(w->g_norm_w)) return fail(MMF_ERR_INVALID_ARG, "g_norm_w must be 16-byte aligned");
    return MMF_OK;
}

template <typename T>
T *pick(T *probe_ptr, T *ws_ptr) { return probe_ptr ? probe_ptr : ws_ptr; }

// The block after the mixer's gates: g_norm, o_proj + residual, MLP + residual.
hipError_t block_tail(const mmf_layer_weights *w, const void *x, void *out, mmf_dtype actt, int64_t m,
                      const LayerWs &L, const float *h, const void *g, const mmf_layer_probe *pr,
                      hipStream_t st, std::string *path) {
    const int d = w->d, inner = w->inner;
    const float eps = w->eps;
    hipError_t e;
    int8_t *cu = pick(pr ? pr->codes_u : nullptr, L.codes_b);
    float *su = pick(pr ? pr->scale_u : nullptr, L.s_b);
    e = t_gnorm_quant(h, static_cast<const float *>(g), ACT_F32, m, d, w->g_norm_w, w->o.norm_w, eps, cu, su, L.sq_b,
                      pr ? pr->u : nullptr, st, path);
    if (e != hipSuccess) return e;

    float *x1 = pick(pr ? pr->x1 : nullptr, L.x1);
    ContractArgs co{};
    for (int q = 0; q < 3; ++q) { co.A[q] = cu; co.s[q] = su; co.sumq[q] = L.sq_b; co.B[q] = w->o.packed; co.mu[q] = w->o.mu; }
    co.m = m; co.nc = d; co.k = d;
    co.out0 = x1; co.res = x; co.res_type = act(actt); co.out_type = ACT_F32;
    co.acc_probe = pr ? pr->acc_o : nullptr;
    if ((e = t_contract(co, EPI_RESID, 1, true, st, path)) != hipSuccess) return e;

    int8_t *c1 = pick(pr ? pr->codes_x1 : nullptr, L.codes_b);
    float *s1 = pick(pr ? pr->scale_x1 : nullptr, L.s_b);
    if ((e = t_norm_quant(x1, ACT_F32, m, d, w->gate.norm_w, eps, c1, s1, L.sq_b, st, path)) != hipSuccess) return e;

    void *z = L.z;
    ContractArgs cg{};
    for (int q = 0; q < 3; ++q) { cg.A[q] = c1; cg.s[q] = s1; cg.sumq[q] = L.sq_b; cg.mu[q] = w->gate.mu; }
    cg.B[0] = w->gate.packed;
    cg.B[1] = w->gate.packed + (size_t)inner * (d / 16);
    cg.B[2] = cg.B[1];
    cg.m = m; cg.nc = inner; cg.k = d;
    cg.out0 = z; cg.aux_type = ACT_F32; cg.aux_probe = pr ? pr->z : nullptr;
    cg.acc_probe = pr ? pr->acc_gate : nullptr;
    if ((e = t_contract(cg, EPI_GLU, 2, true, st, path)) != hipSuccess) return e;

    int8_t *cz = pick(pr ? pr->codes_z : nullptr, L.codes_b);
    float *sz = pick(pr ? pr->scale_z : nullptr, L.s_b);
    if ((e = t_norm_quant(z, ACT_F32, m, inner, w->down.norm_w, eps, cz, sz, L.sq_b, st, path)) != hipSuccess) return e;

    ContractArgs cd{};
    for (int q = 0; q < 3; ++q) { cd.A[q] = cz; cd.s[q] = sz; cd.sumq[q] = L.sq_b; cd.B[q] = w->down.packed; cd.mu[q] = w->down.mu; }
    cd.m = m; cd.nc = d; cd.k = inner;
    cd.out0 = out; cd.out_type = act(actt); cd.res = x1; cd.res_type = ACT_F32;
    cd.acc_probe = pr ? pr->acc_down : nullptr;
    return t_contract(cd, EPI_RESID, 1, true, st, path);
}

// The decode step at up to 16 rows (i/f/g sharing one gain or none): a
// contraction quantises its own input rows (launch_contract_row) where that
// costs each workgroup less than a quantiser launch (contract_row_supported:
// one row with or without a gain, several rows without); otherwise the
// separate quantiser runs first, with the stage's gain. At one row o_proj
// also forms the gated g_norm of (h, g) itself (then applies its own gain, if
// any): four kernels instead of eight; at 16 rows of 2048 with an inner width
// of 5632, six (g_norm keeps its quantiser, and down_proj's rows are too
// wide). A probe receives every stage from the same kernels: codes and scales
// of a self-quantising contraction come from its workgroup 0.

// Timing name of a self-quantising contraction: its epilogue and the type of the rows it reads.
std::string row_name(const char *epi, ActType xt) {
    return std::string("tgemv_row<") + epi + (xt == ACT_F32 ? ",f32>" : ",bf16>");
}

hipError_t decode_row_step(const mmf_layer_weights *w, const void *x, void *out, mmf_dtype actt, int64_t b, float *h,
                           const LayerWs &L, const mmf_layer_probe *pr, hipStream_t st, std::string *path) {
    const ActType at = act(actt);
    const int d = w->d, inner = w->inner;
    const float eps = w->eps;
    auto fused = [&](int k, EpiKind epi, const float *gain) { return contract_row_supported(b, k, epi, gain); };
    const float *gx = w->i.norm_w;  // i/f/g share one gain (or none): one quantisation of x serves all three
    hipError_t e;
    // mixer: i/f/g + gates + the state update; g kept in fp32
    int8_t *cx = pick(pr ? pr->codes_x[0] : nullptr, L.codes_b);
    float *sx = pick(pr ? pr->scale_x[0] : nullptr, L.s_b);
    ContractArgs ca{};
    const mmf_ternary_weight *tw[3] = {&w->i, &w->f, &w->g};
    for (int q = 0; q < 3; ++q) { ca.B[q] = tw[q]->packed; ca.mu[q] = tw[q]->mu; }
    ca.m = b; ca.nc = d; ca.k = d;
    ca.out0 = h; ca.out1 = L.g; ca.out_type = ACT_F32; ca.aux_type = ACT_F32;
    if (pr) { ca.acc_probe = pr->acc_ifg; ca.aux_probe = pr->g; ca.out2 = pr->f; ca.out3 = pr->xt; }
    if (fused(d, EPI_GATES_STEP, gx)) {
        e = timed(row_name("gates_step", at), b, 3 * d, d, st, [&] {
            return launch_contract_row(ca, EPI_GATES_STEP, x, at, gx, eps, pr ? pr->codes_x[0] : nullptr,
                                       pr ? pr->scale_x[0] : nullptr, st, path);
        });
    } else {
        e = t_norm_quant(x, at, b, d, gx, eps, cx, sx, L.sq_b, st, path);
        for (int q = 0; q < 3; ++q) { ca.A[q] = cx; ca.s[q] = sx; ca.sumq[q] = L.sq_b; }
        if (e == hipSuccess) e = t_contract(ca, EPI_GATES_STEP, 3, true, st, path);
    }
    if (e == hipSuccess && pr && pr->h)
        e = hipMemcpyAsync(pr->h, h, (size_t)b * d * sizeof(float), hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
    // g_norm + o_proj + residual
    float *x1 = pick(pr ? pr->x1 : nullptr, L.x1);
    ContractArgs co{};
    for (int q = 0; q < 3; ++q) { co.B[q] = w->o.packed; co.mu[q] = w->o.mu; }
    co.m = b; co.nc = d; co.k = d;
    co.out0 = x1; co.out_type = ACT_F32; co.res = x; co.res_type = at;
    co.acc_probe = pr ? pr->acc_o : nullptr;
    if (contract_row_gnorm_supported(b, d)) {
        e = timed(row_name("resid,gnorm", ACT_F32), b, d, d, st, [&] {
            return launch_contract_row_gnorm(co, h, L.g, ACT_F32, w->g_norm_w, w->o.norm_w, eps,
                                             pr ? pr->codes_u : nullptr, pr ? pr->scale_u : nullptr,
                                             pr ? pr->u : nullptr, st, path);
        });
    } else {
        int8_t *cu = pick(pr ? pr->codes_u : nullptr, L.codes_b);
        float *su = pick(pr ? pr->scale_u : nullptr, L.s_b);
        e = t_gnorm_quant(h, L.g, ACT_F32, b, d, w->g_norm_w, w->o.norm_w, eps, cu, su, L.sq_b, pr ? pr->u : nullptr,
                          st, path);
        for (int q = 0; q < 3; ++q) { co.A[q] = cu; co.s[q] = su; co.sumq[q] = L.sq_b; }
        if (e == hipSuccess) e = t_contract(co, EPI_RESID, 1, true, st, path);
    }
    if (e != hipSuccess) return e;
    // gate_proj + SiLU product; z kept in fp32
    ContractArgs cg{};
    for (int q = 0; q < 3; ++q) cg.mu[q] = w->gate.mu;
    cg.B[0] = w->gate.packed;
    cg.B[1] = w->gate.packed + (size_t)inner * (d / 16);
    cg.B[2] = cg.B[1];
    cg.m = b; cg.nc = inner; cg.k = d;
    cg.out0 = L.z; cg.aux_type = ACT_F32;
    if (pr) { cg.acc_probe = pr->acc_gate; cg.aux_probe = pr->z; }
    if (fused(d, EPI_GLU, w->gate.norm_w)) {
        e = timed(row_name("glu", ACT_F32), b, 2 * inner, d, st, [&] {
            return launch_contract_row(cg, EPI_GLU, x1, ACT_F32, w->gate.norm_w, eps, pr ? pr->codes_x1 : nullptr,
                                       pr ? pr->scale_x1 : nullptr, st, path);
        });
    } else {
        int8_t *c1 = pick(pr ? pr->codes_x1 : nullptr, L.codes_b);
        float *s1 = pick(pr ? pr->scale_x1 : nullptr, L.s_b);
        e = t_norm_quant(x1, ACT_F32, b, d, w->gate.norm_w, eps, c1, s1, L.sq_b, st, path);
        for (int q = 0; q < 3; ++q) { cg.A[q] = c1; cg.s[q] = s1; cg.sumq[q] = L.sq_b; }
        if (e == hipSuccess) e = t_contract(cg, EPI_GLU, 2, true, st, path);
    }
    if (e != hipSuccess) return e;
    // down_proj + residual
    ContractArgs cd{};
    for (int q = 0; q < 3; ++q) { cd.B[q] = w->down.packed; cd.mu[q] = w->down.mu; }
    cd.m = b; cd.nc = d; cd.k = inner;
    cd.out0 = out; cd.out_type = at; cd.res = x1; cd.res_type = ACT_F32;
    cd.acc_probe = pr ? pr->acc_down : nullptr;
    if (fused(inner, EPI_RESID, w->down.norm_w))
        return timed(row_name("resid", ACT_F32), b, d, inner, st, [&] {
            return launch_contract_row(cd, EPI_RESID, L.z, ACT_F32, w->down.norm_w, eps, pr ? pr->codes_z : nullptr,
                                       pr ? pr->scale_z : nullptr, st, path);
        });
    int8_t *cz = pick(pr ? pr->codes_z : nullptr, L.codes_b);
    float *sz = pick(pr ? pr->scale_z : nullptr, L.s_b);
    e = t_norm_quant(L.z, ACT_F32, b, inner, w->down.norm_w, eps, cz, sz, L.sq_b, st, path);
    for (int q = 0; q < 3; ++q) { cd.A[q] = cz; cd.s[q] = sz; cd.sumq[q] = L.sq_b; }
    if (e == hipSuccess) e = t_contract(cd, EPI_RESID, 1, true, st, path);
    return e;
}

// Quantise x for i/f/g (once when their gains coincide) and fill the contraction's A side.
hipError_t quant_ifg(const mmf_layer_weights *w, const void *x, mmf_dtype actt, int64_t m, LayerWs &L,
                     const mmf_layer_probe *pr, ContractArgs &ca, bool *shared, hipStream_t st, std::string *path) {
    *shared = shared_ifg(w);
    const int nq = *shared ? 1 : 3;
    const float *gains[3] = {w->i.norm_w, w->f.norm_w, w->g.norm_w};
    int8_t *codes[3];
    float *scales[3];
    for (int q = 0; q < nq; ++q) {
        codes[q] = pick(pr ? pr->codes_x[q] : nullptr, L.codes_x[q]);
        scales[q] = pick(pr ? pr->scale_x[q] : nullptr, L.s_x[q]);
        hipError_t e = t_norm_quant(x, act(actt), m, w->d, gains[q], w->eps, codes[q], scales[q], L.sq_x[q], st, path);
        if (e != hipSuccess) return e;
    }
    const mmf_ternary_weight *tw[3] = {&w->i, &w->f, &w->g};
    for (int q = 0; q < 3; ++q) {
        const int src = *shared ? 0 : q;
        ca.A[q] = codes[src];
        ca.s[q] = scales[src];
        ca.sumq[q] = L.sq_x[src];
        ca.B[q] = tw[q]->packed;
        ca.mu[q] = tw[q]->mu;
    }
    ca.m = m; ca.nc = w->d; ca.k = w->d;
    ca.acc_probe = pr ? pr->acc_ifg : nullptr;
    return hipSuccess;
}

// The decode step on a validated workspace of at least mmf_layer_workspace_size(w, b, 1) bytes.
mmf_status decode_step_run(const mmf_layer_weights *w, const void *x, void *out, mmf_dtype actt, int64_t b, float *h,
                           void *ws, const mmf_layer_probe *probe, hipStream_t stream) {
    const int mode = g_decode_mode.load();
    std::string path;
    hipError_t e = hipSuccess;
    const bool row_ok = b >= 1 && b <= 16 && shared_ifg(w);
    if (row_ok && mode == 0) {
        Carver c(ws);
        LayerWs L;
        layer_plan(c, w, b, 1, scan_pick_chunks(b, 1, w->d, MMF_SCAN_CHUNK), &L);
        e = decode_row_step(w, x, out, actt, b, h, L, probe, stream, &path);
        mmf_status r = hip_status(e, "mmf_layer_decode_step");
        if (r == MMF_OK) g_path = path;
        return r;
    }
    if (b > 0) {
        Carver c(ws);
        LayerWs L;
        layer_plan(c, w, b, 1, scan_pick_chunks(b, 1, w->d, MMF_SCAN_CHUNK), &L);
        ContractArgs ca{};
        bool shared = true;
        e = quant_ifg(w, x, actt, b, L, probe, ca, &shared, stream, &path);
        void *g = L.g;
        if (e == hipSuccess) {
            ca.out0 = h; ca.out1 = g; ca.out_type = ACT_F32;
            ca.aux_type = ACT_F32; ca.aux_probe = probe ? probe->g : nullptr;
            ca.out2 = probe ? probe->f : nullptr;
            ca.out3 = probe ? probe->xt : nullptr;
            e = t_contract(ca, EPI_GATES_STEP, 3, shared, stream, &path);
        }
        if (e == hipSuccess && probe && probe->h)
            e = hipMemcpyAsync(probe->h, h, (size_t)b * w->d * sizeof(float), hipMemcpyDeviceToDevice, stream);
        if (e == hipSuccess) e = block_tail(w, x, out, actt, b, L, h, g, probe, stream, &path);
    }
    mmf_status r = hip_status(e, "mmf_layer_decode_step");
    if (r == MMF_OK) g_path = path;
    return r;
}

// ------------------------------------------------- decode without allocation --
// The workspace of mmf_layer_decode_step_noalloc: one array per device, held
// until the process ends. Host code never uses the array's name as an address
// (on the host it is only a stand-in for the symbol): the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoallocScratchBytes = size_t(8) << 20;

}  // namespace

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// This device's copy of the scratch array, looked up on the first call on the device.
mmf_status scratch_for_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MMF_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MMF_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MMF_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MMF_OK;
}

}  // namespace

extern "C" {

const char *mmf_last_error(void) { return g_err.c_str(); }
const char *mmf_last_path(void) { return g_path.c_str(); }

mmf_status mmf_ternary_pack_workspace_size(int32_t n, int32_t k, size_t *bytes) {
    if (!bytes) return fail(MMF_ERR_INVALID_ARG, "bytes is NULL");
    if (n <= 0 || k <= 0) return fail(MMF_ERR_INVALID_ARG, "n=%d k=%d must be positive", n, k);
    if (k % 16) return fail(MMF_ERR_UNSUPPORTED, "k=%d is not a multiple of 16", k);
    *bytes = pack_workspace_bytes();
    return MMF_OK;
}

mmf_status mmf_ternary_pack(const float *w, int32_t n, int32_t k, uint32_t *packed, float *mu, void *ws,
                            size_t ws_bytes, hipStream_t stream) {
    size_t need = 0;
    mmf_status st = mmf_ternary_pack_workspace_size(n, k, &need);
    if (st != MMF_OK) return st;
    if (!w || !packed || !mu) return fail(MMF_ERR_INVALID_ARG, "w, packed and mu must be non-NULL");
    if (!aligned16(w) || !aligned16(packed)) return fail(MMF_ERR_INVALID_ARG, "w and packed must be 16-byte aligned");
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(MMF_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
    std::string path;
    mmf_status r = hip_status(launch_pack(w, n, k, packed, mu, ws, stream, &path), "mmf_ternary_pack");
    if (r == MMF_OK) g_path = path;
    return r;
}

mmf_status mmf_bitlinear_workspace_size(int64_t m, int32_t k, size_t *bytes) {
    if (!bytes) return fail(MMF_ERR_INVALID_ARG, "bytes is NULL");
    if (m < 0 || k <= 0) return fail(MMF_ERR_INVALID_ARG, "m=%lld k=%d invalid", (long long)m, k);
    Carver c(nullptr);
    *bytes = bitlinear_plan(c, m, k, nullptr);
    return MMF_OK;
}

mmf_status mmf_bitlinear_fwd(const void *x, mmf_dtype xt, int64_t m, const mmf_ternary_weight *w, float eps,
                             void *y, mmf_dtype yt, int8_t *codes_out, float *scale_out, int32_t *acc_out,
                             void *ws, size_t ws_bytes, hipStream_t stream) {
    mmf_status st = check_weight(w, "weight");
    if (st != MMF_OK) return st;
    if (!valid_dtype(xt) || !valid_dtype(yt)) return fail(MMF_ERR_INVALID_ARG, "bad dtype");
    if (m < 0) return fail(MMF_ERR_INVALID_ARG, "m=%lld < 0", (long long)m);
    if (!(eps >= 0.0f)) return fail(MMF_ERR_INVALID_ARG, "eps must be >= 0");
    if (m > 0 && (!x || !y)) return fail(MMF_ERR_INVALID_ARG, "x and y must be non-NULL");
    if (!aligned16(x) || !aligned16(codes_out)) return fail(MMF_ERR_INVALID_ARG, "x and codes_out must be 16-byte aligned");
    size_t need = 0;
    mmf_bitlinear_workspace_size(m, w->k, &need);
    if (m > 0 && (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)))
        return fail(MMF_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
    std::string path;
    if (m == 0) {
        g_path = "empty";
        g_err.clear();
        return MMF_OK;
    }
    Carver c(ws);
    BitlinearWs B;
    bitlinear_plan(c, m, w->k, &B);
    int8_t *codes = codes_out ? codes_out : B.codes;
    float *s = scale_out ? scale_out : B.s;
    hipError_t e = t_norm_quant(x, act(xt), m, w->k, w->norm_w, eps, codes, s, B.sumq, stream, &path);
    if (e == hipSuccess) {
        ContractArgs a{};
        for (int q = 0; q < 3; ++q) { a.A[q] = codes; a.s[q] = s; a.sumq[q] = B.sumq; a.B[q] = w->packed; a.mu[q] = w->mu; }
        a.m = m; a.nc = w->n; a.k = w->k;
        a.out0 = y; a.out_type = act(yt);
        a.acc_probe = acc_out;
        e = t_contract(a, EPI_LINEAR, 1, true, stream, &path);
    }
    mmf_status r = hip_status(e, "mmf_bitlinear_fwd");
    if (r == MMF_OK) g_path = path;
    return r;
}

// ------------------------------------------------------------ bitlinear bwd --
struct BitlinearBwdWs {
    int8_t *q;
    float *s;
    uint16_t *tT, *dy16, *dyT, *qT;
    float *du, *gpart, *gpart2, *split;
};

// rows of the dW product's operands (its contraction), zero-padded to whole K steps of the
// products (64), so that the product runs on its LDS-DMA kernel at any row count
int64_t pad_k(int64_t m) { return (m + 63) / 64 * 64; }

// floats of the dW product's per-split partial blocks for an n x k weight over m rows (0: no split)
size_t dw_split_floats(int64_t m, int n, int k) {
    const int sp = m > 0 ? gemm_bf16_splits(n, k, (int)pad_k(m)) : 1;
    return sp > 1 ? (size_t)sp * n * k : 0;
}

size_t bitlinear_bwd_plan(Carver &c, int64_t m, int n, int k, mmf_dtype dyt, BitlinearBwdWs *o,
                          size_t split_floats = SIZE_MAX) {
    BitlinearBwdWs w;
    w.q = c.take<int8_t>((size_t)m * k);
    w.s = c.take<float>((size_t)m);
    w.tT = c.take<uint16_t>((size_t)n * k);
    w.dy16 = dyt == MMF_F32 ? c.take<uint16_t>((size_t)m * n) : nullptr;
    w.dyT = c.take<uint16_t>((size_t)n * pad_k(m));
    w.qT = c.take<uint16_t>((size_t)k * pad_k(m));
    w.du = c.take<float>((size_t)m * k);
    const int64_t nblk = m > 0 ? (m + rmsnorm_bwd_rows(m) - 1) / rmsnorm_bwd_rows(m) : 0;
    w.gpart = c.take<float>((size_t)nblk * k);
    w.gpart2 = c.take<float>((size_t)gain_reduce_splits((int)nblk) * k);
    // partial blocks of the dW product when it is split along the rows
    if (split_floats == SIZE_MAX) split_floats = dw_split_floats(m, n, k);
    w.split = split_floats ? c.take<float>(split_floats) : nullptr;
    if (o) *o = w;
    return c.off;
}

// One FusedBitLinear derivative (m > 0) on a carved workspace sized for at
// least (m, n, k) with an fp32 dy: codes from the forward's quantiser, the two
// bf16 products (du before 1 / sw: dy t over n; dW: (dy / s)^T q over the rows),
// the RMSNorm derivative and the gain's sums.
hipError_t bitlinear_bwd_run(const void *x, ActType xt, int64_t m, const mmf_ternary_weight *w, float eps,
                             const void *dy, ActType dyt, void *dx, ActType dxt, float *dw, float *dgain,
                             const BitlinearBwdWs &B, hipStream_t stream, std::string *path) {
    const int n = w->n, k = w->k;
    hipError_t e = t_norm_quant(x, xt, m, k, w->norm_w, eps, B.q, B.s, nullptr, stream, path);
    if (e == hipSuccess && (dx || dgain)) {
        const uint16_t *dy16 = static_cast<const uint16_t *>(dy);
        if (dyt == ACT_F32) {
            e = timed("to_bf16", m, n, n, stream,
                      [&] { return launch_to_bf16(static_cast<const float *>(dy), m * n, B.dy16, stream); });
            dy16 = B.dy16;
        }
        if (e == hipSuccess)
            e = timed("expand_ternary_t", n, k, k, stream,
                      [&] { return launch_expand_ternary_t(w->packed, n, k, B.tT, n, stream); });
        if (e == hipSuccess)  // du (before 1 / sw) [m][k] = dy [m][n] t^T [k][n]^T
            e = timed("gemm_bf16<du>", m, k, n, stream,
                      [&] { return launch_gemm_bf16_nt(dy16, n, B.tT, n, (int)m, k, n, B.du, k, nullptr, stream); });
        if (e == hipSuccess)
            e = timed("rmsnorm_bwd", m, k, k, stream, [&] {
                return launch_rmsnorm_bwd(x, xt, B.du, w->norm_w, w->mu, eps, m, k, dx, dxt, dgain ? B.gpart : nullptr,
                                          stream);
            });
        if (e == hipSuccess && dgain) {
            const int rows = rmsnorm_bwd_rows(m);
            const int nblk = (int)((m + rows - 1) / rows);
            e = timed("gain_reduce", nblk, k, k, stream,
                      [&] { return launch_gain_reduce(B.gpart, nblk, k, B.gpart2, dgain, stream); });
        }
        *path += std::string(dyt == ACT_F32 ? "to_bf16;" : "") + "expand_ternary_t;gemm_bf16<du>;rmsnorm_bwd;" +
                 (dgain ? "gain_reduce;" : "");
    }
    if (e == hipSuccess && dw) {
        const int64_t mp = pad_k(m);
        e = timed("transpose_bf16<dy/s>", m, n, n, stream, [&] {
            return launch_transpose_bf16(dy, dyt == ACT_F32 ? 0 : 1, B.s, m, n, B.dyT, mp, stream);
        });
        if (e == hipSuccess)
            e = timed("transpose_bf16<q>", m, k, k, stream,
                      [&] { return launch_transpose_bf16(B.q, 2, nullptr, m, k, B.qT, mp, stream); });
        if (e == hipSuccess)  // dW [n][k] = (dy / s)^T [n][m] (q^T [k][m])^T
            e = timed("gemm_bf16<dw>", n, k, (int)mp, stream,
                      [&] { return launch_gemm_bf16_nt(B.dyT, mp, B.qT, mp, n, k, (int)mp, dw, k, B.split, stream); });
        *path += "transpose_bf16<dy/s>;transpose_bf16<q>;gemm_bf16<dw>;";
    }
    return e;
}

mmf_status mmf_bitlinear_bwd_workspace_size(int64_t m, const mmf_ternary_weight *w, mmf_dtype dyt, size_t *bytes) {
    if (!bytes) return fail(MMF_ERR_INVALID_ARG, "bytes is NULL");
    mmf_status st = check_weight(w, "weight");
    if (st != MMF_OK) return st;
    if (m < 0) return fail(MMF_ERR_INVALID_ARG, "m=%lld < 0", (long long)m);
    if (!valid_dtype(dyt)) return fail(MMF_ERR_INVALID_ARG, "bad dtype");
    Carver c(nullptr);
    *bytes = bitlinear_bwd_plan(c, m, w->n, w->k, dyt, nullptr);
    return MMF_OK;
}

mmf_status mmf_bitlinear_bwd(const void *x, mmf_dtype xt, int64_t m, const mmf_ternary_weight *w, float eps,
                             const void *dy, mmf_dtype dyt, void *dx, mmf_dtype dxt, float *dw, float *dgain,
                             void *ws, size_t ws_bytes, hipStream_t stream) {
    size_t need = 0;
    mmf_status st = mmf_bitlinear_bwd_workspace_size(m, w, dyt, &need);
    if (st != MMF_OK) return st;
    if (!valid_dtype(xt) || !valid_dtype(dxt)) return fail(MMF_ERR_INVALID_ARG, "bad dtype");
    if (!(eps >= 0.0f)) return fail(MMF_ERR_INVALID_ARG, "eps must be >= 0");
    const int n = w->n, k = w->k;
    if (n % 8) return fail(MMF_ERR_UNSUPPORTED, "n=%d is not a multiple of 8", n);
    if (!rmsnorm_bwd_supported(k)) return fail(MMF_ERR_UNSUPPORTED, "k=%d exceeds %d", k, kMaxNormRow);
    if ((int64_t)n > INT32_MAX || m > INT32_MAX) return fail(MMF_ERR_UNSUPPORTED, "m or n beyond 32-bit GEMM sizes");
    if (m > 0 && (!x || !dy)) return fail(MMF_ERR_INVALID_ARG, "x and dy must be non-NULL");
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(dw) || !aligned16(dgain))
        return fail(MMF_ERR_INVALID_ARG, "x, dy, dx, dw and dgain must be 16-byte aligned");
    if (m > 0 && (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)))
        return fail(MMF_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
    if (m == 0) {
        // no rows: dW and dgain are sums over nothing
        hipError_t e = hipSuccess;
        if (dw) e = launch_zero_f32(dw, (int64_t)n * k, stream);
        if (e == hipSuccess && dgain) e = launch_zero_f32(dgain, k, stream);
        mmf_status r = hip_status(e, "mmf_bitlinear_bwd");
        if (r == MMF_OK) g_path = "empty";
        return r;
    }
    Carver c(ws);
    BitlinearBwdWs B;
    bitlinear_bwd_plan(c, m, n, k, dyt, &B);
    std::string path;
    hipError_t e = bitlinear_bwd_run(x, act(xt), m, w, eps, dy, act(dyt), dx, act(dxt), dw, dgain, B, stream, &path);
    mmf_status r = hip_status(e, "mmf_bitlinear_bwd");
    if (r == MMF_OK) g_path = path;
    return r;
}

// --------------------------------------------------------------- generation --
mmf_status mmf_embed(const int32_t *ids, int64_t count, const void *table, mmf_dtype tt, int64_t vocab, int32_t d,
                     void *out, hipStream_t stream) {
    if (!valid_dtype(tt)) return fail(MMF_ERR_INVALID_ARG, "bad dtype");
    if (count < 0 || vocab <= 0 || d <= 0) return fail(MMF_ERR_INVALID_ARG, "count >= 0, vocab > 0 and d > 0 required");
    const int64_t row_bytes = (int64_t)d * (tt == MMF_F32 ? 4 : 2);
    if (row_bytes % 16) return fail(MMF_ERR_UNSUPPORTED, "a row of %d elements is not a whole number of 16 bytes", d);
    if (count > 0 && (!ids || !table || !out)) return fail(MMF_ERR_INVALID_ARG, "ids, table and out must be non-NULL");
    if (!aligned16(table) || !aligned16(out)) return fail(MMF_ERR_INVALID_ARG, "table and out must be 16-byte aligned");
    if (count > INT32_MAX) return fail(MMF_ERR_UNSUPPORTED, "count beyond 2^31 rows");
    std::string path = "embed;";
    hipError_t e = timed("embed", count, d, d, stream,
                         [&] { return launch_embed(ids, count, table, vocab, row_bytes, out, stream); });
    mmf_status r = hip_status(e, "mmf_embed");
    if (r == MMF_OK) g_path = path;
    return r;
}

struct GreedyWs {
    int8_t *codes;
    float *s;
    int32_t *sumq, *acc;
    float *logits;
};

size_t greedy_plan(Carver &c, int64_t b, int n, int k, GreedyWs *o) {
    GreedyWs w;
    w.codes = c.take<int8_t>((size_t)b * k);
    w.s = c.take<float>((size_t)b);
    w.sumq = c.take<int32_t>((size_t)b);
    w.acc = c.take<int32_t>((size_t)b * n);
    w.logits = c.take<float>((size_t)b * n);
    if (o) *o = w;
    return c.off;
}

mmf_status mmf_greedy_head_workspace_size(int64_t b, const mmf_ternary_weight *head, size_t *bytes) {
    if (!bytes) return fail(MMF_ERR_INVALID_ARG, "bytes is NULL");
    mmf_status st = check_weight(head, "head");
    if (st != MMF_OK) return st;
    if (b < 0) return fail(MMF_ERR_INVALID_ARG, "b=%lld < 0", (long long)b);
    Carver c(nullptr);
    *bytes = greedy_plan(c, b, head->n, head->k, nullptr);
    return MMF_OK;
}

mmf_status mmf_greedy_head(const void *x, mmf_dtype xt, int64_t b, const mmf_ternary_weight *head, float eps,
                           int32_t *tokens, float *logits, void *ws, size_t ws_bytes, hipStream_t stream) {
    size_t need = 0;
    mmf_status st = mmf_greedy_head_workspace_size(b, head, &need);
    if (st != MMF_OK) return st;
    if (!valid_dtype(xt)) return fail(MMF_ERR_INVALID_ARG, "bad dtype");
    if (!(eps >= 0.0f)) return fail(MMF_ERR_INVALID_ARG, "eps must be >= 0");
    if (head->n % 4) return fail(MMF_ERR_UNSUPPORTED, "vocabulary %d is not a multiple of 4", head->n);
    if (b > 0 && (!x || !tokens)) return fail(MMF_ERR_INVALID_ARG, "x and tokens must be non-NULL");
    if (!aligned16(x) || !aligned16(logits)) return fail(MMF_ERR_INVALID_ARG, "x and logits must be 16-byte aligned");
    if (b > 0 && (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)))
        return fail(MMF_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
    if (b == 0) {
        g_path = "empty";
        g_err.clear();
        return MMF_OK;
    }
    Carver c(ws);
    GreedyWs G;
    greedy_plan(c, b, head->n, head->k, &G);
    std::string path;
    // the head: FusedBitLinear with its exact int32 sums kept
    hipError_t e = t_norm_quant(x, act(xt), b, head->k, head->norm_w, eps, G.codes, G.s, G.sumq, stream, &path);
    if (e == hipSuccess) {
        ContractArgs a{};
        for (int q = 0; q < 3; ++q) { a.A[q] = G.codes; a.s[q] = G.s; a.sumq[q] = G.sumq; a.B[q] = head->packed; a.mu[q] = head->mu; }
        a.m = b; a.nc = head->n; a.k = head->k;
        a.out0 = logits ? logits : G.logits; a.out_type = ACT_F32;
        a.acc_probe = G.acc;
        e = t_contract(a, EPI_LINEAR, 1, true, stream, &path);
    }
    if (e == hipSuccess)
        e = timed("argmax_rows", b, head->n, head->n, stream,
                  [&] { return launch_argmax_rows(G.acc, b, head->n, tokens, stream); });
    path += "argmax_rows;";
    mmf_status r = hip_status(e, "mmf_greedy_head");
    if (r == MMF_OK) g_path = path;
    return r;
}

mmf_status mmf_hgrn_scan_workspace_size(int64_t b, int64_t t, int64_t d, mmf_scan_mode mode, size_t *bytes) {
    if (!bytes) return fail(MMF_ERR_INVALID_ARG, "bytes is NULL");
    if (b < 0 || t < 0 || d <= 0) return fail(MMF_ERR_INVALID_ARG, "b, t >= 0 and d > 0 required");
    if (mode != MMF_SCAN_AUTO && mode != MMF_SCAN_RECURRENT && mode != MMF_SCAN_CHUNK)
        return fail(MMF_ERR_INVALID_ARG, "bad scan mode %d", (int)mode);
    *bytes = scan_workspace_bytes(b, d, scan_pick_chunks(b, t, d, (int)mode));
    return MMF_OK;
}

mmf_status mmf_hgrn_scan_fwd(const float *x, const float *f, const float *h0, float *h, float *h_last, int64_t b,
                             int64_t t, int64_t d, mmf_scan_mode mode, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
    size_t need = 0;
    mmf_status st = mmf_hgrn_scan_workspace_size(b, t, d, mode, &need);
    if (st != MMF_OK) return st;
    if (b > 0 && t > 0 && (!x || !f || !h)) return fail(MMF_ERR_INVALID_ARG, "x, f and h must be non-NULL");
    if (need && (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)))
        return fail(MMF_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
    std::string path;
    const int chunks = scan_pick_chunks(b, t, d, (int)mode);
    mmf_status r = hip_status(t_scan(x, f, h0, h, h_last, b, t, d, chunks, ws, stream, &path), "mmf_hgrn_scan_fwd");
    if (r == MMF_OK) g_path = path;
    return r;
}

// tokens from which AUTO takes the chunked form: one whole chunk (measured on MI355X at
// B = 16, d = 2048: faster than the step-wise form at every length from 16 tokens on, heads of
// 64 and 128, e.g. 12.5 against 14.2 us at 16 tokens and 151 against 214 us at 512, heads of 128)
constexpr int64_t kHgrn2ChunkFrom = 16;

mmf_status mmf_hgrn2_scan_fwd(const float *f, const float *i, const float *o, const float *s0, float *y,
                              float *s_last, int64_t b, int64_t t, int64_t d, int64_t e, mmf_scan_mode mode,
                              hipStream_t stream) {
    if (b < 0 || t < 0 || d <= 0) return fail(MMF_ERR_INVALID_ARG, "b, t >= 0 and d > 0 required");
    if (mode != MMF_SCAN_AUTO && mode != MMF_SCAN_RECURRENT && mode != MMF_SCAN_CHUNK)
        return fail(MMF_ERR_INVALID_ARG, "bad scan mode %d", (int)mode);
    if (e != 16 && e != 32 && e != 64 && e != 128)
        return fail(MMF_ERR_UNSUPPORTED, "head width e = %lld: 16, 32, 64 or 128 supported", (long long)e);
    if (mode == MMF_SCAN_CHUNK && e < 64)
        return fail(MMF_ERR_UNSUPPORTED, "the chunked form takes heads of 64 or 128, not %lld", (long long)e);
    // the chunked kernel addresses a sequence's rows (and up to two chunks past its end) with
    // 32-bit byte offsets
    const bool chunk_fits = (t + 32) <= (int64_t)INT32_MAX / 4 / d;
    if (mode == MMF_SCAN_CHUNK && !chunk_fits)
        return fail(MMF_ERR_UNSUPPORTED, "the chunked form takes sequences of under 2 GiB of rows: t = %lld, d = %lld",
                    (long long)t, (long long)d);
    if (d % e) return fail(MMF_ERR_INVALID_ARG, "d = %lld is not a multiple of e = %lld", (long long)d, (long long)e);
    if (b > 0 && t > 0 && (!f || !i || !o || !y)) return fail(MMF_ERR_INVALID_ARG, "f, i, o and y must be non-NULL");
    const void *ins[] = {f, i, o, s0};
    for (const void *p : ins)
        if (p && (p == y || p == s_last) && !(p == s0 && p == s_last))
            return fail(MMF_ERR_INVALID_ARG, "y and s_last may not alias an input (s_last may equal s0)");
    if (y && y == s_last) return fail(MMF_ERR_INVALID_ARG, "y and s_last may not alias");
    const void *all[] = {f, i, o, s0, y, s_last};
    for (const void *p : all)
        if (reinterpret_cast<uintptr_t>(p) & 15u) return fail(MMF_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (hgrn2_workgroups(b, d, (int)e) > INT32_MAX) return fail(MMF_ERR_UNSUPPORTED, "b * d too large");
    if (b == 0) return MMF_OK;
    const char *name = "hgrn2_scan";
    // the chunked kernel from 16 tokens on (heads of 64 or 128, sequences under 2 GiB of rows),
    // else the step-wise one
    const bool chunk =
        mode == MMF_SCAN_CHUNK || (mode == MMF_SCAN_AUTO && e >= 64 && t >= kHgrn2ChunkFrom && chunk_fits);
    // timing label: a one-token call (a decode step) streams the state, a longer one computes
    const std::string label = std::string(chunk ? "hgrn2_chunk<" : t == 1 ? "hgrn2_step<" : "hgrn2_scan<") +
                              std::to_string(e) + ">";
    hipError_t err = timed(label, b * t, (int)d, (int)e, stream, [&] {
        return launch_hgrn2_scan(f, i, o, s0, y, s_last, b, t, d, (int)e, chunk, stream, &name);
    });
    mmf_status r = hip_status(err, "mmf_hgrn2_scan_fwd");
    if (r == MMF_OK) g_path = name;
    return r;
}

mmf_status mmf_hgrn_scan_bwd(const float *f, const float *h, const float *h0, const float *dh, const float *dh_last,
                             float *dx, float *df, float *dh0, int64_t b, int64_t t, int64_t d, mmf_scan_mode mode,
                             hipStream_t stream) {
    if (b < 0 || t < 0 || d <= 0) return fail(MMF_ERR_INVALID_ARG, "b, t >= 0 and d > 0 required");
    if (mode != MMF_SCAN_AUTO && mode != MMF_SCAN_RECURRENT && mode != MMF_SCAN_CHUNK)
        return fail(MMF_ERR_INVALID_ARG, "bad scan mode %d", (int)mode);
    if (b > 0 && t > 0 && (!f || !h || !dh || !dx || !df))
        return fail(MMF_ERR_INVALID_ARG, "f, h, dh, dx and df must be non-NULL");
    const void *ins[] = {f, h, h0, dh, dh_last};
    const void *outs[] = {df, dh0};
    for (const void *o : outs)
        for (const void *i : ins)
            if (o && o == i) return fail(MMF_ERR_INVALID_ARG, "df and dh0 may not alias an input");
    if (dx && (dx == f || dx == h || dx == h0 || dx == dh_last || dx == df || dx == dh0))
        return fail(MMF_ERR_INVALID_ARG, "dx may alias dh only");
    std::string path;
    const int plan = scan_bwd_pick(t, (int)mode);
    hipError_t e = timed(plan == kScanTiled ? "scan_bwd_tiled" : "scan_bwd_recurrent", b * t, (int)d, (int)d, stream,
                         [&] { return launch_scan_bwd(f, h, h0, dh, dh_last, dx, df, dh0, b, t, d, plan, stream, &path); });
    mmf_status r = hip_status(e, "mmf_hgrn_scan_bwd");
    if (r == MMF_OK) g_path = path;
    return r;
}

mmf_status mmf_layer_workspace_size(const mmf_layer_weights *w, int64_t b, int64_t t, size_t *bytes) {
    if (!bytes) return fail(MMF_ERR_INVALID_ARG, "bytes is NULL");
    mmf_status st = check_layer(w);
    if (st != MMF_OK) return st;
    if (b < 0 || t < 0) return fail(MMF_ERR_INVALID_ARG, "b, t must be >= 0");
    const int chunks = scan_pick_chunks(b, t, w->d, MMF_SCAN_CHUNK);
    Carver c(nullptr);
    *bytes = layer_plan(c, w, b, t > 0 ? t : 1, chunks, nullptr);
    return MMF_OK;
}

mmf_status mmf_layer_fwd(const mmf_layer_weights *w, const void *x, void *out, mmf_dtype actt, int64_t b, int64_t t,
                         const float *h0, float *h_last, mmf_scan_mode mode, void *ws, size_t ws_bytes,
                         const mmf_layer_probe *probe, hipStream_t stream) {
    size_t need = 0;
    mmf_status st = mmf_layer_workspace_size(w, b, t, &need);
    if (st != MMF_OK) return st;
    if (!valid_dtype(actt)) return fail(MMF_ERR_INVALID_ARG, "bad activation dtype");
    if (mode != MMF_SCAN_AUTO && mode != MMF_SCAN_RECURRENT && mode != MMF_SCAN_CHUNK)
        return fail(MMF_ERR_INVALID_ARG, "bad scan mode %d", (int)mode);
    const int64_t m = b * t;
    if (m > 0 && (!x || !out)) return fail(MMF_ERR_INVALID_ARG, "x and out must be non-NULL");
    if (!aligned16(x) || !aligned16(out) || !aligned16(h0) || !aligned16(h_last))
        return fail(MMF_ERR_INVALID_ARG, "x, out, h0, h_last must be 16-byte aligned");
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(MMF_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
    std::string path;
    hipError_t e = hipSuccess;
    if (m == 0) {
        e = t_scan(nullptr, nullptr, h0, nullptr, h_last, b, 0, w->d, 1, nullptr, stream, &path);
    } else {
        const int chunks = scan_pick_chunks(b, t, w->d, (int)mode);
        Carver c(ws);
        LayerWs L;
        layer_plan(c, w, b, t, scan_pick_chunks(b, t, w->d, MMF_SCAN_CHUNK), &L);
        ContractArgs ca{};
        bool shared = true;
        e = quant_ifg(w, x, actt, m, L, probe, ca, &shared, stream, &path);
        float *f = pick(probe ? probe->f : nullptr, L.f);
        float *xt = pick(probe ? probe->xt : nullptr, L.xt);
        void *g = L.g;
        float *h = pick(probe ? probe->h : nullptr, L.h);
        if (e == hipSuccess) {
            ca.out0 = f; ca.out1 = xt; ca.out2 = g; ca.out_type = ACT_F32;
            ca.aux_type = ACT_F32; ca.aux_probe = probe ? probe->g : nullptr;
            e = t_contract(ca, EPI_GATES, 3, shared, stream, &path);
        }
        if (e == hipSuccess) e = t_scan(xt, f, h0, h, h_last, b, t, w->d, chunks, L.scan, stream, &path);
        if (e == hipSuccess) e = block_tail(w, x, out, actt, m, L, h, g, probe, stream, &path);
    }
    mmf_status r = hip_status(e, "mmf_layer_fwd");
    if (r == MMF_OK) g_path = path;
    return r;
}

mmf_status mmf_set_decode_kernel(int mode) {
    if (mode < 0 || mode > 1) return fail(MMF_ERR_INVALID_ARG, "decode kernel mode %d (0 auto, 1 separate)", mode);
    g_decode_mode.store(mode);
    g_err.clear();
    return MMF_OK;
}

mmf_status mmf_layer_decode_step(const mmf_layer_weights *w, const void *x, void *out, mmf_dtype actt, int64_t b,
                                 float *h, void *ws, size_t ws_bytes, const mmf_layer_probe *probe,
                                 hipStream_t stream) {
    size_t need = 0;
    mmf_status st = mmf_layer_workspace_size(w, b, 1, &need);
    if (st != MMF_OK) return st;
    if (!valid_dtype(actt)) return fail(MMF_ERR_INVALID_ARG, "bad activation dtype");
    if (b > 0 && (!x || !out || !h)) return fail(MMF_ERR_INVALID_ARG, "x, out and h must be non-NULL");
    if (!aligned16(x) || !aligned16(out) || !aligned16(h))
        return fail(MMF_ERR_INVALID_ARG, "x, out and h must be 16-byte aligned");
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(MMF_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
    return decode_step_run(w, x, out, actt, b, h, ws, probe, stream);
}

mmf_status mmf_layer_decode_step_noalloc(const mmf_layer_weights *w, const void *x, void *out, mmf_dtype actt,
                                         int64_t b, float *h, const mmf_layer_probe *probe, hipStream_t stream) {
    size_t need = 0;
    mmf_status st = mmf_layer_workspace_size(w, b, 1, &need);
    if (st != MMF_OK) return st;
    if (!valid_dtype(actt)) return fail(MMF_ERR_INVALID_ARG, "bad activation dtype");
    if (b > 0 && (!x || !out || !h)) return fail(MMF_ERR_INVALID_ARG, "x, out and h must be non-NULL");
    if (!aligned16(x) || !aligned16(out) || !aligned16(h))
        return fail(MMF_ERR_INVALID_ARG, "x, out and h must be 16-byte aligned");
    if (need > kNoallocScratchBytes)
        return fail(MMF_ERR_WORKSPACE, "decode step needs %zu bytes of scratch, beyond the %zu the library holds "
                    "(use mmf_layer_decode_step with a workspace)", need, kNoallocScratchBytes);
    void *ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != MMF_OK) return st;
    return decode_step_run(w, x, out, actt, b, h, ws, probe, stream);
}

// ------------------------------------------------------ whole-stack decode --
struct StackWs {
    StackLayer *table;
    unsigned *bar;
    void *act[2];
    float *g, *x1, *z;
    int8_t *codes;
    float *s;
    int32_t *sumq;
};

static size_t stack_plan(Carver &c, int32_t n, int64_t b, int d, int inner, StackWs *o) {
    StackWs w;
    w.table = c.take<StackLayer>((size_t)n);
    w.bar = c.take<unsigned>(kStackBarWords);
    w.act[0] = c.take<float>((size_t)b * d);  // fp32-sized: holds either activation dtype
    w.act[1] = c.take<float>((size_t)b * d);
    w.g = c.take<float>((size_t)b * d);
    w.x1 = c.take<float>((size_t)b * d);
    w.z = c.take<float>((size_t)b * inner);
    w.codes = c.take<int8_t>((size_t)16 * (d > inner ? d : inner));
    w.s = c.take<float>(16);
    w.sumq = c.take<int32_t>(16);
    if (o) *o = w;
    return c.off;
}

static mmf_status check_stack(const mmf_layer_weights *layers, int32_t n, int64_t b) {
    if (!layers) return fail(MMF_ERR_INVALID_ARG, "layers is NULL");
    if (n <= 0) return fail(MMF_ERR_INVALID_ARG, "n_layers=%d must be positive", (int)n);
    for (int32_t l = 0; l < n; ++l) {
        mmf_status st = check_layer(&layers[l]);
        if (st != MMF_OK) return st;
        if (layers[l].d != layers[0].d || layers[l].inner != layers[0].inner)
            return fail(MMF_ERR_INVALID_ARG, "layer %d: d/inner differ from layer 0", (int)l);
        if (!shared_ifg(&layers[l]))
            return fail(MMF_ERR_UNSUPPORTED, "layer %d: i/f/g gains must be one tensor (or none)", (int)l);
    }
    if (const char *why = stack_decode_unsupported(b, layers[0].d, layers[0].inner))
        return fail(MMF_ERR_UNSUPPORTED, "stack decode: %s", why);
    return MMF_OK;
}

mmf_status mmf_stack_decode_workspace_size(const mmf_layer_weights *layers, int32_t n_layers, int64_t b,
                                           size_t *bytes) {
    if (!bytes) return fail(MMF_ERR_INVALID_ARG, "bytes is NULL");
    mmf_status st = check_stack(layers, n_layers, b);
    if (st != MMF_OK) return st;
    Carver c(nullptr);
    *bytes = stack_plan(c, n_layers, b, layers[0].d, layers[0].inner, nullptr);
    return MMF_OK;
}

static mmf_status check_stack_ws(const mmf_layer_weights *layers, int32_t n_layers, int64_t b, void *ws, size_t ws_bytes) {
    size_t need = 0;
    mmf_status st = mmf_stack_decode_workspace_size(layers, n_layers, b, &need);
    if (st != MMF_OK) return st;
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(MMF_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
    return MMF_OK;
}

mmf_status mmf_stack_decode_bind(const mmf_layer_weights *layers, int32_t n_layers, int64_t b, float *const *h,
                                 void *ws, size_t ws_bytes, hipStream_t stream) {
    mmf_status st = check_stack_ws(layers, n_layers, b, ws, ws_bytes);
    if (st != MMF_OK) return st;
    if (!h) return fail(MMF_ERR_INVALID_ARG, "h is NULL");
    std::vector<StackLayer> table((size_t)n_layers);
    for (int32_t l = 0; l < n_layers; ++l) {
        const mmf_layer_weights &w = layers[l];
        if (!h[l] || !aligned16(h[l])) return fail(MMF_ERR_INVALID_ARG, "h[%d] must be non-NULL and 16-byte aligned", (int)l);
        const mmf_ternary_weight *tw[6] = {&w.i, &w.f, &w.g, &w.o, &w.gate, &w.down};
        StackLayer &t = table[l];
        for (int q = 0; q < 6; ++q) {
            t.w[q] = tw[q]->packed;
            t.mu[q] = tw[q]->mu;
            t.gain[q] = tw[q]->norm_w;
        }
        t.g_norm_w = w.g_norm_w;
        t.h = h[l];
        t.eps = w.eps;
        t.pad = 0;
    }
    Carver c(ws);
    StackWs W;
    stack_plan(c, n_layers, b, layers[0].d, layers[0].inner, &W);
    hipError_t e = hipMemcpyAsync(W.table, table.data(), table.size() * sizeof(StackLayer), hipMemcpyHostToDevice,
                                  stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);  // the host table goes out of scope
    return hip_status(e, "mmf_stack_decode_bind");
}

mmf_status mmf_stack_decode_step(const mmf_layer_weights *layers, int32_t n_layers, const void *x, void *out,
                                 mmf_dtype actt, int64_t b, void *ws, size_t ws_bytes, hipStream_t stream) {
    mmf_status st = check_stack_ws(layers, n_layers, b, ws, ws_bytes);
    if (st != MMF_OK) return st;
    if (!valid_dtype(actt)) return fail(MMF_ERR_INVALID_ARG, "bad activation dtype");
    if (!x || !out) return fail(MMF_ERR_INVALID_ARG, "x and out must be non-NULL");
    if (!aligned16(x) || !aligned16(out)) return fail(MMF_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
    if (x == out) return fail(MMF_ERR_INVALID_ARG, "x and out must not overlap");
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
        return fail(MMF_ERR_UNSUPPORTED, "a cooperative launch cannot be captured into a HIP graph");
    Carver c(ws);
    StackWs W;
    stack_plan(c, n_layers, b, layers[0].d, layers[0].inner, &W);
    StackArgs a{};
    a.layers = W.table;
    a.n_layers = n_layers;
    a.d = layers[0].d;
    a.inner = layers[0].inner;
    a.b = (int)b;
    a.act_type = act(actt);
    a.x = x;
    a.out = out;
    a.act[0] = W.act[0];
    a.act[1] = W.act[1];
    a.g = W.g;
    a.x1 = W.x1;
    a.z = W.z;
    a.codes = W.codes;
    a.s = W.s;
    a.sumq = W.sumq;
    a.bar = W.bar;
    std::string path;
    hipError_t e = timed("stack_decode", b, n_layers, a.d, stream, [&] { return launch_stack_decode(a, stream, &path); });
    mmf_status r = hip_status(e, "mmf_stack_decode_step");
    if (r == MMF_OK) g_path = path;
    return r;
}

mmf_status mmf_stack_decode_expired(uint32_t *count) {
    if (!count) return fail(MMF_ERR_INVALID_ARG, "count is NULL");
    unsigned c = 0;
    mmf_status r = hip_status(stack_decode_expired_waits(&c), "mmf_stack_decode_expired");
    if (r == MMF_OK) *count = c;
    return r;
}

// --------------------------------------------------------- block derivative --
struct LayerBwdWs {
    int8_t *codes_x[3];
    float *s_x[3];
    int32_t *sq_x[3];
    float *ih, *fh, *gh, *f, *xt, *h, *u, *x1, *ab;
    float *g, *z;  // fp32
    int8_t *codes_b;
    float *s_b;
    int32_t *sq_b;
    float *dz, *dab, *dx1g, *dx1, *du, *dh, *dg, *df, *dxi, *dxf, *dxg, *wpart, *wpart2;
    void *scan;
    BitlinearBwdWs blin;
};

size_t layer_bwd_plan(Carver &c, const mmf_layer_weights *w, int64_t b, int64_t t, int chunks, LayerBwdWs *o) {
    const int64_t m = b * t;
    const size_t d = (size_t)w->d, inner = (size_t)w->inner, md = (size_t)m * d;
    LayerBwdWs L{};
    for (int q = 0; q < 3; ++q) {
        L.codes_x[q] = c.take<int8_t>(md);
        L.s_x[q] = c.take<float>(m);
        L.sq_x[q] = c.take<int32_t>(m);
    }
    float **f32s[] = {&L.ih, &L.fh, &L.gh, &L.f, &L.xt, &L.h, &L.u, &L.x1, &L.dx1g, &L.dx1, &L.du, &L.dh, &L.dg,
                      &L.df, &L.dxi, &L.dxf, &L.dxg};
    for (float **p : f32s) *p = c.take<float>(md);
    L.g = c.take<float>(md);
    L.ab = c.take<float>((size_t)m * 2 * inner);
    L.dab = c.take<float>((size_t)m * 2 * inner);
    L.z = c.take<float>((size_t)m * inner);
    L.dz = c.take<float>((size_t)m * inner);
    L.codes_b = c.take<int8_t>((size_t)m * (d > inner ? d : inner));
    L.s_b = c.take<float>(m);
    L.sq_b = c.take<int32_t>(m);
    const int64_t rows = m > 0 ? rmsnorm_bwd_rows(m) : 1;
    const int64_t nblk = (m + rows - 1) / rows;
    L.wpart = c.take<float>((size_t)nblk * d);
    L.wpart2 = c.take<float>((size_t)gain_reduce_splits((int)nblk) * d);
    L.scan = c.take<char>(scan_workspace_bytes(b, w->d, chunks));
    const int nmax = 2 * w->inner > w->d ? 2 * w->inner : w->d;
    const int kmax = w->inner > w->d ? w->inner : w->d;
    const mmf_ternary_weight *tw[6] = {&w->i, &w->f, &w->g, &w->o, &w->gate, &w->down};
    size_t split_floats = 0;  // the largest split product of the six projections
    for (const mmf_ternary_weight *p : tw) {
        const size_t f = dw_split_floats(m, p->n, p->k);
        if (f > split_floats) split_floats = f;
    }
    bitlinear_bwd_plan(c, m, nmax, kmax, MMF_F32, &L.blin, split_floats);
    if (o) *o = L;
    return c.off;
}

mmf_status mmf_layer_bwd_workspace_size(const mmf_layer_weights *w, int64_t b, int64_t t, size_t *bytes) {
    if (!bytes) return fail(MMF_ERR_INVALID_ARG, "bytes is NULL");
    mmf_status st = check_layer(w);
    if (st != MMF_OK) return st;
    if (b < 0 || t < 0) return fail(MMF_ERR_INVALID_ARG, "b, t must be >= 0");
    Carver c(nullptr);
    *bytes = layer_bwd_plan(c, w, b, t, scan_pick_chunks(b, t, w->d, MMF_SCAN_CHUNK), nullptr);
    return MMF_OK;
}

mmf_status mmf_layer_bwd(const mmf_layer_weights *w, const void *x, const void *dout, mmf_dtype actt, int64_t b,
                         int64_t t, const float *h0, const float *dh_last, mmf_scan_mode mode,
                         const mmf_layer_grads *gr, void *ws, size_t ws_bytes, hipStream_t stream) {
    size_t need = 0;
    mmf_status st = mmf_layer_bwd_workspace_size(w, b, t, &need);
    if (st != MMF_OK) return st;
    if (!valid_dtype(actt)) return fail(MMF_ERR_INVALID_ARG, "bad activation dtype");
    if (mode != MMF_SCAN_AUTO && mode != MMF_SCAN_RECURRENT && mode != MMF_SCAN_CHUNK)
        return fail(MMF_ERR_INVALID_ARG, "bad scan mode %d", (int)mode);
    if (!gr) return fail(MMF_ERR_INVALID_ARG, "grads is NULL");
    const int64_t m = b * t;
    const int d = w->d, inner = w->inner;
    if (m > 0 && (!x || !dout || !gr->dx)) return fail(MMF_ERR_INVALID_ARG, "x, dout and grads->dx must be non-NULL");
    if (!rmsnorm_bwd_supported(d) || !rmsnorm_bwd_supported(inner) || (2 * inner) % 8 || d % 8)
        return fail(MMF_ERR_UNSUPPORTED, "d=%d, inner=%d outside the derivative kernels' limits", d, inner);
    if (m > INT32_MAX) return fail(MMF_ERR_UNSUPPORTED, "b*t beyond 32-bit GEMM sizes");
    if (!aligned16(x) || !aligned16(dout) || !aligned16(gr->dx) || !aligned16(h0) || !aligned16(dh_last))
        return fail(MMF_ERR_INVALID_ARG, "x, dout, dx, h0 and dh_last must be 16-byte aligned");
    if (m > 0 && (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)))
        return fail(MMF_ERR_WORKSPACE, "workspace needs %zu bytes, 256-byte aligned", need);
    const mmf_ternary_weight *tw[6] = {&w->i, &w->f, &w->g, &w->o, &w->gate, &w->down};
    std::string path;
    hipError_t e = hipSuccess;
    if (m == 0) {
        // no tokens: h_last is h0, and every weight and gain sees nothing
        if (gr->dh0 && b > 0) e = launch_scan_bwd(nullptr, nullptr, nullptr, nullptr, dh_last, nullptr, nullptr, gr->dh0,
                                                  b, 0, d, 1, stream, &path);
        for (int q = 0; q < 6 && e == hipSuccess; ++q) {
            if (gr->dw[q]) e = launch_zero_f32(gr->dw[q], (int64_t)tw[q]->n * tw[q]->k, stream);
            if (e == hipSuccess && gr->dgain[q]) e = launch_zero_f32(gr->dgain[q], tw[q]->k, stream);
        }
        if (e == hipSuccess && gr->dg_norm_w) e = launch_zero_f32(gr->dg_norm_w, d, stream);
        mmf_status r = hip_status(e, "mmf_layer_bwd");
        if (r == MMF_OK) g_path = "empty";
        return r;
    }
    const ActType at = act(actt);
    const float eps = w->eps;
    const int chunks = scan_pick_chunks(b, t, d, (int)mode);
    Carver c(ws);
    LayerBwdWs L;
    layer_bwd_plan(c, w, b, t, scan_pick_chunks(b, t, d, MMF_SCAN_CHUNK), &L);
    const int64_t md = m * d;
    // ---- the forward again, keeping what the derivative needs
    const bool shared = shared_ifg(w);
    float *pre[3] = {L.ih, L.fh, L.gh};
    for (int q = 0; q < 3 && e == hipSuccess; ++q) {
        const int src = shared ? 0 : q;
        if (src == q) e = t_norm_quant(x, at, m, d, tw[q]->norm_w, eps, L.codes_x[q], L.s_x[q], L.sq_x[q], stream, &path);
        if (e != hipSuccess) break;
        ContractArgs ca{};
        for (int j = 0; j < 3; ++j) { ca.A[j] = L.codes_x[src]; ca.s[j] = L.s_x[src]; ca.sumq[j] = L.sq_x[src]; ca.B[j] = tw[q]->packed; ca.mu[j] = tw[q]->mu; }
        ca.m = m; ca.nc = d; ca.k = d;
        ca.out0 = pre[q]; ca.out_type = ACT_F32;
        e = t_contract(ca, EPI_LINEAR, 1, true, stream, &path);
    }
    if (e == hipSuccess) e = launch_gates_keep(L.ih, L.fh, L.gh, md, L.f, L.xt, L.g, ACT_F32, stream);
    if (e == hipSuccess) e = t_scan(L.xt, L.f, h0, L.h, nullptr, b, t, d, chunks, L.scan, stream, &path);
    if (e == hipSuccess)
        e = t_gnorm_quant(L.h, L.g, ACT_F32, m, d, w->g_norm_w, w->o.norm_w, eps, L.codes_b, L.s_b, L.sq_b, L.u, stream,
                          &path);
    if (e == hipSuccess) {
        ContractArgs co{};
        for (int j = 0; j < 3; ++j) { co.A[j] = L.codes_b; co.s[j] = L.s_b; co.sumq[j] = L.sq_b; co.B[j] = w->o.packed; co.mu[j] = w->o.mu; }
        co.m = m; co.nc = d; co.k = d;
        co.out0 = L.x1; co.out_type = ACT_F32; co.res = x; co.res_type = at;
        e = t_contract(co, EPI_RESID, 1, true, stream, &path);
    }
    if (e == hipSuccess) e = t_norm_quant(L.x1, ACT_F32, m, d, w->gate.norm_w, eps, L.codes_b, L.s_b, L.sq_b, stream, &path);
    if (e == hipSuccess) {
        ContractArgs cg{};
        for (int j = 0; j < 3; ++j) { cg.A[j] = L.codes_b; cg.s[j] = L.s_b; cg.sumq[j] = L.sq_b; cg.B[j] = w->gate.packed; cg.mu[j] = w->gate.mu; }
        cg.m = m; cg.nc = 2 * inner; cg.k = d;
        cg.out0 = L.ab; cg.out_type = ACT_F32;
        e = t_contract(cg, EPI_LINEAR, 1, true, stream, &path);
    }
    if (e == hipSuccess) e = launch_glu_keep(L.ab, m, inner, L.z, ACT_F32, stream);
    // ---- derivatives, last step first
    if (e == hipSuccess)  // down_proj: dz
        e = bitlinear_bwd_run(L.z, ACT_F32, m, &w->down, eps, dout, at, L.dz, ACT_F32, gr->dw[5], gr->dgain[5],
                              L.blin, stream, &path);
    if (e == hipSuccess) e = launch_glu_bwd(L.dz, L.ab, m, inner, L.dab, stream);
    if (e == hipSuccess)  // gate_proj: into x1
        e = bitlinear_bwd_run(L.x1, ACT_F32, m, &w->gate, eps, L.dab, ACT_F32, L.dx1g, ACT_F32, gr->dw[4], gr->dgain[4],
                              L.blin, stream, &path);
    if (e == hipSuccess) e = launch_sum(dout, at, L.dx1g, nullptr, nullptr, md, L.dx1, stream);  // + the residual
    if (e == hipSuccess)  // o_proj: du
        e = bitlinear_bwd_run(L.u, ACT_F32, m, &w->o, eps, L.dx1, ACT_F32, L.du, ACT_F32, gr->dw[3], gr->dgain[3], L.blin,
                              stream, &path);
    if (e == hipSuccess)  // g_norm: dh, dg^ and the weight's partial sums
        e = launch_gnorm_bwd(L.h, L.g, ACT_F32, L.du, w->g_norm_w, eps, m, d, L.dh, L.dg,
                             gr->dg_norm_w ? L.wpart : nullptr, stream);
    if (e == hipSuccess && gr->dg_norm_w) {
        const int rows = rmsnorm_bwd_rows(m);
        e = launch_gain_reduce(L.wpart, (int)((m + rows - 1) / rows), d, L.wpart2, gr->dg_norm_w, stream);
    }
    if (e == hipSuccess)  // the recurrence: dx~ (over dh), df, dh0
        e = launch_scan_bwd(L.f, L.h, h0, L.dh, dh_last, L.dh, L.df, gr->dh0, b, t, d, scan_bwd_pick(t, (int)mode),
                            stream, &path);
    if (e == hipSuccess) e = launch_gates_bwd(L.dh, L.df, L.ih, L.f, md, stream);  // -> di^, df^
    const float *dpre[3] = {L.dh, L.df, L.dg};
    float *dxq[3] = {L.dxi, L.dxf, L.dxg};
    for (int q = 0; q < 3 && e == hipSuccess; ++q)
        e = bitlinear_bwd_run(x, at, m, tw[q], eps, dpre[q], ACT_F32, dxq[q], ACT_F32, gr->dw[q], gr->dgain[q], L.blin,
                              stream, &path);
    if (e == hipSuccess) e = launch_sum(L.dx1, ACT_F32, L.dxi, L.dxf, L.dxg, md, gr->dx, stream);
    mmf_status r = hip_status(e, "mmf_layer_bwd");
    if (r == MMF_OK) g_path = path;
    return r;
}

mmf_status mmf_hbm_ceiling(int mode, const void *src, void *dst, int64_t bytes, hipStream_t stream) {
    if (mode < 0 || mode > 2) return fail(MMF_ERR_INVALID_ARG, "mode %d (0 read, 1 copy, 2 two reads one write)", mode);
    if (bytes <= 0 || bytes % 16) return fail(MMF_ERR_INVALID_ARG, "bytes=%lld must be a positive multiple of 16",
                                             (long long)bytes);
    if (!src || !dst || !aligned16(src) || !aligned16(dst))
        return fail(MMF_ERR_INVALID_ARG, "src and dst must be non-NULL and 16-byte aligned");
    if (ceiling_blocks() * 4 > MMF_HBM_CEILING_SINK_BYTES) return fail(MMF_ERR_INVALID_ARG, "sink too small");
    const char *s = static_cast<const char *>(src);
    const char *d = static_cast<const char *>(dst);
    const int64_t slen = mode == 2 ? 2 * bytes : bytes;
    const int64_t dlen = mode == 0 ? MMF_HBM_CEILING_SINK_BYTES : bytes;
    if (s < d + dlen && d < s + slen) return fail(MMF_ERR_INVALID_ARG, "src and dst overlap");
    static const char *names[] = {"stream_read", "stream_copy", "stream_2r1w"};
    std::string path = std::string(names[mode]) + ";";
    const hipError_t e = timed(names[mode], bytes, 0, 0, stream, [&] {
        if (mode == 0) return launch_stream_read(src, bytes, static_cast<uint32_t *>(dst), stream);
        return launch_stream_copy(src, mode == 2 ? s + bytes : nullptr, dst, bytes, stream);
    });
    mmf_status r = hip_status(e, "mmf_hbm_ceiling");
    if (r == MMF_OK) g_path = path;
    return r;
}

mmf_status mmf_mfma_ceiling(int64_t iters, void *sink, int64_t sink_bytes, int64_t *ops, hipStream_t stream) {
    if (iters <= 0) return fail(MMF_ERR_INVALID_ARG, "iters=%lld must be positive", (long long)iters);
    if (!sink || !ops) return fail(MMF_ERR_INVALID_ARG, "sink and ops must be non-NULL");
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_status(e, "mmf_mfma_ceiling");
    const int blocks = mfma_ceiling_blocks(cus);
    if (sink_bytes < (int64_t)blocks * 4)
        return fail(MMF_ERR_INVALID_ARG, "sink needs %lld bytes (one word per workgroup)", (long long)blocks * 4);
    *ops = mfma_loop_ops(iters, blocks);
    e = timed("mfma_loop", iters, blocks, 0, stream,
              [&] { return launch_mfma_loop(iters, blocks, static_cast<uint32_t *>(sink), stream); });
    mmf_status r = hip_status(e, "mmf_mfma_ceiling");
    if (r == MMF_OK) g_path = "mfma_loop;";
    return r;
}

mmf_status mmf_timing_enable(int on) {
    if (on) {
        g_recs.clear();
        g_events_used = 0;
    }
    g_timing = on != 0;
    g_err.clear();
    return MMF_OK;
}

mmf_status mmf_timing_collect(mmf_kernel_timing *out, int32_t capacity, int32_t *count) {
    if (!count || capacity < 0 || (capacity > 0 && !out)) return fail(MMF_ERR_INVALID_ARG, "bad timing buffer");
    *count = (int32_t)g_recs.size();
    for (size_t i = 0; i < g_recs.size() && (int32_t)i < capacity; ++i) {
        const TimingRec &r = g_recs[i];
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_status(e, "mmf_timing_collect");
        float ms = 0.0f;
        if ((e = hipEventElapsedTime(&ms, r.start, r.stop)) != hipSuccess) return hip_status(e, "mmf_timing_collect");
        mmf_kernel_timing &o = out[i];
        std::memset(&o, 0, sizeof o);
        std::strncpy(o.kernel, r.kernel.c_str(), sizeof(o.kernel) - 1);
        o.m = r.m;
        o.n = r.n;
        o.k = r.k;
        o.ms = ms;
    }
    g_err.clear();
    return MMF_OK;
}

}  // extern "C"
