// Host-side launchers of the libmmf kernels (internal to the library).
// Every launcher enqueues on `stream` and returns hipGetLastError()'s result;
// arguments are validated by the C-ABI layer before these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

namespace mmf {

enum ActType { ACT_F32 = 0, ACT_BF16 = 1 };

// Every kernel of the library is launched through here (one launch point).
template <typename... KP, typename... A>
inline void launch_k(void (*kernel)(KP...), dim3 grid, dim3 block, size_t lds, hipStream_t st, A... args) {
    kernel<<<grid, block, lds, st>>>(args...);
}

// Row RMSNorm + absmax int8 quantiser over m rows of k elements.
hipError_t launch_norm_quant(const void *x, ActType xt, int64_t m, int k, const float *gain, float eps,
                             int8_t *q, float *s, int32_t *sumq, hipStream_t stream, std::string *path);

// g_norm (RMSNorm(h) * w * SiLU(g)) followed by the o_proj quantiser; u_out optional.
hipError_t launch_gnorm_quant(const float *h, const void *g, ActType g_type, int64_t m, int d, const float *g_norm_w,
                              const float *o_gain, float eps, int8_t *q, float *s, int32_t *sumq,
                              float *u_out, hipStream_t stream, std::string *path);

// Ternarise + pack. ws must hold pack_workspace_bytes().
size_t pack_workspace_bytes();
hipError_t launch_pack(const float *w, int n, int k, uint32_t *packed, float *mu, void *ws,
                       hipStream_t stream, std::string *path);

// Epilogues of the ternary contraction.
enum EpiKind {
    EPI_LINEAR = 0,      // NG=1: y = acc * dq                      (out0, dtype out_type)
    EPI_RESID = 1,       // NG=1: y = res + acc * dq                (out0, dtype out_type; res dtype res_type)
    EPI_GATES = 2,       // NG=3: f = sig(f^), xt = (1-f) SiLU(i^), g = g^   (out0 f, out1 xt fp32; out2 g, aux)
    EPI_GATES_STEP = 3,  // NG=3: h = f h + xt in place on out0; g to out1 (aux); f/xt probes out2/out3
    EPI_GLU = 4          // NG=2: z = SiLU(a) * b                   (out0, aux)
};

struct ContractArgs {
    // per group (i/f/g, or the two halves of gate_proj, or one tensor)
    const int8_t *A[3];      // codes [m][k]
    const float *s[3];       // activation scale per row
    const int32_t *sumq[3];  // sum of codes per row (read by the prefill kernels only)
    const uint32_t *B[3];    // packed rows [nc][k/16]
    const float *mu[3];      // device scalar per group
    int64_t m;
    int nc;                  // output channels per group
    int k;
    void *out0, *out1, *out2, *out3;
    const void *res;
    int32_t *acc_probe;      // [m][ng*nc] (group-major within a row) or NULL
    ActType out_type, res_type;
    ActType aux_type;        // storage type of the g (gates) or z (GLU) output
    float *aux_probe;        // optional fp32 copy of g / z as stored (after rounding to aux_type)
};

// The input rows of a contraction that quantises them itself: x [m][k] in the
// activation type, or (gated g_norm) y = ((h r_h) w) silu(g) formed from h
// [m][k] fp32, g [m][k] in the activation type and the optional gain w [k].
// Optional stage outputs, written by workgroup 0 only: the rows' int8 codes
// [m][k] and scales [m], and (gated g_norm) the gated row u [k] before
// o_proj's own gain.
struct RowSrc {
    const void *x;       // x, or h
    const void *g;       // g (gated g_norm only)
    const float *gnw;    // g_norm's gain or NULL (gated g_norm only)
    const float *gain;   // the FusedBitLinear gain of x, or o_proj's after the gated g_norm; or NULL
    int8_t *codes_out;   // or NULL
    float *scale_out;    // or NULL
    float *u_out;        // or NULL
};

// Prefill-shaped contraction (int8 MFMA tiles) and decode-shaped one (m <= 64).
hipError_t launch_contract(const ContractArgs &a, EpiKind epi, int ng, bool shared_a,
                           hipStream_t stream, std::string *path);

// Decode at up to 16 rows: the contraction quantises its input rows x (type
// xt) itself in every workgroup; a.A, a.s, a.sumq unused. codes_out [m][k] and
// scale_out [m] (each optional) receive the rows' codes and scales.
bool contract_row_supported(int64_t m, int k, EpiKind epi, bool gain);
hipError_t launch_contract_row(const ContractArgs &a, EpiKind epi, const void *x, ActType xt, const float *gain,
                               float eps, int8_t *codes_out, float *scale_out, hipStream_t st, std::string *path);
// o_proj over the gated g_norm of (h, g), quantised in each workgroup (EPI_RESID
// only); optional outputs: the codes, the scale and the gated row u.
bool contract_row_gnorm_supported(int64_t m, int k);
hipError_t launch_contract_row_gnorm(const ContractArgs &a, const float *h, const void *g, ActType gt,
                                     const float *gnw, const float *ogain, float eps, int8_t *codes_out,
                                     float *scale_out, float *u_out, hipStream_t st, std::string *path);

// Whether the contraction over m rows forms each row's sum of codes itself
// (the decode GEMV does); otherwise it reads the quantiser's sumq.
bool contract_sums_codes(int64_t m);

// Variant name of the kernel launch_contract picks, e.g. "tgemm<gates>".
std::string contract_variant(int64_t m, int k, EpiKind epi, bool shared_a);

// HGRN scan. chunks == 1 means the recurrent (sequential) kernel, kScanTiled
// the single-pass tiled kernel, chunks >= 2 the two-pass chunked kernels.
constexpr int kScanTiled = -1;
size_t scan_workspace_bytes(int64_t b, int64_t d, int chunks);
int scan_pick_chunks(int64_t b, int64_t t, int64_t d, int mode);
hipError_t launch_scan(const float *x, const float *f, const float *h0, float *h, float *h_last,
                       int64_t b, int64_t t, int64_t d, int chunks, void *ws, hipStream_t stream,
                       std::string *path);

// The expanded-state recurrence (k_hgrn2.hip): e in {16, 32, 64, 128}, d % e == 0;
// s0 NULL means zeros, s_last may equal s0; chunk picks the chunked kernel (e of 64
// or 128), else the step-wise one; name gets the variant.
int64_t hgrn2_workgroups(int64_t b, int64_t d, int e);
hipError_t launch_hgrn2_scan(const float *f, const float *i, const float *o, const float *s0, float *y,
                             float *s_last, int64_t b, int64_t t, int64_t d, int e, bool chunk, hipStream_t st,
                             const char **name);

// Backward of the HGRN scan: 1 = recurrent, kScanTiled = single-pass tiled
// (reverse time). dh0 and dh_last optional; h0 NULL means zeros.
int scan_bwd_pick(int64_t t, int mode);
hipError_t launch_scan_bwd(const float *f, const float *h, const float *h0, const float *dh, const float *dh_last,
                           float *dx, float *df, float *dh0, int64_t b, int64_t t, int64_t d, int plan,
                           hipStream_t stream, std::string *path);

// Derivative of FusedBitLinear: its two products as hand-written bf16 GEMMs
// (k_gemm_bf16.hip): C[m][n] (fp32, row stride ldc) = A[m][k] B[n][k]^T with bf16
// operands whose rows are k-contiguous (strides lda, ldb elements; k % 8 == 0, rows
// 16-byte aligned); the operand layouts: t^T [k][ldn] bf16 from the packed words
// (columns n..ldn-1 zero), and out [cols][ldm] bf16 = the transpose of src
// [rows][cols] (src_kind 0: fp32 scaled by 1 / s per row, 1: bf16 scaled, 2:
// int8 codes as they are; columns rows..ldm-1 zero; ldm % 8 == 0).
// With part non-NULL a product of few tiles may be split along k: part must hold
// gemm_bf16_splits(m, n, k) * m * ldc floats (the per-split partial blocks).
int gemm_bf16_splits(int m, int n, int k);
hipError_t launch_gemm_bf16_nt(const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb, int m, int n, int k,
                               float *c, int64_t ldc, float *part, hipStream_t st);
hipError_t launch_expand_ternary_t(const uint32_t *packed, int n, int k, uint16_t *out, int ldn, hipStream_t st);
hipError_t launch_transpose_bf16(const void *src, int src_kind, const float *s, int64_t rows, int cols, uint16_t *out,
                                 int64_t ldm, hipStream_t st);
// The rest of the derivative (k_bwd.hip): fp32 -> bf16, the RMSNorm derivative
// (du = du_raw / sw; optional dx, per-workgroup partial sums of the gain's
// derivative) and their reduction.
hipError_t launch_to_bf16(const float *x, int64_t n, uint16_t *out, hipStream_t st);
int rmsnorm_bwd_rows(int64_t m);
bool rmsnorm_bwd_supported(int k);
hipError_t launch_rmsnorm_bwd(const void *x, ActType xt, const float *du_raw, const float *gain, const float *mu,
                              float eps, int64_t m, int k, void *dx, ActType dxt, float *gpart, hipStream_t st);
int gain_reduce_splits(int nblk);  // rows of the second level's workspace ([splits][k] fp32)
hipError_t launch_gain_reduce(const float *gpart, int nblk, int k, float *part2, float *dgain, hipStream_t st);
hipError_t launch_zero_f32(float *p, int64_t n, hipStream_t st);  // a fill kernel (capturable)
// The block derivative's elementwise pieces (k_bwd.hip): the forward's gate and
// GLU values kept for the derivative (same operations as the fused
// epilogues; g, z in the activation type), the GLU and gate derivatives, an
// elementwise sum, and g_norm's row-wise derivative with per-workgroup partial
// sums of its weight's derivative (rows per workgroup: rmsnorm_bwd_rows).
hipError_t launch_gates_keep(const float *ih, const float *fh, const float *gh, int64_t n, float *f, float *xt, void *g,
                             ActType gt, hipStream_t st);
hipError_t launch_glu_keep(const float *ab, int64_t m, int inner, void *z, ActType zt, hipStream_t st);
hipError_t launch_glu_bwd(const float *dz, const float *ab, int64_t m, int inner, float *dab, hipStream_t st);
hipError_t launch_gates_bwd(float *dxt, float *df, const float *ih, const float *f, int64_t n, hipStream_t st);
hipError_t launch_sum(const void *a, ActType at, const float *b, const float *c, const float *d, int64_t n, float *out,
                      hipStream_t st);
hipError_t launch_gnorm_bwd(const float *h, const void *g, ActType gt, const float *du, const float *w, float eps,
                            int64_t m, int d, float *dh, float *dg, float *wpart, hipStream_t st);

// Measured HBM ceilings (k_ceiling.hip): a streaming read of `bytes` (a
// multiple of 16; one word per workgroup to sink, ceiling_blocks() words), a
// streaming copy, and with src2 two read streams into one write stream.
int ceiling_blocks();
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t st);
hipError_t launch_stream_copy(const void *src, const void *src2, void *dst, int64_t bytes, hipStream_t st);

// Generation (k_generate.hip): embedding rows (16-byte pieces of a row of
// row_bytes; zero rows for ids outside [0, vocab)), and per row of an int32
// matrix [m][n] (n % 4 == 0) the smallest index of its largest value.
hipError_t launch_embed(const int32_t *ids, int64_t count, const void *table, int64_t vocab, int64_t row_bytes,
                        void *out, hipStream_t st);
hipError_t launch_argmax_rows(const int32_t *acc, int64_t m, int64_t n, int32_t *tokens, hipStream_t st);

}  // namespace mmf
