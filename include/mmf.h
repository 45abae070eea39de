/*
 * mmf.h -- C ABI of the MI355X (gfx950) HGRNBit layer forward library, libmmf.so.
 *
 * The operations follow the MatMul-free LM model as described on:
 *   [R1] "MatMul-Free LLM 深度分析报告" (nightvoyager.top), section "核心价值提炼":
 *        table "创新之处" (ternary weight_quant, round to nearest {-1,0,+1};
 *        HGRN recurrence h_t = gate_t * h_{t-1} + x_t with a step-wise and a
 *        chunked form) and list "可复用的模式与技巧" (RMSNorm fused with INT8
 *        activation quantisation; RMSNorm fused with a Swish gate).
 *   [R3] "MatMul-Free LM：把矩陣乘法從語言模型裡拿掉之後，剩下什麼" (hysenlabs.com),
 *        section "HGRNBitBlock 的結構": i/f/g/o FusedBitLinear projections, each
 *        with an eps = 1e-8 RMSNorm, a g_norm RMSNorm-Swish gate, an MLP of
 *        gate_proj (2 x inner outputs), SiLU and down_proj; section
 *        "什麼情況下這個工具是錯的選擇" (a FusedBitLinear that silently falls back to
 *        a slow path is a failure mode: here every call reports its path).
 *   [R4] mooersco.com article, sections 4.1 and 5.1 (ternary product as
 *        conditional add/subtract; pack low-bit weights into words).
 * Readings where the pages are silent (stated with the operations below):
 * per-token absmax int8 scale 127/amax, per-tensor mean-|W| weight scale,
 * f = sigmoid(f_proj), x~ = (1 - f) * SiLU(i_proj), SiLU(first half of
 * gate_proj) * second half, plain residual adds, no bias.
 *
 * Conventions (all entry points):
 *  - Every tensor pointer is DEVICE memory owned by the caller; struct
 *    arguments are host memory read during the call only. The library
 *    allocates nothing, keeps no state between calls and never synchronises:
 *    all work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *    Scratch memory comes from the caller's workspace (`ws`, `ws_bytes`,
 *    256-byte aligned), sized by the matching *_workspace_size call.
 *  - Layouts are row-major with the last dimension contiguous. Activation
 *    tensors are [rows][features]; sequences are [b][t][d].
 *  - Arguments are validated on the host before any HIP call. A failure
 *    returns a status other than MMF_OK, enqueues nothing and sets the
 *    thread-local message read by mmf_last_error(). A failed kernel launch
 *    returns MMF_ERR_HIP; faults during execution surface at the caller's
 *    next synchronisation.
 *  - Inputs and outputs must not overlap, except where an entry point says so.
 *  - mmf_last_path() names the kernel variants the last successful call on
 *    this thread launched (there is no silent fallback to another path).
 */
#ifndef MMF_H
#define MMF_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enumerated values travel as plain 32-bit integers, so any value a caller
 * passes is well defined and is checked (an unknown one is INVALID_ARG). */
typedef int32_t mmf_status;
enum {
    MMF_OK = 0,
    MMF_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad enum value      */
    MMF_ERR_UNSUPPORTED = 2,   /* valid but not handled (e.g. k % 16 != 0)     */
    MMF_ERR_WORKSPACE = 3,     /* workspace missing, too small or misaligned   */
    MMF_ERR_HIP = 4            /* a HIP launch or runtime call failed          */
};

typedef int32_t mmf_dtype;
enum { MMF_F32 = 0, MMF_BF16 = 1 };

/* [R1] the recurrence has a step-wise and a chunked implementation. */
typedef int32_t mmf_scan_mode;
enum {
    MMF_SCAN_AUTO = 0,         /* library picks from b*d and t                 */
    MMF_SCAN_RECURRENT = 1,    /* sequential in t per channel: same order as the definition */
    MMF_SCAN_CHUNK = 2         /* t split in chunks, carries composed as (a,b) pairs */
};

/*
 * One packed ternary weight ([R1] weight_quant; [R4] section 5.1 packing).
 *  packed : [n][k/16] uint32. Word w of row r holds the codes c = t + 1 in
 *           {0,1,2} of t[r][16w .. 16w+15]; t[r][16w + 4j + b] sits at bits
 *           [8b + 2j, 8b + 2j + 2) (j, b in 0..3), so (word >> 2j) & 0x03030303
 *           is four int8 codes in k order. Code 3 is never written.
 *  mu     : device scalar, mean |W| of the latent tensor (binary32).
 *           The weight approximates W ~ t / sw with sw = 1 / max(mu, 1e-5).
 *  norm_w : [k] gain of this projection's input RMSNorm, or NULL for ones.
 *  n, k   : output and input features; k % 16 == 0.
 */
typedef struct {
    const uint32_t *packed;
    const float *mu;
    const float *norm_w;
    int32_t n, k;
} mmf_ternary_weight;

/*
 * One HGRNBit block ([R3] section "HGRNBitBlock 的結構").
 *  i, f, g, o : n = k = d.  gate : n = 2*inner, k = d (rows [0, inner) are the
 *  SiLU branch, rows [inner, 2*inner) the linear branch, one mu for the whole
 *  tensor).  down : n = d, k = inner.  g_norm_w : [d] or NULL.
 *  eps : RMSNorm epsilon of every norm in the block (1e-8 on [R3]).
 */
typedef struct {
    mmf_ternary_weight i, f, g, o, gate, down;
    const float *g_norm_w;
    int32_t d, inner;
    float eps;
} mmf_layer_weights;

/*
 * Optional stage outputs of a layer call, for validation. Every pointer may be
 * NULL; non-NULL ones receive the named stage over all m = b*t rows (decode:
 * m = b). Element types are fixed (fp32 for real-valued stages) whatever the
 * activation dtype. When the i/f/g gains are the same pointer (or all NULL)
 * x is quantised once and only codes_x[0] / scale_x[0] are written.
 */
typedef struct {
    int8_t *codes_x[3];  float *scale_x[3];    /* quantised x for i, f, g: [m][d], [m] */
    int32_t *acc_ifg;                          /* [m][3][d] exact sum t*q for i, f, g   */
    float *f, *xt, *g;                         /* forget gate, scan input, g_proj output [m][d] */
    float *h;                                  /* recurrent state after each token [m][d] */
    float *u;                                  /* g_norm output, o_proj's input [m][d]  */
    int8_t *codes_u;     float *scale_u;
    int32_t *acc_o;                            /* [m][d] */
    float *x1;                                 /* x + o_proj(u) [m][d] */
    int8_t *codes_x1;    float *scale_x1;
    int32_t *acc_gate;                         /* [m][2*inner] */
    float *z;                                  /* SiLU(a) * b [m][inner] */
    int8_t *codes_z;     float *scale_z;
    int32_t *acc_down;                         /* [m][d] */
} mmf_layer_probe;

/* Thread-local text of the last error on this thread ("" if none). */
const char *mmf_last_error(void);

/* Kernel variants launched by the last successful call on this thread. */
const char *mmf_last_path(void);

/*
 * mmf_ternary_pack -- ternarise and pack a latent weight ([R1] weight_quant).
 *  w      : [n][k] fp32 device input.
 *  packed : [n][k/16] uint32 device output (layout above).
 *  mu     : device scalar output, (float)(sum |w| / (n*k)) with the sum in
 *           binary64; then t = clamp(rint(w * sw), -1, 1), rint = round half
 *           to even, sw = 1 / max(mu, 1e-5) in binary32.
 *  Deterministic: the reduction order is fixed for given n, k.
 *  Errors: INVALID_ARG (null, n <= 0, k <= 0), UNSUPPORTED (k % 16),
 *  WORKSPACE (ws_bytes < mmf_ternary_pack_workspace_size).
 */
mmf_status mmf_ternary_pack_workspace_size(int32_t n, int32_t k, size_t *bytes);
mmf_status mmf_ternary_pack(const float *w, int32_t n, int32_t k, uint32_t *packed, float *mu,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * mmf_bitlinear_fwd -- one FusedBitLinear ([R1] RMSNorm + INT8 quantisation
 * fused; [R3] eps; [R4] section 4.1 ternary contraction), no bias:
 *   r     = (float)(1 / sqrt(sum_k x_k^2 / k + eps))   (binary64 inside)
 *   y_k   = (x_k * r) * norm_w_k                       (binary32)
 *   s     = 127 / max(max_k |y_k|, 1e-5)
 *   q_k   = clamp(rint(y_k * s), -128, 127)
 *   acc_n = sum_k q_k * t[n][k]                        (exact int32)
 *   out_n = acc_n / (s * sw)
 *  x : [m][k] in dtype xt.  y : [m][n] in dtype yt.
 *  codes_out [m][k] int8, scale_out [m] fp32 (s), acc_out [m][n] int32: optional.
 *  m may be 0 (nothing is launched). Errors: INVALID_ARG, UNSUPPORTED
 *  (k % 16), WORKSPACE.
 */
mmf_status mmf_bitlinear_workspace_size(int64_t m, int32_t k, size_t *bytes);
mmf_status mmf_bitlinear_fwd(const void *x, mmf_dtype xt, int64_t m, const mmf_ternary_weight *w,
                             float eps, void *y, mmf_dtype yt, int8_t *codes_out, float *scale_out,
                             int32_t *acc_out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * mmf_bitlinear_bwd -- derivative of mmf_bitlinear_fwd with straight-through
 * quantisers ([R1] list "可复用的模式与技巧": weight_quant rounds in the forward
 * pass and lets the gradient through unchanged in the backward pass; the
 * activation quantiser is read the same way). With u = RMSNorm(x) * gain and
 * the forward's dequantised operands u^ = q / s, W^ = t / sw:
 *   du = dy W^;   dw = dy^T u^   (the latent weight's gradient)
 *   dx_k = r gain_k du_k - (r^3 / k) x_k sum_j x_j gain_j du_j,  r = (mean(x^2) + eps)^(-1/2)
 *   dgain_k = sum over rows of du_k x_k r
 *  x : [m][k] in dtype xt (the forward's input); dy : [m][n] in dtype dyt;
 *  dx : [m][k] in dtype dxt or NULL; dw : [n][k] fp32 or NULL; dgain : [k] fp32
 *  or NULL (also without a gain: the derivative at gain = 1). The codes are
 *  recomputed from x with the forward's quantiser. The two products are
 *  hand-written bf16 GEMMs with fp32 accumulation: t and q are exact in bf16;
 *  for du an fp32 dy is rounded to bf16, for dw each dy / s is (one rounding of
 *  the product). Outputs do not alias inputs. m may be 0 (dw and dgain are
 *  zero). Errors: INVALID_ARG, UNSUPPORTED (n % 8, k > 8192), WORKSPACE, HIP.
 */
mmf_status mmf_bitlinear_bwd_workspace_size(int64_t m, const mmf_ternary_weight *w, mmf_dtype dyt,
                                            size_t *bytes);
mmf_status mmf_bitlinear_bwd(const void *x, mmf_dtype xt, int64_t m, const mmf_ternary_weight *w,
                             float eps, const void *dy, mmf_dtype dyt, void *dx, mmf_dtype dxt,
                             float *dw, float *dgain, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * mmf_embed -- embedding rows for token ids, the entry of the token-to-token
 * loop of generation ([R3] section "安裝與初始化：三行指令與一個 config 物件":
 * a 32000-token vocabulary, a generation example):
 *   out[i][:] = table[ids[i]][:]      (a zero row when ids[i] is outside [0, vocab))
 *  ids : [count] int32 (device); table : [vocab][d] in dtype tt; out : [count][d]
 *  in dtype tt. A row must be a whole number of 16 bytes. count may be 0.
 *  Errors: INVALID_ARG, UNSUPPORTED.
 */
mmf_status mmf_embed(const int32_t *ids, int64_t count, const void *table, mmf_dtype tt, int64_t vocab,
                     int32_t d, void *out, hipStream_t stream);

/*
 * mmf_greedy_head -- the next token of each row from a FusedBitLinear head
 * (read as ternary, like every projection of the model): the head's logits are
 * acc_n / (s * sw) with one positive factor per row, so the greedy token is the
 * smallest n holding the largest exact int32 sum acc_n.
 *  x : [b][k] in dtype xt (the last block's output); head : [vocab][k] packed,
 *  vocab % 4 == 0; tokens : [b] int32; logits : [b][vocab] fp32 or NULL.
 *  b may be 0. Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE.
 */
mmf_status mmf_greedy_head_workspace_size(int64_t b, const mmf_ternary_weight *head, size_t *bytes);
mmf_status mmf_greedy_head(const void *x, mmf_dtype xt, int64_t b, const mmf_ternary_weight *head,
                           float eps, int32_t *tokens, float *logits, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * mmf_layer_bwd -- derivative of mmf_layer_fwd with straight-through quantisers
 * (as mmf_bitlinear_bwd) for a loss with dL/dout = dout and dL/dh_last =
 * dh_last (or NULL: 0). The forward is run again from x and h0, keeping the
 * pre-activations; then, last step first: down_proj, the SiLU product, gate_proj
 * plus the residual, o_proj, g_norm (RMSNorm of h times weight times SiLU(g)),
 * the recurrence (mmf_hgrn_scan_bwd), the gates f = sigmoid(f^),
 * x~ = (1 - f) SiLU(i^), and i/f/g, whose input derivatives add to the
 * residual's.
 *  x, dout : [b][t][d] in dtype act; h0, dh_last : [b][d] fp32 or NULL.
 *  grads : dx [b][t][d] fp32 (required); dh0 [b][d]; dw[q] [n][k] and dgain[q]
 *  [k] for q = i, f, g, o, gate, down; dg_norm_w [d] -- each fp32 or NULL.
 *  mode picks the scan kernels of the forward's recompute and of the
 *  derivative. Errors: INVALID_ARG, UNSUPPORTED (d, inner beyond 8192 or not
 *  multiples of 8), WORKSPACE, HIP.
 */
typedef struct {
    float *dx;
    float *dh0;
    float *dw[6];
    float *dgain[6];
    float *dg_norm_w;
} mmf_layer_grads;

mmf_status mmf_layer_bwd_workspace_size(const mmf_layer_weights *w, int64_t b, int64_t t, size_t *bytes);
mmf_status mmf_layer_bwd(const mmf_layer_weights *w, const void *x, const void *dout, mmf_dtype act,
                         int64_t b, int64_t t, const float *h0, const float *dh_last, mmf_scan_mode mode,
                         const mmf_layer_grads *grads, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * mmf_hgrn_scan_fwd -- the HGRN recurrence ([R1] table "创新之处"), fp32:
 *   h[b][t][c] = f[b][t][c] * h[b][t-1][c] + x[b][t][c],   h[b][-1][c] = h0[b][c]
 *  x, f, h : [b][t][d] fp32; h0 : [b][d] or NULL (zeros); h_last : [b][d] or NULL.
 *  h may equal x (in place). RECURRENT evaluates in the definition's order;
 *  CHUNK splits t into chunks, composes chunk carries as (prod f, partial h)
 *  pairs and re-runs each chunk from its carry (same value up to rounding).
 *  t may be 0 (h_last = h0). Errors: INVALID_ARG, WORKSPACE.
 */
mmf_status mmf_hgrn_scan_workspace_size(int64_t b, int64_t t, int64_t d, mmf_scan_mode mode,
                                        size_t *bytes);
mmf_status mmf_hgrn_scan_fwd(const float *x, const float *f, const float *h0, float *h,
                             float *h_last, int64_t b, int64_t t, int64_t d, mmf_scan_mode mode,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * mmf_hgrn_scan_bwd -- derivative of mmf_hgrn_scan_fwd's recurrence, fp32
 * (the recurrence of [R1] table "创新之处", differentiated; [R1] list
 * "可复用的模式与技巧" names training through the quantisers with a
 * straight-through estimator, which leaves this step exact). For a loss with
 * dL/dh = dh [b][t][d] and dL/dh_last = dh_last [b][d] (or NULL: zeros):
 *   D_t   = dh_t + f_{t+1} D_{t+1}     (f_T taken as 1, D_T = dh_last)
 *   dx_t  = D_t;   df_t = D_t * h_{t-1};   dh0 = f_0 * D_0   (h_{-1} = h0 or 0)
 *  f, h (the forward's output), dh, dx, df : [b][t][d] fp32; h0, dh_last, dh0 :
 *  [b][d] fp32 or NULL (dh0 NULL: not computed). dx may equal dh (in place);
 *  no other output may alias an input. RECURRENT runs each channel from
 *  t-1 down to 0; CHUNK (and AUTO from t = 64) walks the sequence in chunks
 *  from the end, composing chunk carries as (prod f, partial) pairs (same value
 *  up to rounding). No workspace. t may be 0 (dh0 = dh_last).
 *  Errors: INVALID_ARG.
 */
mmf_status mmf_hgrn_scan_bwd(const float *f, const float *h, const float *h0, const float *dh,
                             const float *dh_last, float *dx, float *df, float *dh0, int64_t b,
                             int64_t t, int64_t d, mmf_scan_mode mode, hipStream_t stream);

/*
 * mmf_hgrn2_scan_fwd -- the recurrence with an expanded state (HGRN2), fp32.
 * [R1] (section "核心价值提炼", table "创新之处" and list "关键设计决策") names
 * HGRN2 as the gated linear recurrence that replaces attention and prints only
 * the elementwise h_t = gate_t * h_{t-1} + x_t; the expanded state is a
 * reading: the d channels split into d/e heads of e channels, each head's state
 * is an e x e matrix S (row a, column c), the forget gate acts on its rows, the
 * input is the outer product of (1 - f) with i, and the output gate reads it:
 *   S_t[a][c] = f_t[a] * S_{t-1}[a][c] + (1 - f_t[a]) * i_t[c]
 *   y_t[c]    = sum_a o_t[a] * S_t[a][c]
 * (with e = 1 it is mmf_hgrn_scan_fwd with x = (1 - f) i, read out as o h).
 *  f, i, o, y : [b][t][d] fp32 (head n owns channels n*e .. n*e+e-1);
 *  s0, s_last : [b][d/e][e][e] fp32 or NULL (s0 NULL: zeros; s_last NULL: not
 *  written). s_last may equal s0 (in place: a decode step is t = 1); y and
 *  s_last may not alias anything else. No workspace. t may be 0 (s_last = s0).
 *  RECURRENT runs the tokens in order, each state block held in registers, so
 *  a call over t tokens and t calls of one token give the same bits. CHUNK
 *  (heads of 64 or 128) takes 16 tokens at a time: with every decay a product
 *  of gates, Y = Q~ S0 + A V and S1 = diag(prod f) S0 + K^T V, where
 *  Q~[t][a] = o_t[a] prod_{r<=t} f_r[a], K^[s][a] = (1 - f_s[a]) prod_{r>s} f_r[a]
 *  and A[t][s] = sum_a o_t[a] (1 - f_s[a]) prod_{s<r<=t} f_r[a] (s <= t): the
 *  same value up to rounding. CHUNK needs (t + 32) * d * 4 < 2^31 (a sequence's
 *  rows are addressed with 32-bit byte offsets). AUTO takes CHUNK from 16
 *  tokens on where it can (RECURRENT below, the one-token step included).
 *  e in {16, 32, 64, 128}, d a multiple of e; every tensor 16-byte aligned.
 *  Errors: INVALID_ARG, UNSUPPORTED (e; CHUNK with e < 64 or a sequence too
 *  long for it), HIP.
 */
mmf_status mmf_hgrn2_scan_fwd(const float *f, const float *i, const float *o, const float *s0, float *y,
                              float *s_last, int64_t b, int64_t t, int64_t d, int64_t e, mmf_scan_mode mode,
                              hipStream_t stream);

/*
 * mmf_layer_fwd -- one HGRNBit block over b sequences of t tokens ([R3]):
 *   i^, f^, g^ = BitLinear_{i,f,g}(x)
 *   f  = sigmoid(f^);  x~ = (1 - f) * SiLU(i^)
 *   h_t = f_t * h_{t-1} + x~_t                      (fp32 state; h_{-1} = h0 or 0)
 *   u  = RMSNorm(h) * g_norm_w * SiLU(g^)           ([R1] RMSNorm + Swish gate)
 *   x1 = x + BitLinear_o(u)
 *   [a | b] = BitLinear_gate(x1);  z = SiLU(a) * b
 *   out = x1 + BitLinear_down(z)
 *  x, out : [b][t][d] in dtype act (fp32 or bf16); everything inside is fp32
 *  (quantised codes int8, contractions exact int32), including the stored
 *  g_proj output and the MLP product z.
 *  h0 : [b][d] fp32 or NULL; h_last : [b][d] fp32 output or NULL.
 *  probe : NULL or stage outputs (above).
 *  Errors: INVALID_ARG (shapes inconsistent with d/inner, null weights),
 *  UNSUPPORTED (d or inner % 16), WORKSPACE.
 */
mmf_status mmf_layer_workspace_size(const mmf_layer_weights *w, int64_t b, int64_t t, size_t *bytes);
mmf_status mmf_layer_fwd(const mmf_layer_weights *w, const void *x, void *out, mmf_dtype act,
                         int64_t b, int64_t t, const float *h0, float *h_last, mmf_scan_mode mode,
                         void *ws, size_t ws_bytes, const mmf_layer_probe *probe, hipStream_t stream);

/*
 * mmf_layer_decode_step -- the same block for one new token per sequence,
 * with the recurrent state carried by the caller ([R1] step-wise recurrence):
 *  x, out : [b][d] in dtype act.  h : [b][d] fp32, read as h_{t-1} and
 *  overwritten with h_t.  Equivalent to mmf_layer_fwd with t = 1, h0 = h.
 *  Errors as mmf_layer_fwd (workspace from mmf_layer_workspace_size(w, b, 1)).
 *  Two implementations give the same bits: separate kernels per stage
 *  (quantisers and contractions: eight launches), and contractions that
 *  quantise their own input rows in every workgroup where a row fits (b <= 16,
 *  i/f/g sharing one gain or none; one row up to 8192 wide, where o_proj also
 *  forms the gated g_norm of h and g; 2 to 16 rows up to 2048 wide, 12 for a
 *  stage with a gain; the other stages keep their quantisers: four launches
 *  at one row, six at the 1.3B shape and 16 rows without gains). A probe does
 *  not change which kernels run: the self-quantising contractions write the
 *  codes and scales of their input rows (and the gated g_norm its row) from
 *  their first workgroup.
 */
mmf_status mmf_layer_decode_step(const mmf_layer_weights *w, const void *x, void *out, mmf_dtype act,
                                 int64_t b, float *h, void *ws, size_t ws_bytes,
                                 const mmf_layer_probe *probe, hipStream_t stream);

/*
 * mmf_layer_decode_step_noalloc -- mmf_layer_decode_step for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and the same bits, with
 * the workspace taken from an 8 MiB array the library holds in device memory,
 * one per GPU, until the process ends. The call allocates nothing and calls no
 * allocating routine. The first call on a device looks up that device's array
 * (hipGetSymbolAddress) and should not be made while the stream is being
 * captured; later calls may be.
 *  Arguments as mmf_layer_decode_step, without ws / ws_bytes.
 *  Errors as mmf_layer_decode_step; WORKSPACE when mmf_layer_workspace_size(w,
 *  b, 1) exceeds 8 MiB (about b = 64 at d = 4096, inner = 11008; b = 128 at the
 *  1.3B shape).
 *  Every call on a GPU shares that GPU's array and leaves its last contents
 *  there (nothing in it needs to start at zero: every stage writes its part
 *  before reading it): calls that overlap on one GPU (on different streams, or
 *  from several threads without ordering) race and may return wrong results.
 */
mmf_status mmf_layer_decode_step_noalloc(const mmf_layer_weights *w, const void *x, void *out, mmf_dtype act,
                                         int64_t b, float *h, const mmf_layer_probe *probe, hipStream_t stream);

/*
 * mmf_set_decode_kernel -- which implementation mmf_layer_decode_step uses,
 * process-wide: 0 = the fastest measured on MI355X (default: the
 * self-quantising contractions where they apply, else the separate kernels;
 * at the 1.3B shape in a HIP graph 21 / 33 us per layer at batch 1 / 16,
 * against 29 / 33 for the separate kernels); 1 = always the separate kernels.
 * INVALID_ARG for other values.
 */
mmf_status mmf_set_decode_kernel(int mode);

/*
 * mmf_stack_decode_step -- one decode step (one new token per sequence)
 * through a whole stack of n_layers HGRNBit blocks in a single persistent
 * kernel ([R3] section "HGRNBitBlock 的結構": the blocks are stacked; [R1] list
 * "可复用的模式与技巧": the step-wise recurrence used for generation). Block l
 * takes block l-1's output (block 0 takes x) and updates its state h[l] in
 * place; the result is that of n_layers mmf_layer_decode_step calls chained
 * through buffers of the activation dtype, bit for bit.
 *  layers : [n_layers] host array; every block has the same d and inner, and
 *           i/f/g share one gain tensor (or none) in each block.
 *  x, out : [b][d] device, activation dtype act; they must not overlap.
 *  b      : 1..16. d and inner multiples of 256 whose 16 rows of codes fit
 *           in LDS (the 370M, 1.3B and 2.7B widths do); else UNSUPPORTED.
 *  The kernel is launched cooperatively with one workgroup per CU (the launch
 *  fails with MMF_ERR_HIP if they cannot all be resident); the phases of
 *  every block are separated by barriers across the grid, and each
 *  contraction's packed weights are loaded during the barrier before the
 *  quantiser that precedes it. Every barrier wait is bounded (about a
 *  second): a wait that expires aborts the launch, every workgroup writes NaN
 *  over `out` (the states h are then undefined) and the count read by
 *  mmf_stack_decode_expired grows. A cooperative launch cannot be captured
 *  into a HIP graph: on a stream that is being captured the call returns
 *  UNSUPPORTED and enqueues nothing.
 *  Workspace: mmf_stack_decode_workspace_size bytes, bound to the stack and
 *  its states by mmf_stack_decode_bind, which copies a table of the blocks'
 *  device pointers into it and SYNCHRONISES with `stream` (call it once,
 *  outside graph capture); every later mmf_stack_decode_step on that
 *  workspace must pass the same layers, n_layers and b. The workspace holds
 *  the step's intermediate values: calls that share it must not overlap.
 *  Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
mmf_status mmf_stack_decode_workspace_size(const mmf_layer_weights *layers, int32_t n_layers, int64_t b,
                                           size_t *bytes);
mmf_status mmf_stack_decode_bind(const mmf_layer_weights *layers, int32_t n_layers, int64_t b, float *const *h,
                                 void *ws, size_t ws_bytes, hipStream_t stream);
mmf_status mmf_stack_decode_step(const mmf_layer_weights *layers, int32_t n_layers, const void *x, void *out,
                                 mmf_dtype act, int64_t b, void *ws, size_t ws_bytes, hipStream_t stream);
/* Barrier waits of mmf_stack_decode_step that expired since the library was
 * loaded, on the current device (synchronous; 0 in a healthy process). */
mmf_status mmf_stack_decode_expired(uint32_t *count);

/*
 * Measurement support (not part of the computation). While enabled on a
 * thread, every kernel launch made by the entry points above on that thread
 * is bracketed by two HIP events recorded on the call's stream, and one
 * record per launch is kept: the kernel variant, its shape and the event
 * pair. This is the only part of the library that allocates (HIP events,
 * created without the system-scope fence; host records), and it must stay
 * off while a stream is being captured into a HIP graph.
 *  mmf_timing_enable(1) clears earlier records; mmf_timing_enable(0) stops
 *  recording and keeps the records.
 *  mmf_timing_collect synchronises on the recorded events, copies up to
 *  `capacity` records into `out` (which may be NULL when capacity is 0) and
 *  returns the number recorded in *count.
 *  kernel : variant name, e.g. "tgemm_dma<gates>", "tgemv<resid>",
 *           "norm_quant<bf16>" (the quantiser's input type).
 *  m, n, k: rows, total output columns (all groups) and reduction length of a
 *  contraction; rows and row length of a quantiser; b*t, d of a scan.
 */
typedef struct {
    char kernel[40];
    int64_t m;
    int32_t n, k;
    float ms;
} mmf_kernel_timing;

mmf_status mmf_timing_enable(int on);
mmf_status mmf_timing_collect(mmf_kernel_timing *out, int32_t capacity, int32_t *count);

/*
 * mmf_hbm_ceiling -- measured HBM roof (measurement support): streams device
 * memory in the access pattern of the library's bandwidth-bound kernels
 * (16-byte loads by consecutive lanes, eight in flight per lane, each
 * workgroup of 256 threads streaming its own contiguous range; 8192
 * workgroups and cached loads for the read stream, 16384 and non-temporal
 * accesses for the others).
 *  mode 0 : read `bytes` of src (the packed-weight stream of a GEMV); dst
 *           receives one uint32 per workgroup (MMF_HBM_CEILING_SINK_BYTES).
 *  mode 1 : copy `bytes` from src to dst (one read and one write stream).
 *  mode 2 : dst = src[0:bytes) ^ src[bytes:2*bytes) (two read streams and one
 *           write stream: the scan's pattern); src holds 2 * bytes.
 *  bytes % 16 == 0; src and dst 16-byte aligned and not overlapping.
 *  Timed like every other launch while mmf_timing_enable is on ("stream_read",
 *  "stream_copy", "stream_2r1w"). Errors: INVALID_ARG.
 */
#define MMF_HBM_CEILING_SINK_BYTES 32768
mmf_status mmf_hbm_ceiling(int mode, const void *src, void *dst, int64_t bytes, hipStream_t stream);

/*
 * mmf_mfma_ceiling -- measured int8 MFMA roof (measurement support): four
 * 256-thread workgroups per CU, every wave running `iters` rounds of four
 * independent v_mfma_i32_32x32x32_i8 on register operands (the instruction
 * the prefill contractions use), nothing else in the loop. *ops receives the
 * operations the launch performs (2 * 32^3 per MFMA); divided by the launch's
 * duration it is the int8 rate this GPU sustains, clock included, against
 * which a contraction's rate is read next to the published 5.0 POP/s.
 *  sink : device memory, one uint32 per workgroup (4 * CUs words; sink_bytes
 *         checked). Timed as "mfma_loop" while mmf_timing_enable is on.
 *  Errors: INVALID_ARG, HIP.
 */
mmf_status mmf_mfma_ceiling(int64_t iters, void *sink, int64_t sink_bytes, int64_t *ops, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MMF_H */
