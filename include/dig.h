/*
 * dig.h -- C ABI of the DiG hot path on one AMD MI355X (gfx950):
 *   the gated-linear-attention (GLA) token mixer, forward and backward, and the SREM step
 *   (scan-direction reorient + 3x3 depthwise conv), forward and backward.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers on the current HIP device, 16-byte aligned,
 *     contiguous.  The caller owns every buffer; the library never allocates or frees
 *     device memory.  Its state between calls: a host-side call counter that tags the
 *     look-back flags, and one device word per GPU (dig_lookback_status).
 *   - A workspace holds scratch only: it needs no initialisation and may be reused by later
 *     calls, but two calls that may run at the same time (other streams) must not share one.
 *   - Work is enqueued on `stream` and the call returns without synchronising.
 *   - Arguments are checked on the host before anything is enqueued.  A non-OK status
 *     means nothing was written; dig_last_error() gives a thread-local description.
 *     DIG_ERR_DEVICE means a launch failed; faults inside kernels surface at the
 *     caller's next synchronisation.  Nothing throws or aborts across the ABI.
 *   - Outputs may not overlap inputs (DIG_ERR_ALIAS): no in-place operation (one
 *     exception: dig_linear's residual may be its own output).
 *   - Empty problems (batch == 0 or seq_len == 0) return DIG_OK and touch nothing.
 *   - Element type of the activations is DIG_BF16 (bfloat16) or DIG_F32; arithmetic is
 *     fp32 throughout.  Norm weights, conv weights/bias and their gradients are fp32.
 *
 * Sources (the pages describing DiG):
 *   GLA: DiG study-group slides (docswell), slide "GLA の導入", eqs. (5)-(10); the DiG
 *        paper write-up (volcengine), section 2 "Linear Attention Transformer" (identity
 *        feature map, no normalizer) and section 3 "Preliminaries" (tau is a temperature).
 *   Chunkwise form: write-up section 3 "Efficiency Analysis" and the slides' efficiency
 *        slide: the sequence is cut into chunks of size M computed on-chip,
 *        O(TMD + TD^2) work.
 *   SREM: slides "SREM の導入" and write-up section 3 "DiG Block": reshape to 2-D,
 *        3x3 depthwise conv, transpose the token matrix and flip the flattened sequence to
 *        change the next block's scan direction.
 *   Block: slides Figure 4 (RMS Norm, Scale & Shift, Gated Linear Attention, Scale,
 *        RMS Norm, Scale & Shift, Feedforward, Scale, SREM; an MLP from the conditioning)
 *        and write-up section 3 "DiG Block" (adaptive normalisation regressed from the
 *        summed timestep and label embeddings).
 */
#ifndef DIG_H_
#define DIG_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIG_OK = 0,
  DIG_ERR_NULL = 1,        /* a required pointer is NULL */
  DIG_ERR_SHAPE = 2,       /* negative/zero sizes, L != grid_h*grid_w, bad tau/eps, bad enum */
  DIG_ERR_UNSUPPORTED = 3, /* valid but not implemented: d_k/d_v limits, chunk, dtype */
  DIG_ERR_WORKSPACE = 4,   /* workspace pointer NULL or smaller than the query says */
  DIG_ERR_ALIAS = 5,       /* an output overlaps an input or another output */
  DIG_ERR_DEVICE = 6,      /* a HIP call or kernel launch failed */
  DIG_ERR_ALIGN = 7        /* a tensor pointer is not 16-byte aligned */
} dig_status;

typedef enum { DIG_F32 = 0, DIG_BF16 = 1 } dig_dtype;

/*
 * Scan directions on a grid_h x grid_w token grid with canonical id c(i, j) = i*grid_w + j.
 * A sequence "in order d" holds at position p the token with canonical id pi_d(p):
 *   ROW:     pi(p) = p                          (row-major)
 *   ROW_REV: pi(p) = L-1-p                      (flipped)
 *   COL:     pi(p) = (p mod grid_h)*grid_w + p div grid_h   (transposed, column-major)
 *   COL_REV: pi(p) = pi_COL(L-1-p)              (transposed and flipped)
 * The four basic scan patterns of the write-up's introduction; a block flips after every
 * block and transposes after every second one, giving the period-4 schedule
 * ROW, ROW_REV, COL, COL_REV.
 */
typedef enum { DIG_SCAN_ROW = 0, DIG_SCAN_ROW_REV = 1, DIG_SCAN_COL = 2, DIG_SCAN_COL_REV = 3 } dig_scan;

/* ------------------------------------------------------------------ GLA token mixer */

typedef struct {
  int32_t batch;      /* B >= 0 */
  int32_t seq_len;    /* L >= 0 tokens per image, in the current scan order */
  int32_t heads;      /* H >= 1 */
  int32_t d_k;        /* key dim per head, 1..64 (true size; MFMA padding is internal) */
  int32_t d_v;        /* value dim per head, 1..128 */
  int32_t chunk;      /* 16, 32 or 64 tokens per chunk (the pages' M) */
  float tau;          /* gate temperature, > 0 (DiG uses 16) */
  float q_scale;      /* multiplies q (1 in DiG: eq. (8) applies no scale) */
  float norm_eps;     /* RMSNorm epsilon, >= 0 */
  int32_t dtype;      /* dig_dtype of q, k, v, gate_logit, r, y, o_pre, dy and gradients */
  int32_t seg_chunks; /* tuning: chunks per sequence segment (0 = automatic) */
} dig_gla_desc;

/*
 * Bytes of the forward->backward buffer `saved` (opaque to the caller; each region starts
 * 256-byte aligned): the fp32 state entering every chunk, [B][H][ceil(L/chunk)][d_k][d_v];
 * the normalised output o * rsqrt(mean o^2 + eps) of every token in fp32 (the backward's
 * RMSNorm gradient cancels against it), as 16 x 16 (token x value) tiles over d_v rounded up
 * to 16; the fp32 rsqrt(mean o^2 + eps) of every token.  0 for an invalid descriptor.
 */
size_t dig_gla_saved_bytes(const dig_gla_desc* desc);

/* Bytes of forward workspace (segment states and decays).  0 for an invalid descriptor. */
size_t dig_gla_fwd_workspace_bytes(const dig_gla_desc* desc);

/*
 * dig_gla_fwd -- GLA mixer forward (slides eqs. (5)-(10), without the projections):
 *   log(alpha_t) = logsigmoid(z_t) / tau                  (per key dim; alpha = sigmoid^(1/tau))
 *   S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,  S_{-1} = 0   (per image and head)
 *   o_t = (q_scale q_t) S_t
 *   y_t = o_t * rsqrt(mean_j o_tj^2 + eps) * norm_w * r_t * sigmoid(r_t)
 * computed chunkwise on bf16/fp32 matrix cores with fp32 accumulation.
 *   q, k, gate_logit : [B, L, H, d_k];  v, r : [B, L, H, d_v]   (token-major)
 *   norm_w           : [d_v] fp32, or NULL for ones (shared by all heads)
 *   y                : [B, L, H, d_v] output
 *   o_pre_opt        : [B, L, H, d_v] pre-norm o, or NULL
 *   saved_opt        : dig_gla_saved_bytes() bytes for dig_gla_bwd, or NULL
 *   workspace        : dig_gla_fwd_workspace_bytes() bytes (NULL allowed if that is 0)
 */
dig_status dig_gla_fwd(const dig_gla_desc* desc, const void* q, const void* k, const void* v,
                       const void* gate_logit, const void* r, const float* norm_w, void* y,
                       void* o_pre_opt, void* saved_opt, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* Bytes of backward workspace.  0 for an invalid descriptor. */
size_t dig_gla_bwd_workspace_bytes(const dig_gla_desc* desc);

/*
 * dig_gla_bwd -- gradients of <dy, y> for the forward above (chain rule through eqs.
 * (5)-(10)), given the `saved` buffer written by dig_gla_fwd with the same inputs:
 *   dq, dk, d_gate_logit : [B, L, H, d_k];  dv, dr : [B, L, H, d_v]   (overwritten)
 *   d_norm_w             : [d_v] fp32 sum over batch, tokens and heads (overwritten), or NULL
 * d_gate_logit = dlog(alpha) * sigmoid(-z) / tau.  The d_norm_w reduction runs in a fixed
 * order, so repeated calls give identical bits.  Sequences of 2..8 chunks whose chunks all
 * fit one round of workgroups (batch * heads * chunks <= 256) run as one launch in which
 * each chunk's workgroup reads the later chunks' gradient contributions through flags in
 * the workspace (bounded waits; the flags carry a per-call tag and every launch clears
 * them before it ends, so a call captured in a HIP graph may be replayed).  dig_gla_fwd
 * does the same for the state entering each chunk (exact head shapes 32/64, 36/72, 16/32).
 */
dig_status dig_gla_bwd(const dig_gla_desc* desc, const void* q, const void* k, const void* v,
                       const void* gate_logit, const void* r, const float* norm_w,
                       const void* dy, const void* saved, void* dq, void* dk, void* dv,
                       void* d_gate_logit, void* dr, float* d_norm_w, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * dig_gla_fwd_lowrank -- dig_gla_fwd with the key gate in its low-rank form (slides eq. (5):
 * the gate logits are (x W_a1) W_a2 + b_alpha) formed inside the chunk kernels instead of read:
 * for token t, head h and key column c
 *   z = gate_bias[h d_k + c] + sum_{r < 16} gate_factor[t][r] * gate_w[h d_k + c][r]
 * summed in fp32 from the bf16 products; the logits are never written to memory.
 *   gate_factor : [B, L, 16] bf16, x W_a1 per token (shared by every head), 16-byte aligned
 *   gate_w      : [H d_k][16] bf16, W_a2 as a linear layer's weight (out x in), 4-byte aligned
 *   gate_bias   : [H d_k] fp32 b_alpha, 4-byte aligned, or NULL for zeros
 *   gate_rank   : 16 (the only rank built: DIG_ERR_UNSUPPORTED otherwise)
 * desc->dtype must be DIG_BF16 (DIG_ERR_UNSUPPORTED otherwise).  Everything else, errors
 * included, as dig_gla_fwd; the gate inputs may not overlap the outputs.  `saved` feeds
 * dig_gla_bwd_lowrank with the same inputs.  Workspace and saved sizes: dig_gla_fwd's.
 */
dig_status dig_gla_fwd_lowrank(const dig_gla_desc* desc, const void* q, const void* k,
                               const void* v, const void* gate_factor, const void* gate_w,
                               const float* gate_bias, int32_t gate_rank, const void* r,
                               const float* norm_w, void* y, void* o_pre_opt, void* saved_opt,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dig_gla_bwd_lowrank -- dig_gla_bwd for dig_gla_fwd_lowrank (same gate inputs, the logits
 * formed again the same way).  d_gate_logit [B, L, H, d_k] is the gradient with respect to
 * those logits z; the gradients of gate_factor, gate_w and gate_bias are its products with
 * the up-projection's operands (a projection backward, not part of this call).  Workspace:
 * dig_gla_bwd_workspace_bytes().
 */
dig_status dig_gla_bwd_lowrank(const dig_gla_desc* desc, const void* q, const void* k,
                               const void* v, const void* gate_factor, const void* gate_w,
                               const float* gate_bias, int32_t gate_rank, const void* r,
                               const float* norm_w, const void* dy, const void* saved, void* dq,
                               void* dk, void* dv, void* d_gate_logit, void* dr,
                               float* d_norm_w, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * The general gate of eq. (5) (slides, slide "GLA の導入"): G_t = alpha_t^T beta_t, a key-side
 * gate alpha_t (d_k) times a value-side gate beta_t (d_v), both sigmoid(logit)^(1/tau):
 *   S_t = (alpha_t^T beta_t) (.) S_{t-1} + k_t^T v_t,  o_t = (q_scale q_t) S_t,
 * output stage as dig_gla_fwd.  DiG itself runs beta = 1 (dig_gla_fwd); these calls are the
 * variant with a value gate.  desc->dtype must be DIG_BF16, desc->chunk 64, d_k <= 48 and
 * d_v <= 80 with d_k <= 16, d_v <= 32 or d_k <= 32, d_v <= 64 or d_k <= 48, d_v <= 80
 * (DIG_ERR_UNSUPPORTED otherwise); desc->seg_chunks is ignored.  Any gate strength is
 * handled: inside a 16-token tile the products are factored about the row before the tile
 * only where both gates decay by at most 2^64 across it (factors within 2^-64..2^64), and
 * every pair takes its own factor <= 1 elsewhere.
 *
 * Bytes of the forward->backward buffer (opaque; regions 256-byte aligned): the fp32 state
 * entering every 64-token chunk, [B][H][ceil(L/64)][d_k][d_v], then the fp32 pre-norm
 * output of every token.  0 for a descriptor these calls reject.
 */
size_t dig_gla_beta_saved_bytes(const dig_gla_desc* desc);
/* Workspace bytes of dig_gla_fwd_beta (chunk states and decays) and dig_gla_bwd_beta
 * (gradient states, decays, norm-weight partials).  0 for a rejected descriptor. */
size_t dig_gla_beta_fwd_workspace_bytes(const dig_gla_desc* desc);
size_t dig_gla_beta_bwd_workspace_bytes(const dig_gla_desc* desc);

/*
 * dig_gla_fwd_beta -- forward with both gates.
 *   q, k, gate_logit : [B, L, H, d_k] bf16;  v, value_gate_logit, r : [B, L, H, d_v] bf16
 *   norm_w, y, o_pre_opt : as dig_gla_fwd
 *   saved_opt        : dig_gla_beta_saved_bytes() bytes for dig_gla_bwd_beta, or NULL
 *   workspace        : dig_gla_beta_fwd_workspace_bytes() bytes
 * Errors as dig_gla_fwd.
 */
dig_status dig_gla_fwd_beta(const dig_gla_desc* desc, const void* q, const void* k,
                            const void* v, const void* gate_logit, const void* value_gate_logit,
                            const void* r, const float* norm_w, void* y, void* o_pre_opt,
                            void* saved_opt, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * dig_gla_bwd_beta -- gradients of <dy, y> for dig_gla_fwd_beta, given its `saved`:
 *   dq, dk, d_gate_logit : [B, L, H, d_k];  dv, d_value_gate_logit, dr : [B, L, H, d_v]
 *   d_norm_w             : [d_v] fp32 (overwritten; fixed-order sum), or NULL
 * d_gate_logit = dlog(alpha) sigmoid(-z) / tau, d_value_gate_logit = dlog(beta) sigmoid(-w) /
 * tau.  Workspace: dig_gla_beta_bwd_workspace_bytes().  Errors as dig_gla_bwd.
 */
dig_status dig_gla_bwd_beta(const dig_gla_desc* desc, const void* q, const void* k,
                            const void* v, const void* gate_logit, const void* value_gate_logit,
                            const void* r, const float* norm_w, const void* dy,
                            const void* saved, void* dq, void* dk, void* dv, void* d_gate_logit,
                            void* d_value_gate_logit, void* dr, float* d_norm_w,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ projections */

/*
 * dig_linear -- the dense projections of a DiG block as one bf16 matrix-core launch: the
 * token mixer's inputs and output (slides eqs. (5), (9), (10): Q = X W_Q, K = X W_K,
 * V = X W_V, the low-rank gate logits (X W_a1) W_a2 + b_alpha, R = X W_r + b_r,
 * Y = (Swish(R) * Norm(O)) W_O) and the feedforward with the alpha-scaled residual adds
 * (slides Figure 4; write-up section 3 "DiG Block").  For every output o (up to
 * DIG_LINEAR_MAX_OUT sharing the input a):
 *   t[i][j] = sum_l a[i][l] * w[j][l] + bias[j]              fp32 accumulation
 *   t = GELU(t) = t * Phi(t)    if act == DIG_ACT_GELU (exact, erf form), then bf16
 *   c[i][j] = bf16(res[i][j] + gate[i / rows_per_gate][j] * t[i][j])   if res != NULL
 *   c[i][j] = t[i][j]                                                 otherwise
 * (bf16 values rounded to nearest even; the gated form rounds t to bf16 first).
 *   a          : [m][k] bf16, row-major (m rows, e.g. batch * tokens)
 *   w          : [n][k] bf16 (out features x in features, as a linear layer's weight)
 *   bias       : [n] fp32 or NULL
 *   c          : [m][n] bf16 output (contiguous: [B, L, H, d] for the mixer's operands)
 *   res        : NULL, or [m][n] bf16; may be c itself (in-place residual add)
 *   gate       : with res: rows of n bf16 gate values, row g at gate + g * gate_ld, one row
 *                per rows_per_gate consecutive rows of c (one per image); gate_ld >= n
 * dtype must be DIG_BF16; k, every n and gate_ld must be multiples of 8.  Outputs may not
 * overlap a, w, bias, gate, other outputs, or a res other than their own c (DIG_ERR_ALIAS).
 */
#define DIG_LINEAR_MAX_OUT 6
#define DIG_ACT_NONE 0
#define DIG_ACT_GELU 1
typedef struct {
  void* c;
  const void* w;
  const float* bias;
  int32_t n;
  int32_t act;
  const void* res;
  const void* gate;
  int64_t gate_ld;
  int64_t rows_per_gate;
} dig_linear_out;
dig_status dig_linear(int32_t m, int32_t k, int32_t dtype, const void* a, int32_t n_out,
                      const dig_linear_out* outs, hipStream_t stream);

/*
 * dig_linear_ws -- dig_linear with a workspace: a one-output product whose grid of 128 x 128
 * tiles would not fill the GPU splits K into fp32 partial sums in the workspace (up to eight
 * splits) and finishes them, with the same epilogue, in a second launch.  Same results up to
 * the order of the fp32 sums.  dig_linear_workspace_bytes() gives the bytes it uses (0: no
 * split for this shape; the call then runs exactly as dig_linear).  The workspace may not
 * overlap any argument.
 */
size_t dig_linear_workspace_bytes(int32_t m, int32_t k, int32_t n_out, const dig_linear_out* outs);
dig_status dig_linear_ws(int32_t m, int32_t k, int32_t dtype, const void* a, int32_t n_out,
                         const dig_linear_out* outs, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* ---------------------------------------------------------------------- DiG block */

/*
 * dig_rmsnorm_modulate -- the adaptive normalisation in front of a DiG block's GLA layer
 * and feedforward (slides Figure 4: RMS Norm, then Scale & Shift by gamma, beta regressed
 * from the conditioning; write-up section 3 "DiG Block"):
 *   h[i][:] = x[i][:] * rsqrt(mean_j x[i][j]^2 + eps) * scale[g][:] + shift[g][:],
 *   g = i / rows_per_group (the image of row i), scale/shift row g at scale + g * mod_ld.
 * x, h: [rows][dim] bf16; scale, shift: bf16 rows; dim and mod_ld multiples of 8,
 * dim <= 2048.  fp32 arithmetic, h rounded to bf16.  h may not overlap the inputs.
 */
dig_status dig_rmsnorm_modulate(int64_t rows, int32_t dim, int64_t rows_per_group, float eps,
                                const void* x, const void* scale, const void* shift,
                                int64_t mod_ld, void* h, hipStream_t stream);

/*
 * One DiG block's shapes (slides Figure 4 and Table 1; write-up section 3 "DiG Block" and
 * "Architecture Details").  The GLA layer's projections read the block's normalised input:
 *   [q | k | v | u | r] = h W_in^T + b_in     (q, k: H*d_k; v, r: H*d_v; u: gate_rank)
 *   z = u W_gate^T + b_gate                    (gate logits, H*d_k; b_gate is b_alpha)
 * and the feedforward is dim -> ffn_dim -> dim with GELU between.  With gate_rank 16 the
 * logits z are formed inside the mixer's kernels (dig_gla_fwd_lowrank: fp32, never stored);
 * with another rank a projection writes them (bf16) and dig_gla_fwd reads them.
 */
typedef struct {
  int32_t batch, grid_h, grid_w; /* tokens per image L = grid_h * grid_w */
  int32_t dim;                   /* hidden size D (multiple of 8, <= 2048) */
  int32_t heads, d_k, d_v;       /* the GLA layer: H * d_k, H * d_v multiples of 8 */
  int32_t gate_rank;             /* rank of the gate logits' factorisation (multiple of 8) */
  int32_t ffn_dim;               /* feedforward hidden width (multiple of 8) */
  int32_t chunk;                 /* GLA chunk: 16 | 32 | 64 */
  float tau;                     /* gate temperature */
  float norm_eps;                /* epsilon of the block's RMSNorms and the head-wise one */
} dig_block_desc;

/* One block's weights: bf16 matrices [out features][in features], fp32 vectors. */
typedef struct {
  const void* w_in;         /* [2 H d_k + 2 H d_v + gate_rank][dim]: rows q | k | v | u | r */
  const float* b_in;        /* the same rows, or NULL */
  const void* w_gate;       /* [H d_k][gate_rank] */
  const float* b_gate;      /* [H d_k] or NULL */
  const float* gla_norm_w;  /* [d_v] head-wise RMSNorm weight, or NULL (ones) */
  const void* w_out;        /* [dim][H d_v] */
  const float* b_out;       /* [dim] or NULL */
  const void* w_ffn1;       /* [ffn_dim][dim] */
  const float* b_ffn1;      /* [ffn_dim] or NULL */
  const void* w_ffn2;       /* [dim][ffn_dim] */
  const float* b_ffn2;      /* [dim] or NULL */
  const float* conv_w;      /* [dim][3][3] SREM depthwise conv */
  const float* conv_b;      /* [dim] or NULL */
} dig_block_weights;

/*
 * dig_block_cond -- the conditioning regression of a stack of n_blocks DiG blocks (slides
 * Figure 4: the MLP from the summed timestep and label embeddings to each block's
 * gamma, beta, alpha):
 *   mod[b][:] = SiLU(c[b][:]) W_ada^T + b_ada,   c: [batch][dim] bf16,
 *   W_ada: [n_blocks * 6 * dim][dim] bf16, b_ada: fp32 or NULL, mod: [batch][n_blocks*6*dim].
 * Block l's parameters are mod[b][6 dim l + ...] in the order
 *   gamma_1 | beta_1 | alpha_1 | gamma_2 | beta_2 | alpha_2   (dim each),
 * gamma used as the multiplier itself (h * gamma + beta).  workspace: batch * dim * 2 bytes
 * (dig_block_cond_workspace_bytes).
 */
size_t dig_block_cond_workspace_bytes(int32_t batch, int32_t dim);
dig_status dig_block_cond(int32_t batch, int32_t dim, int32_t n_blocks, const void* c,
                          const void* w_ada, const float* b_ada, void* mod, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * dig_block_fwd -- one DiG block forward (slides Figure 4; write-up section 3 "DiG Block"),
 * on x in scan order `layout`, writing the result in scan order `out_layout`:
 *   x1 = x  + alpha_1 * GLA(RMSNorm(x)  * gamma_1 + beta_1)        GLA: eqs. (5)-(10), W_O
 *   x2 = x1 + alpha_2 * FFN(RMSNorm(x1) * gamma_2 + beta_2)        FFN: W_ffn2 GELU(W_ffn1 .)
 *   x_out = DWConv3x3(x2) reoriented from `layout` to `out_layout` (SREM)
 * x, x_out: [batch][L][dim] bf16; mod: this block's 6*dim parameters of image 0 (see
 * dig_block_cond), image b's at mod + b * mod_ld.  The GLA layer runs dig_gla_fwd's kernels
 * with the same limits (d_k <= 64, d_v <= 128).  workspace: dig_block_fwd_workspace_bytes.
 * x_out may not overlap x, mod, the weights or the workspace.
 */
size_t dig_block_fwd_workspace_bytes(const dig_block_desc* desc);
dig_status dig_block_fwd(const dig_block_desc* desc, const dig_block_weights* wts,
                         const void* mod, int64_t mod_ld, int32_t layout, int32_t out_layout,
                         const void* x, void* x_out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* ------------------------------------------------------------------------- SREM */

/*
 * dig_srem_reorient -- exact gather of whole token rows from scan order `from` to `to`:
 *   y[b, p, :] = x[b, p_from(pi_to(p)), :]   (p_from = inverse of pi_from)
 * x, y: [batch, grid_h*grid_w, channels] of `dtype`.  Bit-exact copy.
 */
dig_status dig_srem_reorient(int32_t batch, int32_t grid_h, int32_t grid_w, int32_t channels,
                             int32_t dtype, int32_t from, int32_t to, const void* x, void* y,
                             hipStream_t stream);

/*
 * dig_dwconv3x3 -- SREM's 3x3 depthwise conv, zero padding 1, stride 1, on the
 * current-order sequence reshaped row-major to (grid_h, grid_w) for ROW/ROW_REV and to
 * (grid_w, grid_h) for COL/COL_REV, with the output written in scan order `out_layout`
 * (out_layout == layout: plain conv; otherwise conv fused with the reorient):
 *   y_conv[i*cols + j, c] = bias[c] + sum_{a,s=-1..1} w[c, a+1, s+1] x[(i+a)*cols + (j+s), c]
 *   y[b, p, :] = y_conv[b, p_layout(pi_out(p)), :]
 * x, y: [batch, L, channels] of `dtype`; w: [channels, 3, 3] fp32; bias: [channels] fp32 or NULL.
 */
dig_status dig_dwconv3x3(int32_t batch, int32_t grid_h, int32_t grid_w, int32_t channels,
                         int32_t dtype, int32_t layout, int32_t out_layout, const void* x,
                         const float* w, const float* bias, void* y, hipStream_t stream);

/* Bytes of workspace for dig_dwconv3x3_bwd (per-tile partial sums of dw, dbias). */
size_t dig_dwconv3x3_bwd_workspace_bytes(int32_t batch, int32_t grid_h, int32_t grid_w,
                                         int32_t channels);

/*
 * dig_dwconv3x3_bwd -- gradients of <dy, y> for dig_dwconv3x3 with the same layouts:
 *   dx [batch, L, channels] (`dtype`, overwritten), dw [channels, 3, 3] fp32 (overwritten),
 *   dbias_opt [channels] fp32 (overwritten) or NULL.  dw/dbias are reduced in a fixed
 *   order (deterministic).
 */
dig_status dig_dwconv3x3_bwd(int32_t batch, int32_t grid_h, int32_t grid_w, int32_t channels,
                             int32_t dtype, int32_t layout, int32_t out_layout, const void* x,
                             const float* w, const void* dy, void* dx, float* dw,
                             float* dbias_opt, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * dig_dwconv3x3_bwd_noalloc -- dig_dwconv3x3_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels and results.  The
 * dw/dbias partial sums go to a scratch array the library holds on each GPU for the life of
 * the process (dig_dwconv3x3_bwd_noalloc_max_bytes() bytes, 8 MiB).  Problems whose partials
 * need more (dig_dwconv3x3_bwd_workspace_bytes() larger than that) return DIG_ERR_WORKSPACE.
 * Nothing is allocated or freed.  Every call on one GPU shares that GPU's array: calls that
 * may overlap on one GPU (other streams, other threads) race and must be serialised.
 */
dig_status dig_dwconv3x3_bwd_noalloc(int32_t batch, int32_t grid_h, int32_t grid_w,
                                     int32_t channels, int32_t dtype, int32_t layout,
                                     int32_t out_layout, const void* x, const float* w,
                                     const void* dy, void* dx, float* dw, float* dbias_opt,
                                     hipStream_t stream);

/* Bytes of the per-GPU scratch array of dig_dwconv3x3_bwd_noalloc. */
size_t dig_dwconv3x3_bwd_noalloc_max_bytes(void);

/* ------------------------------------------------------------------------ misc */

/* Static name of a status code. */
const char* dig_status_str(dig_status s);

/* Thread-local description of the last non-OK status returned on this thread ("" if none). */
const char* dig_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int32_t dig_abi_version(void);

/*
 * dig_lookback_status -- status of the look-back waits on the current device.
 * Short sequences run dig_gla_fwd / dig_gla_bwd as one launch in which a chunk's workgroup
 * waits (bounded: about 2^18 polls, far past any real wait) for values published by the
 * workgroups of the other chunks of its sequence.  A wait that gives up leaves NaN in what the
 * missing values fed (y of that chunk; dq, dk, dv, d_gate_logit of that chunk; d_norm_w) and
 * sets a sticky status word of the device (a library-held device variable, one per GPU).
 * This call synchronises `stream`, then returns DIG_OK if no wait has given up since the last
 * call, else clears the word and returns DIG_ERR_DEVICE.  A wait can only give up when other
 * work keeps the earlier-dispatched workgroups from running for that long.
 */
dig_status dig_lookback_status(hipStream_t stream);

/*
 * dig_debug_lookback -- test hook for the path above: the launches that follow bound each
 * look-back wait by `spins` polls (0 restores the default) and, if never_match != 0, wait for a
 * flag value no workgroup ever raises, so every wait gives up (and every kernel still ends).
 * Process-wide; not for production use.
 */
void dig_debug_lookback(uint32_t spins, int32_t never_match);

#ifdef __cplusplus
}
#endif

#endif /* DIG_H_ */
