/*
 * dig.h -- C ABI of the DiG hot path on one AMD MI355X (gfx950):
 *   the gated-linear-attention (GLA) token mixer, forward and backward, and the SREM step
 *   (scan-direction reorient + 3x3 depthwise conv), forward and backward.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers on the current HIP device, 16-byte aligned,
 *     contiguous.  The caller owns every buffer; the library never allocates or frees
 *     device memory and keeps no device state between calls (its only state is a host-side
 *     call counter that tags the backward's look-back flags).
 *   - A workspace holds scratch only: it needs no initialisation and may be reused by later
 *     calls, but two calls that may run at the same time (other streams) must not share one.
 *   - Work is enqueued on `stream` and the call returns without synchronising.
 *   - Arguments are checked on the host before anything is enqueued.  A non-OK status
 *     means nothing was written; dig_last_error() gives a thread-local description.
 *     DIG_ERR_DEVICE means a launch failed; faults inside kernels surface at the
 *     caller's next synchronisation.  Nothing throws or aborts across the ABI.
 *   - Outputs may not overlap inputs (DIG_ERR_ALIAS): no in-place operation.
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

/* ------------------------------------------------------------------------ misc */

/* Static name of a status code. */
const char* dig_status_str(dig_status s);

/* Thread-local description of the last non-OK status returned on this thread ("" if none). */
const char* dig_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int32_t dig_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIG_H_ */
