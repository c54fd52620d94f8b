// dig_internal.h -- host-side parameter blocks and launchers shared by the C-ABI layer
// (dig_api.cpp) and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dig {

// Rank of the low-rank key gate formed inside the chunk kernels (x W_a1 has 16 columns).
constexpr int kGateRank = 16;

// ------------------------------------------------------------------ GLA forward
struct GlaShape {
  int B, L, H, dk, dv, C;   // C = chunk
  int bf16;                 // 1: bf16 I/O, 0: fp32 I/O
  int NC;                   // chunks per sequence = ceil(L / C)
  int sc;                   // chunks per segment
  int nseg;                 // segments per sequence = ceil(NC / sc)
  int prefix;               // forward: 1 = each segment recomputes its incoming state
  int bprefix;              // backward: the same choice (its recompute is costlier)
  int lookback;             // one chunk per workgroup, the carried state through a look-back
                            // over flags (forward: S0; backward: G), one launch
  int ndk, ndv;             // compiled head-dim class: d_k <= 16*ndk, d_v <= 16*ndv
  int lr;                   // 1: the key gate is the rank-16 product formed in the kernels
};

// Head-dim classes the kernels are compiled for (16-wide tiles of d_k and d_v).
bool gla_dim_class(int dk, int dv, int* ndk, int* ndv);

struct GlaFwdParams {
  int C, prefix;
  const void* q;
  const void* k;
  const void* v;
  const void* z;        // gate logits [B*L*H][dk], or (low-rank gate) the factor [B*L][16]
  const void* zw;       // low-rank gate: up-projection [H*dk][16] bf16, else null
  const float* zb;      // low-rank gate: bias [H*dk] fp32, or null
  const void* r;
  const float* norm_w;
  void* y;
  void* o_pre;
  float* states;   // [B*H][NC][dk][dv] fp32: state entering each chunk
  float* seg_lg;   // [B*H][nseg][dk] fp32: log2 of each segment's total decay (look-back:
                   // each chunk's decay factor)
  float* lb_u;     // look-back: [B*H][NC][dk][dv] each chunk's own state contribution
  unsigned* lb_flag;  // look-back: [2][B*H][NC] chunk published, chunk done (== lb_tag)
  unsigned lb_tag;    // this call's flag value
  unsigned lb_wait_tag;  // the value the waits look for (lb_tag; another only under test)
  unsigned lb_spins;     // bound on the polls of one wait
  unsigned* lb_status;   // sticky status word: set when a wait gives up
  void* obar;      // saved for the backward, or null: normalised o in fragment order
  float* rstd;     // saved for the backward, or null: [B*H][NC][C] RMSNorm reciprocal rms
  int B, L, H, dk, dv, NC, sc, nseg;
  float g2scale;   // log2(e) / tau
  float q_scale, eps;
  int write_states;
};

// Launch plan of one pass (bwd selects the backward's automatic segment length).
GlaShape gla_plan(int B, int L, int H, int dk, int dv, int C, int bf16, int seg_chunks, bool bwd);
// LDS bytes of the forward's output pass for this shape (0 if no kernel exists for it).
int gla_fwd_lds_bytes(const GlaShape& s);
size_t gla_states_bytes(const GlaShape& s);
// The forward->backward buffer: chunk states, then the normalised output ō of every token
// (fp32 whatever the I/O type: dO = rstd (dn - o rstd mean(dn . o rstd)) must stay orthogonal
// to o to fp32 precision, or dO . v at the first token, where o is parallel to v, loses its
// cancellation; [B*H][NC][C/16][NDV] 16 x 16 tiles in MFMA fragment order, NDV =
// ceil(d_v/16)), then the rows' rsqrt(mean o^2 + eps) (fp32 [B*H][NC][C]); offsets 256-aligned.
size_t gla_saved_bytes(const GlaShape& s);
size_t gla_saved_obar_offset(const GlaShape& s);
size_t gla_saved_rstd_offset(const GlaShape& s);
size_t gla_seglg_bytes(const GlaShape& s);

hipError_t launch_gla_fwd(const GlaShape& s, GlaFwdParams p, hipStream_t st);
// Pass B of the three-pass forward: exclusive scan of segment states.
hipError_t launch_gla_state_scan(const GlaShape& s, float* states, const float* seg_lg,
                                 hipStream_t st);

// ----------------------------------------------------------------- GLA backward
struct GlaBwdParams {
  int C, prefix;
  const void* q;
  const void* k;
  const void* v;
  const void* z;        // gate logits, or the low-rank gate's factor (as in GlaFwdParams)
  const void* zw;
  const float* zb;
  const void* r;
  const float* norm_w;
  const void* dy;
  const float* states;  // forward's chunk-entry states [B*H][NC][dk][dv]
  const void* obar;     // forward's normalised output, fragment order (see gla_saved_bytes)
  const float* rstd;    // forward's per-row rsqrt(mean o^2 + eps) [B*H][NC][C]
  void* dq;
  void* dk_;
  void* dv_;
  void* dz;
  void* dr;
  float* d_norm_w;
  float* gstates;       // [B*H][nseg][dk][dv] gradient entering each segment's end
  float* seg_lg;        // [B*H][nseg][dk]
  float* dgamma_part;   // [B*H*nseg][dv] per-workgroup partial sums
  void* dofrag;         // [B*H][NC] chunks of pass A's dO in fragment order (reuse), or null
  float* diagws;        // [B*H][NC][2][C] pass A's dO.v diagonals (reuse), or null
  unsigned* lb_flag;    // look-back: [2][B*H][nseg] segment published, segment done (== lb_tag)
  unsigned lb_tag;      // this call's flag value (differs from every earlier call's)
  unsigned lb_wait_tag; // the value the waits look for (lb_tag; another only under test)
  unsigned lb_spins;    // bound on the polls of one wait
  unsigned* lb_status;  // sticky status word: set when a wait gives up
  int B, L, H, dk, dv, NC, sc, nseg;
  float g2scale, inv_tau, q_scale, eps;
};

// LDS bytes of the backward's final pass for this shape (0 if no kernel exists for it).
int gla_bwd_lds_bytes(const GlaShape& s);
// Pass B of the three-pass backward: reverse scan of segment gradient states.
hipError_t launch_gla_gstate_scan(const GlaShape& s, const GlaBwdParams& p, hipStream_t st);
size_t gla_bwd_workspace(const GlaShape& s);
// Bytes of the final pass's reuse buffers (dO fragments, then diagonals), 0 when it recomputes.
size_t gla_bwd_reuse_bytes(const GlaShape& s);
size_t gla_bwd_reuse_diag_offset(const GlaShape& s);
// Offset of the look-back flags in the workspace ([B*H][nseg] unsigned).
size_t gla_bwd_flag_offset(const GlaShape& s);
// Look-back flag value for one call: differs from every earlier call's in this process.
unsigned next_call_tag();
// Look-back wait settings for the next launches: the bound on one wait's polls, and whether
// the waits look for a value no flag ever holds (a test of the expiry path).
struct LookbackWait {
  unsigned spins;
  bool never_match;
};
LookbackWait lookback_wait();
void set_lookback_wait(unsigned spins, bool never_match);
// The current device's sticky look-back status word (device address), or null on failure.
unsigned* lookback_status_word();
hipError_t launch_gla_bwd(const GlaShape& s, GlaBwdParams p, hipStream_t st);

// ------------------------------------------------------- GLA with the value-side gate
// The general gate of eq. (5), G_t = alpha_t^T beta_t (gla_beta.hip): bf16 I/O, chunk 64,
// head-dim classes (1,2), (2,4), (3,5).
struct GlaBetaFwd {
  const void* q;
  const void* k;
  const void* v;
  const void* z;  // key-gate logits [B, L, H, dk]
  const void* w;  // value-gate logits [B, L, H, dv]
  const void* r;
  const float* norm_w;
  void* y;
  void* o_pre;
  void* saved;      // gla_beta_saved_bytes, or null
  void* workspace;  // gla_beta_fwd_workspace
  float inv_tau, q_scale, eps;
};
struct GlaBetaBwd {
  const void* q;
  const void* k;
  const void* v;
  const void* z;
  const void* w;
  const void* r;
  const float* norm_w;
  const void* dy;
  const void* saved;
  void* dq;
  void* dk;
  void* dv;
  void* dz;
  void* dw;
  void* dr;
  float* d_norm_w;  // or null
  void* workspace;  // gla_beta_bwd_workspace
  float inv_tau, q_scale, eps;
};
// LDS bytes of the forward (bwd false) or backward output pass; above any limit when no kernel
// exists for the shape's head-dim class.
int gla_beta_lds_bytes(const GlaShape& s, bool bwd);
// saved: the fp32 state entering every 64-token chunk, then the fp32 pre-norm output of every
// token ([B*H][NC*64][dv]), each 256-byte aligned.
size_t gla_beta_saved_bytes(const GlaShape& s);
size_t gla_beta_fwd_workspace(const GlaShape& s);
size_t gla_beta_bwd_workspace(const GlaShape& s);
hipError_t launch_gla_beta_fwd(const GlaShape& s, const GlaBetaFwd& f, hipStream_t st);
hipError_t launch_gla_beta_bwd(const GlaShape& s, const GlaBetaBwd& f, hipStream_t st);

// ------------------------------------------------------------------- projections
constexpr int kLinearMaxOut = 6;
enum { kActNone = 0, kActGelu = 1 };
struct LinearOut {
  void* c;             // [M][n] bf16
  const void* w;       // [n][K] bf16 (out features x in features)
  const float* bias;   // [n] fp32 or null
  int n;
  int act;             // kActNone | kActGelu, applied to A W^T + bias
  const void* res;     // null, or R [M][n] bf16 (may be c): C = R + g * (A W^T + bias)
  const void* gate;    // g rows [M / rows_per_gate][gate_ld] bf16 (with res)
  long gate_ld;
  int rows_per_gate;
};
// C_o = epilogue_o(A W_o^T + bias_o) for every output o, A [M][K] bf16, one launch.  With a
// workspace of at least linear_splitk_bytes() (one output only), products whose grid of
// 128 x 128 tiles would not fill the GPU split K into fp32 partial sums there and finish in a
// second, reducing launch.
hipError_t launch_linear(int M, int K, const void* a, int nout, const LinearOut* outs,
                         hipStream_t st, void* ws = nullptr, size_t ws_bytes = 0);
size_t linear_splitk_bytes(int M, int K, int n);

// ------------------------------------------------------------------ DiG block
// h[r] = x[r] * rsqrt(mean(x[r]^2) + eps) * scale[r / rows_per_group] + shift[...], bf16 rows
// of D (a multiple of 8, at most 2048); scale and shift rows are mod_ld apart.
hipError_t launch_rmsnorm_modulate(long rows, int D, long rows_per_group, float eps,
                                   const void* x, const void* scale, const void* shift,
                                   long mod_ld, void* h, hipStream_t st);
// y = x * sigmoid(x), n bf16 elements.
hipError_t launch_silu(long n, const void* x, void* y, hipStream_t st);

// ------------------------------------------------------------------------- misc
// Zero n floats with a kernel (usable inside captured graphs, unlike a memset node).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st);

// ------------------------------------------------------------------------- SREM
hipError_t launch_reorient(int B, int gh, int gw, int D, int elt, int from, int to,
                           const void* x, void* y, hipStream_t st);
hipError_t launch_dwconv(int B, int gh, int gw, int D, int bf16, int layout, int out_layout,
                         const void* x, const float* w, const float* bias, void* y,
                         hipStream_t st);
size_t dwconv_bwd_workspace(int B, int gh, int gw, int D);
hipError_t launch_dwconv_bwd(int B, int gh, int gw, int D, int bf16, int layout, int out_layout,
                             const void* x, const float* w, const void* dy, void* dx, float* dw,
                             float* dbias, void* workspace, hipStream_t st);
// The same with the partials in the library's per-GPU scratch array (no allocation); fails
// with hipErrorInvalidValue if they need more than kNoAllocScratchBytes.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
hipError_t launch_dwconv_bwd_noalloc(int B, int gh, int gw, int D, int bf16, int layout,
                                     int out_layout, const void* x, const float* w, const void* dy,
                                     void* dx, float* dw, float* dbias, hipStream_t st);

}  // namespace dig
