// gla_bwd.hip -- host side of the GLA backward: workspace layout, the reverse scan of
// segment gradient states, the fixed-order d_norm_w reduction, and dispatch to the chunk
// kernels compiled per element type in gla_bwd_bf16.hip / gla_bwd_f32.hip (kernel in
// gla_bwd_kernel.h).
//
// Gradients of <dy, y> through the forward in gla_fwd.hip (DiG study-group slides,
// eqs. (5)-(10), by the chain rule).  Per image and head, with do the gradient at the
// pre-norm output o, S_t the state after token t and dS_t the gradient flowing into S_t:
//   dq_t = S_t do_t,   dk_t = dS_t v_t,   dv_t = k_t dS_t,
//   dlog(alpha_u) = sum_{t >= u} (q_t.dq_t - k_t.dk_t)          (elementwise per key dim)
// Chunk form: b = in-chunk inclusive cumsum of log(alpha), S0 = state entering the chunk
// (saved by the forward), G = gradient reaching the chunk's end state from later chunks,
// D = dO V^T and P = gated Q K^T (both causal inside the chunk):
//   dq_i = e^{b_i} (do_i S0^T + sum_{j<=i} D_ij k_j e^{-b_j})
//   dk_j = e^{-b_j} sum_{i>=j} D_ij q_i e^{b_i} + e^{b_last-b_j} (G v_j)
//   dv_j = sum_{i>=j} P_ij do_i + (k_j e^{b_last-b_j}) G
//   dlog(alpha_u) = sum_{t>=u in chunk} (q.dq - k.dk)_t + sum_e (S_end (.) G)[:, e]
//   G_prev = diag(e^{b_last}) G + sum_i (q_i e^{b_i})^T do_i
// The last identity carries G backwards.  A segment's incoming G comes from one of:
//  - the look-back (short sequences, one chunk per workgroup, one launch): each workgroup
//    publishes its chunk's (q e^b)^T dO and decay and sums the later chunks' ones;
//  - one segment per sequence (the workgroup walks every chunk itself);
//  - pass A (per-segment local G from zero) + a reverse scan over segments + the final pass.
// The output-stage backward (head-wise RMSNorm x weight x Swish) starts from the normalised
// output o rstd and rstd that the forward saved.
#include <atomic>
#include <type_traits>

#include "dig_device.h"
#include "dig_internal.h"

namespace dig {

constexpr int kBThreads = 256;
size_t gla_bwd_workspace(const GlaShape& s) {
  const size_t BH = (size_t)s.B * s.H;
  size_t g = BH * s.nseg * s.dk * s.dv * sizeof(float);
  size_t lg = BH * s.nseg * s.dk * sizeof(float);
  size_t part = BH * s.nseg * s.dv * sizeof(float);
  auto a = [](size_t x) { return (x + 255) / 256 * 256; };
  return a(g) + a(lg) + a(part) + gla_bwd_reuse_bytes(s) +
         (s.lookback ? a(2 * BH * s.nseg * sizeof(unsigned)) : 0);  // published, done
}
size_t gla_bwd_flag_offset(const GlaShape& s) {
  const size_t BH = (size_t)s.B * s.H;
  auto a = [](size_t x) { return (x + 255) / 256 * 256; };
  return a(BH * s.nseg * s.dk * s.dv * sizeof(float)) + a(BH * s.nseg * s.dk * sizeof(float)) +
         a(BH * s.nseg * s.dv * sizeof(float)) + gla_bwd_reuse_bytes(s);
}

// Reverse exclusive scan over segments, in place: slot(p) <- gradient reaching the end of
// segment p from later segments.  G(nseg-1) = 0, G(p-1) = 2^{lg(p)} G(p) + dG(p).
template <int NB>
__device__ __forceinline__ void gstate_scan_one(float* gst, const float* seg_lg, long idx,
                                                int nseg, int dk, int dv) {
  const long per = (long)dk * dv;
  const long bh = idx / per, ce = idx - bh * per;
  const int c = (int)(ce / dv);
  float* base = gst + bh * nseg * per + ce;
  const float* lg = seg_lg + bh * nseg * dk + c;
  float G = 0.f;
  // each batch's loads are issued together (indices clamped; they read segments no store of
  // the batch before touches), then the recurrence runs through them in order; NB is sized to
  // the segment count (clamped loads past the first segment still cost instructions)
  for (int p0 = nseg - 1; p0 >= 1; p0 -= NB) {
    float d[NB], l[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int ps = max(p0 - i, 1);
      d[i] = base[(long)ps * per];
      l[i] = lg[ps * dk];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (p0 - i >= 1) {
        base[(long)(p0 - i) * per] = G;
        G = exp2f(l[i]) * G + d[i];
      }
    }
  }
  base[0] = G;
}

// out[e] = sum over parts of part[i][e] for the block's column e: a fixed-order tree (the
// same bits on every run).
__device__ __forceinline__ void dgamma_reduce_one(const float* part, int nparts, int dv, int e,
                                                  float* out) {
  __shared__ float red[kBThreads];
  const int tid = threadIdx.x;
  float s = 0.f;
  for (int i = tid; i < nparts; i += kBThreads) s += part[(long)i * dv + e];
  red[tid] = s;
  __syncthreads();
  for (int w = kBThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) out[e] = red[0];
}

// Pass B of the backward: blocks [0, nscan) scan the segment gradient states; the next dv
// blocks (when out is given) reduce the dgamma partials that pass A wrote.
template <int NB>
__global__ __launch_bounds__(kBThreads) void gla_gstate_scan(float* gst, const float* seg_lg,
                                                            int BH, int nseg, int dk, int dv,
                                                            int nscan, const float* part,
                                                            int nparts, float* out) {
  if ((int)blockIdx.x >= nscan) {
    dgamma_reduce_one(part, nparts, dv, (int)blockIdx.x - nscan, out);
    return;
  }
  const long idx = (long)blockIdx.x * kBThreads + threadIdx.x;
  if (idx < (long)BH * dk * dv) gstate_scan_one<NB>(gst, seg_lg, idx, nseg, dk, dv);
}

// dgamma alone (single-segment backward: the final pass wrote the partials).
__global__ __launch_bounds__(kBThreads) void gla_dgamma_reduce(const float* part, int nparts,
                                                              int dv, float* out) {
  dgamma_reduce_one(part, nparts, dv, (int)blockIdx.x, out);
}

hipError_t launch_gla_gstate_scan(const GlaShape& s, const GlaBwdParams& p, hipStream_t st) {
  const long BH = (long)s.B * s.H;
  const long nthreads = BH * s.dk * s.dv;
  const int nscan = (int)((nthreads + kBThreads - 1) / kBThreads);
  const int nred = p.d_norm_w ? s.dv : 0;
  if (s.nseg - 1 <= 8)
    hipLaunchKernelGGL(gla_gstate_scan<8>, dim3((unsigned)(nscan + nred)), dim3(kBThreads), 0,
                       st, p.gstates, p.seg_lg, (int)BH, s.nseg, s.dk, s.dv, nscan,
                       p.dgamma_part, (int)(BH * s.nseg), p.d_norm_w);
  else
    hipLaunchKernelGGL(gla_gstate_scan<32>, dim3((unsigned)(nscan + nred)), dim3(kBThreads), 0,
                       st, p.gstates, p.seg_lg, (int)BH, s.nseg, s.dk, s.dv, nscan,
                       p.dgamma_part, (int)(BH * s.nseg), p.d_norm_w);
  return hipGetLastError();
}

// Chunk kernels, instantiated per element type in their own translation units.
template <typename T, bool LR>
hipError_t launch_gla_bwd_t(const GlaShape& s, GlaBwdParams p, hipStream_t st, int* lds_out,
                            size_t* ru_out);
extern template hipError_t launch_gla_bwd_t<bf16, false>(const GlaShape&, GlaBwdParams,
                                                         hipStream_t, int*, size_t*);
extern template hipError_t launch_gla_bwd_t<float, false>(const GlaShape&, GlaBwdParams,
                                                          hipStream_t, int*, size_t*);
extern template hipError_t launch_gla_bwd_t<bf16, true>(const GlaShape&, GlaBwdParams,
                                                        hipStream_t, int*, size_t*);

// the kernels for the element type and key-gate form (the low-rank gate exists for bf16)
static hipError_t bwd_kernels(const GlaShape& s, GlaBwdParams p, hipStream_t st, int* lds_out,
                              size_t* ru_out) {
  if (s.lr)
    return s.bf16 ? launch_gla_bwd_t<bf16, true>(s, p, st, lds_out, ru_out)
                  : hipErrorInvalidValue;
  return s.bf16 ? launch_gla_bwd_t<bf16, false>(s, p, st, lds_out, ru_out)
                : launch_gla_bwd_t<float, false>(s, p, st, lds_out, ru_out);
}

int gla_bwd_lds_bytes(const GlaShape& s) {
  int bytes = 0;
  const hipError_t e = bwd_kernels(s, GlaBwdParams{}, nullptr, &bytes, nullptr);
  return e == hipSuccess ? bytes : 0;
}

static void reuse_sizes(const GlaShape& s, size_t (&b)[2]) {
  b[0] = b[1] = 0;
  const hipError_t e = bwd_kernels(s, GlaBwdParams{}, nullptr, nullptr, b);
  if (e != hipSuccess) b[0] = b[1] = 0;
}
static size_t a256(size_t x) { return (x + 255) / 256 * 256; }
size_t gla_bwd_reuse_bytes(const GlaShape& s) {
  size_t b[2];
  reuse_sizes(s, b);
  return b[0] ? a256(b[0]) + a256(b[1]) : 0;
}
size_t gla_bwd_reuse_diag_offset(const GlaShape& s) {
  size_t b[2];
  reuse_sizes(s, b);
  return a256(b[0]);
}

// Look-back flag values: a fresh one per call (a bijective hash of a call counter), so that
// flags left in a reused workspace by earlier calls never match.
unsigned next_call_tag() {
  static std::atomic<unsigned> calls{0};
  const unsigned t = (calls.fetch_add(1, std::memory_order_relaxed) + 1u) * 0x9E3779B1u;
  return t ? t : 1u;
}

hipError_t launch_gla_bwd(const GlaShape& s, GlaBwdParams p, hipStream_t st) {
  p.B = s.B; p.L = s.L; p.H = s.H; p.dk = s.dk; p.dv = s.dv;
  p.lb_tag = next_call_tag();
  const LookbackWait w = lookback_wait();
  p.lb_wait_tag = w.never_match ? ((p.lb_tag ^ 0x5A5A5A5Au) | 1u) : p.lb_tag;
  p.lb_spins = w.spins;
  if (s.lookback) {
    p.lb_status = lookback_status_word();
    if (!p.lb_status) return hipErrorInvalidSymbol;
  }
  p.NC = s.NC; p.sc = s.sc; p.nseg = s.nseg;
  p.C = s.C; p.prefix = s.bprefix;
  hipError_t e = bwd_kernels(s, p, st, nullptr, nullptr);
  if (e != hipSuccess) return e;
  if (p.d_norm_w && s.nseg == 1) {  // with more segments the scan launch reduces dgamma
    const long parts = (long)s.B * s.H * s.nseg;
    hipLaunchKernelGGL(gla_dgamma_reduce, dim3(s.dv), dim3(kBThreads), 0, st, p.dgamma_part,
                       (int)parts, s.dv, p.d_norm_w);
  }
  return hipGetLastError();
}

}  // namespace dig
