// gla_fwd.hip -- host side of the GLA forward: launch planning (segments, LDS layout), the
// cross-segment state scan (pass B), and dispatch to the chunk kernels compiled per element
// type in gla_fwd_bf16.hip / gla_fwd_f32.hip (kernel in gla_fwd_kernel.h).
//
// The sequence is cut into segments of `sc` chunks, one workgroup per (image, head,
// segment).  A segment's incoming state comes either
//   - from recomputing the state over all earlier chunks inside the same workgroup
//     (short sequences: one launch), or
//   - from three passes: pass A (chunk kernel, OUT=false) carries each segment's local
//     state from zero and records it with the segment's log2 decay; pass B
//     (gla_state_scan) scans those per state element; pass C (OUT=true) emits outputs.
// Head dims are compiled in 16-wide tile classes (NDK x NDV tiles); smaller dims are padded
// with zeros inside LDS, which leaves every product unchanged.
#include <atomic>
#include <mutex>

#include "dig_device.h"
#include "dig_internal.h"

namespace dig {

static int rup(int x, int m) { return (x + m - 1) / m * m; }

bool gla_dim_class(int dk, int dv, int* ndk, int* ndv) {
  static const int cls[][2] = {{1, 2}, {2, 4}, {3, 5}, {4, 8}};
  for (const auto& c : cls)
    if (dk <= 16 * c[0] && dv <= 16 * c[1]) {
      *ndk = c[0];
      *ndv = c[1];
      return true;
    }
  return false;
}

// Compute units of the target GPU; the automatic segment length aims at one round of
// workgroups over them: two co-resident workgroups per unit for the forward's chunk kernels,
// one for the backward's (their registers allow no second workgroup).
constexpr long kComputeUnits = 256;
// Longest sequence (in chunks) whose backward runs as one launch with the look-back: every
// workgroup reads the contributions of all later chunks of its sequence.
constexpr int kLookbackMaxChunks = 8;

GlaShape gla_plan(int B, int L, int H, int dk, int dv, int C, int bf16, int seg_chunks,
                  bool bwd) {
  GlaShape s;
  s.B = B; s.L = L; s.H = H; s.dk = dk; s.dv = dv; s.C = C; s.bf16 = bf16;
  s.ndk = s.ndv = 0;
  s.lr = 0;
  gla_dim_class(dk, dv, &s.ndk, &s.ndv);
  s.NC = (L + C - 1) / C;
  int sc = seg_chunks;
  // a short sequence whose chunks all fit one round of workgroups: one chunk per workgroup,
  // the carried state through the look-back (a single launch); the forward's look-back
  // kernel exists for the exact head shapes
  const bool exact = (dk == 32 && dv == 64) || (dk == 36 && dv == 72) || (dk == 16 && dv == 32);
  const bool lb_ok = bwd || exact;
  if (lb_ok && sc <= 0 && s.NC >= 2 && s.NC <= kLookbackMaxChunks &&
      (long)B * H * s.NC <= kComputeUnits)
    sc = 1;
  if (sc <= 0) {
    // as many segments per sequence as fill that round; one segment when the (image, head)
    // units alone already do
    const long units = (long)B * H;
    const long target = kComputeUnits * (bwd ? 1 : 2);
    const long nseg = units >= target || units < 1 ? 1 : target / units;
    sc = (int)(((long)s.NC + nseg - 1) / nseg);
  }
  if (sc > s.NC) sc = s.NC;
  if (sc < 1) sc = 1;
  s.sc = sc;
  s.nseg = (s.NC + sc - 1) / sc;
  // Recomputing earlier chunks in-workgroup beats the extra launches of the three-pass
  // scheme only while the grid is at most one workgroup per compute unit (latency-bound)
  // and there are few segments; the backward's recompute (a full output-stage backward per
  // chunk) never pays off.
  s.lookback = lb_ok && s.sc == 1 && s.nseg >= 2 && s.nseg <= kLookbackMaxChunks &&
               (long)B * H * s.nseg <= kComputeUnits;
  s.prefix = !s.lookback && s.nseg <= 4 && (long)B * H * s.nseg <= 256;
  s.bprefix = s.nseg <= 1;
  return s;
}

size_t gla_states_bytes(const GlaShape& s) {
  return (size_t)s.B * s.H * s.NC * s.dk * s.dv * sizeof(float);
}
static size_t al256(size_t x) { return (x + 255) / 256 * 256; }
size_t gla_saved_obar_offset(const GlaShape& s) { return al256(gla_states_bytes(s)); }
size_t gla_saved_rstd_offset(const GlaShape& s) {
  const size_t ob = (size_t)s.B * s.H * s.NC * s.C * 16 * s.ndv * sizeof(float);
  return gla_saved_obar_offset(s) + al256(ob);
}
size_t gla_saved_bytes(const GlaShape& s) {
  return gla_saved_rstd_offset(s) + al256((size_t)s.B * s.H * s.NC * s.C * sizeof(float));
}
size_t gla_seglg_bytes(const GlaShape& s) {
  return (size_t)s.B * s.H * s.nseg * s.dk * sizeof(float);
}

// Exclusive scan over segments, in place: slot(p) <- state entering segment p.
// Forward direction: S(0) = 0, S(p+1) = 2^{lg(p)} S(p) + dS(p).
constexpr int kScanThreads = 256;
template <int NB>
__global__ __launch_bounds__(kScanThreads) void gla_state_scan(float* states,
                                                              const float* seg_lg, int BH,
                                                              int NC, int sc, int nseg, int dk,
                                                              int dv) {
  const long idx = (long)blockIdx.x * kScanThreads + threadIdx.x;
  const long per = (long)dk * dv;
  if (idx >= (long)BH * per) return;
  const long bh = idx / per, ce = idx - bh * per;
  const int c = (int)(ce / dv);
  float S = 0.f;
  float* base = states + bh * NC * per + ce;
  const float* lg = seg_lg + bh * nseg * dk + c;
  // each batch's loads are issued together (indices clamped; they read segments no store of
  // the batch before touches), then the recurrence runs through them in order; NB is sized to
  // the segment count (clamped loads past the last segment still cost instructions)
  for (int p0 = 0; p0 < nseg - 1; p0 += NB) {
    float d[NB], l[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int ps = min(p0 + i, nseg - 2);
      d[i] = base[(long)ps * sc * per];
      l[i] = lg[ps * dk];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (p0 + i < nseg - 1) {
        base[(long)(p0 + i) * sc * per] = S;
        S = exp2f(l[i]) * S + d[i];
      }
    }
  }
  base[(long)(nseg - 1) * sc * per] = S;
}

hipError_t launch_gla_state_scan(const GlaShape& s, float* states, const float* seg_lg,
                                 hipStream_t st) {
  const long BH = (long)s.B * s.H;
  const long nthreads = BH * s.dk * s.dv;
  const dim3 grid((unsigned)((nthreads + kScanThreads - 1) / kScanThreads));
  if (s.nseg - 1 <= 8)
    hipLaunchKernelGGL(gla_state_scan<8>, grid, dim3(kScanThreads), 0, st, states, seg_lg,
                       (int)BH, s.NC, s.sc, s.nseg, s.dk, s.dv);
  else
    hipLaunchKernelGGL(gla_state_scan<32>, grid, dim3(kScanThreads), 0, st, states, seg_lg,
                       (int)BH, s.NC, s.sc, s.nseg, s.dk, s.dv);
  return hipGetLastError();
}

// Chunk kernels, instantiated per element type in their own translation units.
template <typename T, bool LR>
hipError_t launch_gla_fwd_t(const GlaShape& s, GlaFwdParams p, hipStream_t st, int* lds_out);
extern template hipError_t launch_gla_fwd_t<bf16, false>(const GlaShape&, GlaFwdParams,
                                                         hipStream_t, int*);
extern template hipError_t launch_gla_fwd_t<float, false>(const GlaShape&, GlaFwdParams,
                                                          hipStream_t, int*);
extern template hipError_t launch_gla_fwd_t<bf16, true>(const GlaShape&, GlaFwdParams,
                                                        hipStream_t, int*);

// the kernels for the element type and key-gate form (the low-rank gate exists for bf16)
static hipError_t fwd_kernels(const GlaShape& s, GlaFwdParams p, hipStream_t st, int* lds_out) {
  if (s.lr)
    return s.bf16 ? launch_gla_fwd_t<bf16, true>(s, p, st, lds_out) : hipErrorInvalidValue;
  return s.bf16 ? launch_gla_fwd_t<bf16, false>(s, p, st, lds_out)
                : launch_gla_fwd_t<float, false>(s, p, st, lds_out);
}

int gla_fwd_lds_bytes(const GlaShape& s) {
  int bytes = 0;
  const hipError_t e = fwd_kernels(s, GlaFwdParams{}, nullptr, &bytes);
  return e == hipSuccess ? bytes : 0;
}

// Sticky look-back status: one word per GPU (every device holds its own copy of the variable,
// zero when the code object is loaded).  A look-back wait that gives up sets it; the host reads
// and clears it (dig_lookback_status).  Host code reaches each device's copy through the
// address hipGetSymbolAddress returns with that device current.
__device__ unsigned g_lb_status;
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_status_mu;
unsigned* g_status_ptr[kMaxDevices];
std::atomic<unsigned> g_lb_spins{kLbSpinLimit};
std::atomic<bool> g_lb_never{false};
}  // namespace

unsigned* lookback_status_word() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_status_mu);
  if (!g_status_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_lb_status)) != hipSuccess || !ptr) return nullptr;
    g_status_ptr[dev] = static_cast<unsigned*>(ptr);
  }
  return g_status_ptr[dev];
}

LookbackWait lookback_wait() { return {g_lb_spins.load(), g_lb_never.load()}; }
void set_lookback_wait(unsigned spins, bool never_match) {
  g_lb_spins.store(spins ? spins : kLbSpinLimit);
  g_lb_never.store(never_match);
}

hipError_t launch_gla_fwd(const GlaShape& s, GlaFwdParams p, hipStream_t st) {
  p.B = s.B; p.L = s.L; p.H = s.H; p.dk = s.dk; p.dv = s.dv;
  p.NC = s.NC; p.sc = s.sc; p.nseg = s.nseg;
  p.C = s.C; p.prefix = s.prefix;
  p.lb_tag = next_call_tag();
  const LookbackWait w = lookback_wait();
  p.lb_wait_tag = w.never_match ? ((p.lb_tag ^ 0x5A5A5A5Au) | 1u) : p.lb_tag;
  p.lb_spins = w.spins;
  if (s.lookback) {
    p.lb_status = lookback_status_word();
    if (!p.lb_status) return hipErrorInvalidSymbol;
  }
  return fwd_kernels(s, p, st, nullptr);
}

}  // namespace dig
