// dig_api.cpp -- the extern "C" entry points of libdig: argument validation on the host
// (before anything is enqueued), workspace carving, and dispatch to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/dig.h"
#include "dig_internal.h"

namespace {

thread_local char g_err[512] = "";

dig_status fail(dig_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dig_status ok() {
  g_err[0] = '\0';
  return DIG_OK;
}

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range rng(const char* name, const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{name, a, a + bytes};
}

bool overlap(const Range& a, const Range& b) {
  return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

// outputs must not overlap inputs nor each other
dig_status check_alias(const Range* in, int nin, const Range* out, int nout) {
  for (int i = 0; i < nout; ++i) {
    if (!out[i].lo) continue;
    for (int j = 0; j < nin; ++j)
      if (in[j].lo && overlap(out[i], in[j]))
        return fail(DIG_ERR_ALIAS, "output %s overlaps input %s", out[i].name, in[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (out[j].lo && overlap(out[i], out[j]))
        return fail(DIG_ERR_ALIAS, "output %s overlaps output %s", out[i].name, out[j].name);
  }
  return DIG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t a256(size_t x) { return (x + 255) / 256 * 256; }

constexpr int kLdsLimit = 160 * 1024;

// Validates the descriptor; fills the plan.  Returns DIG_OK or an error (message set).
enum Pass { kFwd, kBwd };

dig_status check_desc(const dig_gla_desc* d, dig::GlaShape* s, Pass pass, bool lowrank = false,
                      bool key_gate_kernels = true) {
  if (!d) return fail(DIG_ERR_NULL, "desc is NULL");
  if (d->batch < 0 || d->seq_len < 0)
    return fail(DIG_ERR_SHAPE, "batch (%d) and seq_len (%d) must be >= 0", d->batch, d->seq_len);
  if (d->heads < 1 || d->d_k < 1 || d->d_v < 1)
    return fail(DIG_ERR_SHAPE, "heads, d_k, d_v must be >= 1 (got %d, %d, %d)", d->heads, d->d_k,
                d->d_v);
  if (d->dtype != DIG_F32 && d->dtype != DIG_BF16)
    return fail(DIG_ERR_UNSUPPORTED, "dtype %d is not DIG_F32 or DIG_BF16", d->dtype);
  if (d->chunk != 16 && d->chunk != 32 && d->chunk != 64)
    return fail(DIG_ERR_UNSUPPORTED, "chunk %d is not 16, 32 or 64", d->chunk);
  if (!(d->tau > 0.f) || !std::isfinite(d->tau))
    return fail(DIG_ERR_SHAPE, "tau must be finite and > 0");
  if (!(d->norm_eps >= 0.f) || !std::isfinite(d->norm_eps))
    return fail(DIG_ERR_SHAPE, "norm_eps must be finite and >= 0");
  if (!std::isfinite(d->q_scale)) return fail(DIG_ERR_SHAPE, "q_scale must be finite");
  if (d->seg_chunks < 0) return fail(DIG_ERR_SHAPE, "seg_chunks must be >= 0");
  int ndk = 0, ndv = 0;
  if (!dig::gla_dim_class(d->d_k, d->d_v, &ndk, &ndv))
    return fail(DIG_ERR_UNSUPPORTED, "d_k (%d) must be <= 64 and d_v (%d) <= 128", d->d_k, d->d_v);
  const long long rows = (long long)d->batch * d->seq_len * d->heads;
  if (rows * (d->d_k > d->d_v ? d->d_k : d->d_v) > (1LL << 40))
    return fail(DIG_ERR_UNSUPPORTED, "tensor too large");
  if ((long long)d->batch * d->heads > (1LL << 30))
    return fail(DIG_ERR_UNSUPPORTED, "batch * heads too large");
  if (lowrank && d->dtype != DIG_BF16)
    return fail(DIG_ERR_UNSUPPORTED, "the low-rank gate needs DIG_BF16");
  *s = dig::gla_plan(d->batch, d->seq_len, d->heads, d->d_k, d->d_v, d->chunk,
                     d->dtype == DIG_BF16, d->seg_chunks, pass == kBwd);
  s->lr = lowrank ? 1 : 0;
  if (!key_gate_kernels) return DIG_OK;  // the caller checks its own kernels' limits
  const int lds = pass == kFwd ? dig::gla_fwd_lds_bytes(*s) : dig::gla_bwd_lds_bytes(*s);
  if (lds > kLdsLimit)
    return fail(DIG_ERR_UNSUPPORTED, "%s needs %d bytes of LDS for this shape (limit %d)",
                pass == kFwd ? "forward" : "backward", lds, kLdsLimit);
  return DIG_OK;
}

dig_status check_dev(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DIG_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool valid_scan(int32_t d) { return d >= DIG_SCAN_ROW && d <= DIG_SCAN_COL_REV; }

dig_status check_srem(int32_t batch, int32_t gh, int32_t gw, int32_t ch, int32_t dtype,
                      int32_t a, int32_t b) {
  if (batch < 0 || gh < 0 || gw < 0)
    return fail(DIG_ERR_SHAPE, "batch, grid_h, grid_w must be >= 0");
  if (ch < 1) return fail(DIG_ERR_SHAPE, "channels must be >= 1");
  if (dtype != DIG_F32 && dtype != DIG_BF16)
    return fail(DIG_ERR_UNSUPPORTED, "dtype %d is not DIG_F32 or DIG_BF16", dtype);
  if (!valid_scan(a) || !valid_scan(b)) return fail(DIG_ERR_SHAPE, "scan direction out of range");
  if ((long long)gh * gw > (1LL << 31)) return fail(DIG_ERR_UNSUPPORTED, "grid too large");
  if ((long long)batch * gh * gw * ch > (1LL << 40)) return fail(DIG_ERR_UNSUPPORTED, "too large");
  return DIG_OK;
}

}  // namespace

extern "C" {

const char* dig_status_str(dig_status s) {
  switch (s) {
    case DIG_OK: return "DIG_OK";
    case DIG_ERR_NULL: return "DIG_ERR_NULL";
    case DIG_ERR_SHAPE: return "DIG_ERR_SHAPE";
    case DIG_ERR_UNSUPPORTED: return "DIG_ERR_UNSUPPORTED";
    case DIG_ERR_WORKSPACE: return "DIG_ERR_WORKSPACE";
    case DIG_ERR_ALIAS: return "DIG_ERR_ALIAS";
    case DIG_ERR_DEVICE: return "DIG_ERR_DEVICE";
    case DIG_ERR_ALIGN: return "DIG_ERR_ALIGN";
  }
  return "DIG_ERR_UNKNOWN";
}

const char* dig_last_error(void) { return g_err; }

int32_t dig_abi_version(void) { return 105; }

dig_status dig_lookback_status(hipStream_t stream) {
  unsigned* word = dig::lookback_status_word();
  if (!word) return fail(DIG_ERR_DEVICE, "look-back status word unavailable on this device");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return check_dev(e, "dig_lookback_status: stream synchronize");
  unsigned v = 0;
  e = hipMemcpy(&v, word, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return check_dev(e, "dig_lookback_status: read");
  if (v == 0) return ok();
  const unsigned zero = 0;
  e = hipMemcpy(word, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return check_dev(e, "dig_lookback_status: clear");
  return fail(DIG_ERR_DEVICE,
              "a look-back wait gave up before the values it waited for arrived; the outputs "
              "of the affected calls hold NaN");
}

void dig_debug_lookback(uint32_t spins, int32_t never_match) {
  dig::set_lookback_wait(spins, never_match != 0);
}

size_t dig_gla_saved_bytes(const dig_gla_desc* d) {
  dig::GlaShape s;
  if (check_desc(d, &s, kFwd) != DIG_OK) return 0;
  return dig::gla_saved_bytes(s);
}

size_t dig_gla_fwd_workspace_bytes(const dig_gla_desc* d) {
  dig::GlaShape s;
  if (check_desc(d, &s, kFwd) != DIG_OK) return 0;
  const size_t flags =  // look-back flags: published, done
      s.lookback ? a256(2 * (size_t)s.B * s.H * s.nseg * sizeof(unsigned)) : 0;
  if (!s.lookback && (s.nseg == 1 || s.prefix)) return 0;  // no cross-segment exchange
  return a256(dig::gla_states_bytes(s)) + a256(dig::gla_seglg_bytes(s)) + flags;
}

size_t dig_gla_bwd_workspace_bytes(const dig_gla_desc* d) {
  dig::GlaShape s;
  if (check_desc(d, &s, kBwd) != DIG_OK) return 0;
  return dig::gla_bwd_workspace(s);
}

}  // extern "C"

namespace {

// The low-rank key gate's inputs (all null: the caller passes the logits themselves).
struct LowRank {
  const void* factor;   // [B*L][16] bf16
  const void* w;        // [H*d_k][16] bf16
  const float* bias;    // [H*d_k] fp32 or null
};

// Checks the low-rank gate's arguments and adds their byte ranges to `in` (at *nin).
dig_status check_lowrank(const dig_gla_desc* d, const LowRank* lr, int32_t rank, Range* in,
                         int* nin) {
  if (rank != dig::kGateRank)
    return fail(DIG_ERR_UNSUPPORTED, "gate_rank %d: only %d is built", rank, dig::kGateRank);
  if (!lr->factor || !lr->w) return fail(DIG_ERR_NULL, "gate_factor and gate_w are required");
  if (!aligned16(lr->factor)) return fail(DIG_ERR_ALIGN, "gate_factor must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(lr->w) | reinterpret_cast<uintptr_t>(lr->bias)) & 3u)
    return fail(DIG_ERR_ALIGN, "gate_w and gate_bias must be 4-byte aligned");
  const size_t cols = (size_t)d->heads * d->d_k;
  in[(*nin)++] = rng("gate_factor", lr->factor, (size_t)d->batch * d->seq_len * rank * 2);
  in[(*nin)++] = rng("gate_w", lr->w, cols * rank * 2);
  in[(*nin)++] = rng("gate_bias", lr->bias, lr->bias ? cols * 4 : 0);
  return DIG_OK;
}

dig_status gla_fwd_impl(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                        const void* gate_logit, const LowRank* lr, int32_t rank, const void* r,
                        const float* norm_w, void* y, void* o_pre_opt, void* saved_opt,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dig::GlaShape s;
  dig_status st = check_desc(d, &s, kFwd, lr != nullptr);
  if (st != DIG_OK) return st;
  if ((long long)d->batch * d->seq_len == 0) return ok();
  if (!q || !k || !v || (!lr && !gate_logit) || !r || !y)
    return fail(DIG_ERR_NULL, "q, k, v, the gate, r and y are required");
  const void* ptrs[] = {q, k, v, gate_logit, r, norm_w, y, o_pre_opt, saved_opt, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t need = dig_gla_fwd_workspace_bytes(d);
  if (need && (!workspace || workspace_bytes < need))
    return fail(DIG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const size_t elt = d->dtype == DIG_BF16 ? 2 : 4;
  const size_t rows = (size_t)d->batch * d->seq_len * d->heads;
  const size_t bk = rows * d->d_k * elt, bv = rows * d->d_v * elt;
  Range in[9] = {rng("q", q, bk), rng("k", k, bk), rng("v", v, bv),
                 rng("gate_logit", lr ? nullptr : gate_logit, lr ? 0 : bk), rng("r", r, bv),
                 rng("norm_w", norm_w, norm_w ? d->d_v * 4 : 0)};
  int nin = 6;
  if (lr && (st = check_lowrank(d, lr, rank, in, &nin)) != DIG_OK) return st;
  const Range out[] = {rng("y", y, bv), rng("o_pre", o_pre_opt, o_pre_opt ? bv : 0),
                       rng("saved", saved_opt, saved_opt ? dig::gla_saved_bytes(s) : 0),
                       rng("workspace", workspace, workspace ? need : 0)};
  st = check_alias(in, nin, out, 4);
  if (st != DIG_OK) return st;

  dig::GlaFwdParams p{};
  p.q = q; p.k = k; p.v = v; p.r = r; p.norm_w = norm_w;
  p.z = lr ? lr->factor : gate_logit;
  if (lr) { p.zw = lr->w; p.zb = lr->bias; }
  p.y = y; p.o_pre = o_pre_opt;
  char* ws = static_cast<char*>(workspace);
  p.states = saved_opt ? static_cast<float*>(saved_opt) : reinterpret_cast<float*>(ws);
  if (saved_opt) {
    p.obar = static_cast<char*>(saved_opt) + dig::gla_saved_obar_offset(s);
    p.rstd = reinterpret_cast<float*>(static_cast<char*>(saved_opt) + dig::gla_saved_rstd_offset(s));
  }
  p.seg_lg = reinterpret_cast<float*>(ws + a256(dig::gla_states_bytes(s)));
  if (s.lookback) {  // chunk contributions, decays and flags
    p.lb_u = reinterpret_cast<float*>(ws);
    p.lb_flag = reinterpret_cast<unsigned*>(ws + a256(dig::gla_states_bytes(s)) +
                                            a256(dig::gla_seglg_bytes(s)));
  }
  p.write_states = saved_opt != nullptr;
  p.g2scale = 1.4426950408889634f / d->tau;
  p.q_scale = d->q_scale;
  p.eps = d->norm_eps;
  return check_dev(dig::launch_gla_fwd(s, p, stream), "dig_gla_fwd launch");
}

dig_status gla_bwd_impl(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                        const void* gate_logit, const LowRank* lr, int32_t rank, const void* r,
                        const float* norm_w, const void* dy, const void* saved, void* dq,
                        void* dk, void* dv, void* d_gate_logit, void* dr, float* d_norm_w,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dig::GlaShape s;
  dig_status st = check_desc(d, &s, kBwd, lr != nullptr);
  if (st != DIG_OK) return st;
  if ((long long)d->batch * d->seq_len == 0) {
    // empty problem: the weight gradient is an empty sum
    if (d_norm_w) {
      if (!aligned16(d_norm_w)) return fail(DIG_ERR_ALIGN, "d_norm_w must be 16-byte aligned");
      return check_dev(dig::launch_fill_zero(d_norm_w, (size_t)d->d_v, stream), "dig_gla_bwd fill");
    }
    return ok();
  }
  if (!q || !k || !v || (!lr && !gate_logit) || !r || !dy || !saved || !dq || !dk || !dv ||
      !d_gate_logit || !dr)
    return fail(DIG_ERR_NULL, "q, k, v, the gate, r, dy, saved and all gradients are required");
  const void* ptrs[] = {q, k, v, gate_logit, r, norm_w, dy, saved, dq, dk, dv, d_gate_logit, dr,
                        d_norm_w, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t need = dig_gla_bwd_workspace_bytes(d);
  if (need && (!workspace || workspace_bytes < need))
    return fail(DIG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const size_t elt = d->dtype == DIG_BF16 ? 2 : 4;
  const size_t rows = (size_t)d->batch * d->seq_len * d->heads;
  const size_t bk = rows * d->d_k * elt, bv = rows * d->d_v * elt;
  Range in[11] = {rng("q", q, bk), rng("k", k, bk), rng("v", v, bv),
                  rng("gate_logit", lr ? nullptr : gate_logit, lr ? 0 : bk), rng("r", r, bv),
                  rng("norm_w", norm_w, norm_w ? d->d_v * 4 : 0), rng("dy", dy, bv),
                  rng("saved", saved, dig::gla_saved_bytes(s))};
  int nin = 8;
  if (lr && (st = check_lowrank(d, lr, rank, in, &nin)) != DIG_OK) return st;
  const Range out[] = {rng("dq", dq, bk), rng("dk", dk, bk), rng("dv", dv, bv),
                       rng("d_gate_logit", d_gate_logit, bk), rng("dr", dr, bv),
                       rng("d_norm_w", d_norm_w, d_norm_w ? d->d_v * 4 : 0),
                       rng("workspace", workspace, workspace ? need : 0)};
  st = check_alias(in, nin, out, 7);
  if (st != DIG_OK) return st;

  const size_t BH = (size_t)s.B * s.H;
  char* ws = static_cast<char*>(workspace);
  dig::GlaBwdParams p{};
  p.q = q; p.k = k; p.v = v; p.r = r; p.norm_w = norm_w; p.dy = dy;
  p.z = lr ? lr->factor : gate_logit;
  if (lr) { p.zw = lr->w; p.zb = lr->bias; }
  p.states = static_cast<const float*>(saved);
  p.obar = static_cast<const char*>(saved) + dig::gla_saved_obar_offset(s);
  p.rstd = reinterpret_cast<const float*>(static_cast<const char*>(saved) +
                                          dig::gla_saved_rstd_offset(s));
  p.dq = dq; p.dk_ = dk; p.dv_ = dv; p.dz = d_gate_logit; p.dr = dr; p.d_norm_w = d_norm_w;
  p.gstates = reinterpret_cast<float*>(ws);
  size_t off = a256(BH * s.nseg * s.dk * s.dv * sizeof(float));
  p.seg_lg = reinterpret_cast<float*>(ws + off);
  off += a256(BH * s.nseg * s.dk * sizeof(float));
  p.dgamma_part = reinterpret_cast<float*>(ws + off);
  off += a256(BH * s.nseg * s.dv * sizeof(float));
  if (dig::gla_bwd_reuse_bytes(s)) {  // pass A's dO for the final pass
    p.dofrag = ws + off;
    p.diagws = reinterpret_cast<float*>(ws + off + dig::gla_bwd_reuse_diag_offset(s));
  }
  if (s.lookback) p.lb_flag = reinterpret_cast<unsigned*>(ws + dig::gla_bwd_flag_offset(s));
  p.g2scale = 1.4426950408889634f / d->tau;
  p.inv_tau = 1.f / d->tau;
  p.q_scale = d->q_scale;
  p.eps = d->norm_eps;
  return check_dev(dig::launch_gla_bwd(s, p, stream), "dig_gla_bwd launch");
}

// The value-gate calls: the common descriptor checks, then bf16, chunk 64 and the head-dim
// classes their kernels are built for.
dig_status check_beta(const dig_gla_desc* d, dig::GlaShape* s, Pass pass) {
  dig_status st = check_desc(d, s, pass, false, false);
  if (st != DIG_OK) return st;
  if (d->dtype != DIG_BF16) return fail(DIG_ERR_UNSUPPORTED, "the value gate needs DIG_BF16");
  if (d->chunk != 64) return fail(DIG_ERR_UNSUPPORTED, "the value gate runs chunk 64 only");
  *s = dig::gla_plan(d->batch, d->seq_len, d->heads, d->d_k, d->d_v, 64, 1, 0, pass == kBwd);
  const int lds = dig::gla_beta_lds_bytes(*s, pass == kBwd);
  if (lds > kLdsLimit)
    return fail(DIG_ERR_UNSUPPORTED, "the value gate is built for d_k <= 48 and d_v <= 80 "
                "(head-dim classes 16/32, 32/64, 48/80); got %d/%d", d->d_k, d->d_v);
  return DIG_OK;
}

dig_status gla_fwd_beta_impl(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                             const void* z, const void* w, const void* r, const float* norm_w,
                             void* y, void* o_pre_opt, void* saved_opt, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  dig::GlaShape s;
  dig_status st = check_beta(d, &s, kFwd);
  if (st != DIG_OK) return st;
  if ((long long)d->batch * d->seq_len == 0) return ok();
  if (!q || !k || !v || !z || !w || !r || !y)
    return fail(DIG_ERR_NULL, "q, k, v, both gates, r and y are required");
  const void* ptrs[] = {q, k, v, z, w, r, norm_w, y, o_pre_opt, saved_opt, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t need = dig::gla_beta_fwd_workspace(s);
  if (!workspace || workspace_bytes < need)
    return fail(DIG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const size_t rows = (size_t)d->batch * d->seq_len * d->heads;
  const size_t bk = rows * d->d_k * 2, bv = rows * d->d_v * 2;
  const Range in[] = {rng("q", q, bk), rng("k", k, bk), rng("v", v, bv),
                      rng("gate_logit", z, bk), rng("value_gate_logit", w, bv), rng("r", r, bv),
                      rng("norm_w", norm_w, norm_w ? d->d_v * 4 : 0)};
  const Range out[] = {rng("y", y, bv), rng("o_pre", o_pre_opt, o_pre_opt ? bv : 0),
                       rng("saved", saved_opt, saved_opt ? dig::gla_beta_saved_bytes(s) : 0),
                       rng("workspace", workspace, need)};
  st = check_alias(in, 7, out, 4);
  if (st != DIG_OK) return st;
  dig::GlaBetaFwd f{};
  f.q = q; f.k = k; f.v = v; f.z = z; f.w = w; f.r = r; f.norm_w = norm_w;
  f.y = y; f.o_pre = o_pre_opt; f.saved = saved_opt; f.workspace = workspace;
  f.inv_tau = 1.f / d->tau; f.q_scale = d->q_scale; f.eps = d->norm_eps;
  return check_dev(dig::launch_gla_beta_fwd(s, f, stream), "dig_gla_fwd_beta launch");
}

dig_status gla_bwd_beta_impl(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                             const void* z, const void* w, const void* r, const float* norm_w,
                             const void* dy, const void* saved, void* dq, void* dk, void* dv,
                             void* dz, void* dw, void* dr, float* d_norm_w, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  dig::GlaShape s;
  dig_status st = check_beta(d, &s, kBwd);
  if (st != DIG_OK) return st;
  if ((long long)d->batch * d->seq_len == 0) {
    if (d_norm_w) {
      if (!aligned16(d_norm_w)) return fail(DIG_ERR_ALIGN, "d_norm_w must be 16-byte aligned");
      return check_dev(dig::launch_fill_zero(d_norm_w, (size_t)d->d_v, stream),
                       "dig_gla_bwd_beta fill");
    }
    return ok();
  }
  if (!q || !k || !v || !z || !w || !r || !dy || !saved || !dq || !dk || !dv || !dz || !dw || !dr)
    return fail(DIG_ERR_NULL, "q, k, v, both gates, r, dy, saved and all gradients are required");
  const void* ptrs[] = {q, k, v, z, w, r, norm_w, dy, saved, dq, dk, dv, dz, dw, dr, d_norm_w,
                        workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t need = dig::gla_beta_bwd_workspace(s);
  if (!workspace || workspace_bytes < need)
    return fail(DIG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const size_t rows = (size_t)d->batch * d->seq_len * d->heads;
  const size_t bk = rows * d->d_k * 2, bv = rows * d->d_v * 2;
  const Range in[] = {rng("q", q, bk), rng("k", k, bk), rng("v", v, bv),
                      rng("gate_logit", z, bk), rng("value_gate_logit", w, bv), rng("r", r, bv),
                      rng("norm_w", norm_w, norm_w ? d->d_v * 4 : 0), rng("dy", dy, bv),
                      rng("saved", saved, dig::gla_beta_saved_bytes(s))};
  const Range out[] = {rng("dq", dq, bk), rng("dk", dk, bk), rng("dv", dv, bv),
                       rng("d_gate_logit", dz, bk), rng("d_value_gate_logit", dw, bv),
                       rng("dr", dr, bv), rng("d_norm_w", d_norm_w, d_norm_w ? d->d_v * 4 : 0),
                       rng("workspace", workspace, need)};
  st = check_alias(in, 9, out, 8);
  if (st != DIG_OK) return st;
  dig::GlaBetaBwd f{};
  f.q = q; f.k = k; f.v = v; f.z = z; f.w = w; f.r = r; f.norm_w = norm_w; f.dy = dy;
  f.saved = saved; f.dq = dq; f.dk = dk; f.dv = dv; f.dz = dz; f.dw = dw; f.dr = dr;
  f.d_norm_w = d_norm_w; f.workspace = workspace;
  f.inv_tau = 1.f / d->tau; f.q_scale = d->q_scale; f.eps = d->norm_eps;
  return check_dev(dig::launch_gla_beta_bwd(s, f, stream), "dig_gla_bwd_beta launch");
}

}  // namespace

extern "C" {

size_t dig_gla_beta_saved_bytes(const dig_gla_desc* d) {
  dig::GlaShape s;
  if (check_beta(d, &s, kFwd) != DIG_OK) return 0;
  return dig::gla_beta_saved_bytes(s);
}

size_t dig_gla_beta_fwd_workspace_bytes(const dig_gla_desc* d) {
  dig::GlaShape s;
  if (check_beta(d, &s, kFwd) != DIG_OK) return 0;
  return dig::gla_beta_fwd_workspace(s);
}

size_t dig_gla_beta_bwd_workspace_bytes(const dig_gla_desc* d) {
  dig::GlaShape s;
  if (check_beta(d, &s, kBwd) != DIG_OK) return 0;
  return dig::gla_beta_bwd_workspace(s);
}

dig_status dig_gla_fwd_beta(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                            const void* gate_logit, const void* value_gate_logit, const void* r,
                            const float* norm_w, void* y, void* o_pre_opt, void* saved_opt,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return gla_fwd_beta_impl(d, q, k, v, gate_logit, value_gate_logit, r, norm_w, y, o_pre_opt,
                           saved_opt, workspace, workspace_bytes, stream);
}

dig_status dig_gla_bwd_beta(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                            const void* gate_logit, const void* value_gate_logit, const void* r,
                            const float* norm_w, const void* dy, const void* saved, void* dq,
                            void* dk, void* dv, void* d_gate_logit, void* d_value_gate_logit,
                            void* dr, float* d_norm_w, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return gla_bwd_beta_impl(d, q, k, v, gate_logit, value_gate_logit, r, norm_w, dy, saved, dq,
                           dk, dv, d_gate_logit, d_value_gate_logit, dr, d_norm_w, workspace,
                           workspace_bytes, stream);
}

dig_status dig_gla_fwd(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                       const void* gate_logit, const void* r, const float* norm_w, void* y,
                       void* o_pre_opt, void* saved_opt, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return gla_fwd_impl(d, q, k, v, gate_logit, nullptr, 0, r, norm_w, y, o_pre_opt, saved_opt,
                      workspace, workspace_bytes, stream);
}

dig_status dig_gla_fwd_lowrank(const dig_gla_desc* d, const void* q, const void* k,
                               const void* v, const void* gate_factor, const void* gate_w,
                               const float* gate_bias, int32_t gate_rank, const void* r,
                               const float* norm_w, void* y, void* o_pre_opt, void* saved_opt,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const LowRank lr{gate_factor, gate_w, gate_bias};
  return gla_fwd_impl(d, q, k, v, nullptr, &lr, gate_rank, r, norm_w, y, o_pre_opt, saved_opt,
                      workspace, workspace_bytes, stream);
}

dig_status dig_gla_bwd(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                       const void* gate_logit, const void* r, const float* norm_w,
                       const void* dy, const void* saved, void* dq, void* dk, void* dv,
                       void* d_gate_logit, void* dr, float* d_norm_w, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return gla_bwd_impl(d, q, k, v, gate_logit, nullptr, 0, r, norm_w, dy, saved, dq, dk, dv,
                      d_gate_logit, dr, d_norm_w, workspace, workspace_bytes, stream);
}

dig_status dig_gla_bwd_lowrank(const dig_gla_desc* d, const void* q, const void* k,
                               const void* v, const void* gate_factor, const void* gate_w,
                               const float* gate_bias, int32_t gate_rank, const void* r,
                               const float* norm_w, const void* dy, const void* saved, void* dq,
                               void* dk, void* dv, void* d_gate_logit, void* dr,
                               float* d_norm_w, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  const LowRank lr{gate_factor, gate_w, gate_bias};
  return gla_bwd_impl(d, q, k, v, nullptr, &lr, gate_rank, r, norm_w, dy, saved, dq, dk, dv,
                      d_gate_logit, dr, d_norm_w, workspace, workspace_bytes, stream);
}

dig_status dig_srem_reorient(int32_t batch, int32_t grid_h, int32_t grid_w, int32_t channels,
                             int32_t dtype, int32_t from, int32_t to, const void* x, void* y,
                             hipStream_t stream) {
  dig_status st = check_srem(batch, grid_h, grid_w, channels, dtype, from, to);
  if (st != DIG_OK) return st;
  const size_t L = (size_t)grid_h * grid_w;
  if (batch == 0 || L == 0) return ok();
  if (!x || !y) return fail(DIG_ERR_NULL, "x and y are required");
  if (!aligned16(x) || !aligned16(y)) return fail(DIG_ERR_ALIGN, "x, y must be 16-byte aligned");
  const size_t elt = dtype == DIG_BF16 ? 2 : 4;
  const size_t bytes = (size_t)batch * L * channels * elt;
  const Range in[] = {rng("x", x, bytes)};
  const Range out[] = {rng("y", y, bytes)};
  st = check_alias(in, 1, out, 1);
  if (st != DIG_OK) return st;
  return check_dev(dig::launch_reorient(batch, grid_h, grid_w, channels, (int)elt, from, to, x, y,
                                        stream),
                   "dig_srem_reorient launch");
}

dig_status dig_dwconv3x3(int32_t batch, int32_t grid_h, int32_t grid_w, int32_t channels,
                         int32_t dtype, int32_t layout, int32_t out_layout, const void* x,
                         const float* w, const float* bias, void* y, hipStream_t stream) {
  dig_status st = check_srem(batch, grid_h, grid_w, channels, dtype, layout, out_layout);
  if (st != DIG_OK) return st;
  const size_t L = (size_t)grid_h * grid_w;
  if (batch == 0 || L == 0) return ok();
  if (!x || !w || !y) return fail(DIG_ERR_NULL, "x, w and y are required");
  if (!aligned16(x) || !aligned16(y) || !aligned16(w) || (bias && !aligned16(bias)))
    return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t elt = dtype == DIG_BF16 ? 2 : 4;
  const size_t bytes = (size_t)batch * L * channels * elt;
  const Range in[] = {rng("x", x, bytes), rng("w", w, (size_t)channels * 36),
                      rng("bias", bias, bias ? (size_t)channels * 4 : 0)};
  const Range out[] = {rng("y", y, bytes)};
  st = check_alias(in, 3, out, 1);
  if (st != DIG_OK) return st;
  return check_dev(dig::launch_dwconv(batch, grid_h, grid_w, channels, dtype == DIG_BF16, layout,
                                      out_layout, x, w, bias, y, stream),
                   "dig_dwconv3x3 launch");
}

size_t dig_dwconv3x3_bwd_workspace_bytes(int32_t batch, int32_t grid_h, int32_t grid_w,
                                         int32_t channels) {
  if (batch < 0 || grid_h < 0 || grid_w < 0 || channels < 1) return 0;
  if ((long long)batch * grid_h * grid_w == 0) return 0;
  return dig::dwconv_bwd_workspace(batch, grid_h, grid_w, channels);
}

}  // extern "C"

namespace {
// Argument checks shared by the conv backward entry points (the workspace aside).  *empty is
// set for an empty problem, whose dw (and dbias) have then been zero-filled on the stream.
dig_status check_dwconv_bwd(int32_t batch, int32_t grid_h, int32_t grid_w, int32_t channels,
                            int32_t dtype, int32_t layout, int32_t out_layout, const void* x,
                            const float* w, const void* dy, void* dx, float* dw, float* dbias_opt,
                            hipStream_t stream, bool* empty) {
  *empty = false;
  dig_status st = check_srem(batch, grid_h, grid_w, channels, dtype, layout, out_layout);
  if (st != DIG_OK) return st;
  if (batch == 0 || (size_t)grid_h * grid_w == 0) {
    if (!dw) return fail(DIG_ERR_NULL, "dw is required");
    if (!aligned16(dw) || (dbias_opt && !aligned16(dbias_opt)))
      return fail(DIG_ERR_ALIGN, "dw, dbias must be 16-byte aligned");
    *empty = true;
    hipError_t e = dig::launch_fill_zero(dw, (size_t)channels * 9, stream);
    if (e == hipSuccess && dbias_opt) e = dig::launch_fill_zero(dbias_opt, (size_t)channels, stream);
    return check_dev(e, "dig_dwconv3x3_bwd fill");
  }
  if (!x || !w || !dy || !dx || !dw) return fail(DIG_ERR_NULL, "x, w, dy, dx and dw are required");
  const void* ptrs[] = {x, w, dy, dx, dw, dbias_opt};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  return DIG_OK;
}
}  // namespace

extern "C" {

dig_status dig_dwconv3x3_bwd(int32_t batch, int32_t grid_h, int32_t grid_w, int32_t channels,
                             int32_t dtype, int32_t layout, int32_t out_layout, const void* x,
                             const float* w, const void* dy, void* dx, float* dw,
                             float* dbias_opt, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  bool empty = false;
  dig_status st = check_dwconv_bwd(batch, grid_h, grid_w, channels, dtype, layout, out_layout, x,
                                   w, dy, dx, dw, dbias_opt, stream, &empty);
  if (st != DIG_OK || empty) return st;
  const size_t L = (size_t)grid_h * grid_w;
  if (workspace && !aligned16(workspace))
    return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t need = dig_dwconv3x3_bwd_workspace_bytes(batch, grid_h, grid_w, channels);
  if (need && (!workspace || workspace_bytes < need))
    return fail(DIG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const size_t elt = dtype == DIG_BF16 ? 2 : 4;
  const size_t bytes = (size_t)batch * L * channels * elt;
  const Range in[] = {rng("x", x, bytes), rng("w", w, (size_t)channels * 36), rng("dy", dy, bytes)};
  const Range out[] = {rng("dx", dx, bytes), rng("dw", dw, (size_t)channels * 36),
                       rng("dbias", dbias_opt, dbias_opt ? (size_t)channels * 4 : 0),
                       rng("workspace", workspace, workspace ? need : 0)};
  st = check_alias(in, 3, out, 4);
  if (st != DIG_OK) return st;
  return check_dev(dig::launch_dwconv_bwd(batch, grid_h, grid_w, channels, dtype == DIG_BF16,
                                          layout, out_layout, x, w, dy, dx, dw, dbias_opt,
                                          workspace, stream),
                   "dig_dwconv3x3_bwd launch");
}

size_t dig_dwconv3x3_bwd_noalloc_max_bytes(void) { return dig::kNoAllocScratchBytes; }

}  // extern "C"

namespace {

// dig_linear's checks and launch; a workspace (the block's) lets one-output products split K.
dig_status linear_impl(int32_t m, int32_t k, int32_t dtype, const void* a, int32_t n_out,
                       const dig_linear_out* outs, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  if (dtype != DIG_BF16) return fail(DIG_ERR_UNSUPPORTED, "dig_linear runs on bf16 operands");
  if (m < 0 || k < 1) return fail(DIG_ERR_SHAPE, "m must be >= 0 and k >= 1");
  if (n_out < 1 || n_out > DIG_LINEAR_MAX_OUT)
    return fail(DIG_ERR_SHAPE, "n_out must be 1..%d", (int)DIG_LINEAR_MAX_OUT);
  if (!outs) return fail(DIG_ERR_NULL, "outs is required");
  if (k % 8) return fail(DIG_ERR_UNSUPPORTED, "k must be a multiple of 8 (16-byte rows)");
  if ((long long)(m + 255) / 256 > 65535) return fail(DIG_ERR_UNSUPPORTED, "m too large");
  for (int i = 0; i < n_out; ++i) {
    const dig_linear_out& o = outs[i];
    if (o.n < 1) return fail(DIG_ERR_SHAPE, "outs[%d].n must be >= 1", i);
    if (o.n % 8) return fail(DIG_ERR_UNSUPPORTED, "outs[%d].n must be a multiple of 8", i);
    if (o.act != DIG_ACT_NONE && o.act != DIG_ACT_GELU)
      return fail(DIG_ERR_SHAPE, "outs[%d].act must be DIG_ACT_NONE or DIG_ACT_GELU", i);
    if (o.res) {
      if (o.rows_per_gate < 1)
        return fail(DIG_ERR_SHAPE, "outs[%d].rows_per_gate must be >= 1", i);
      if (o.gate_ld < o.n) return fail(DIG_ERR_SHAPE, "outs[%d].gate_ld must be >= n", i);
      if (o.gate_ld % 8)
        return fail(DIG_ERR_UNSUPPORTED, "outs[%d].gate_ld must be a multiple of 8", i);
    }
  }
  if (m == 0) return ok();
  if (!a) return fail(DIG_ERR_NULL, "a is required");
  for (int i = 0; i < n_out; ++i) {
    if (!outs[i].c || !outs[i].w) return fail(DIG_ERR_NULL, "outs[%d].c and .w are required", i);
    if (outs[i].res && !outs[i].gate)
      return fail(DIG_ERR_NULL, "outs[%d].gate is required with a residual", i);
  }
  if (!aligned16(a)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  for (int i = 0; i < n_out; ++i) {
    const dig_linear_out& o = outs[i];
    const void* ptrs[] = {o.c, o.w, o.bias, o.res, o.gate};
    for (const void* q : ptrs)
      if (q && !aligned16(q)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  }
  Range in[1 + 4 * DIG_LINEAR_MAX_OUT], out[DIG_LINEAR_MAX_OUT];
  int nin = 0;
  in[nin++] = rng("a", a, (size_t)m * k * 2);
  for (int i = 0; i < n_out; ++i) {
    const dig_linear_out& o = outs[i];
    const size_t cbytes = (size_t)m * o.n * 2;
    in[nin++] = rng("w", o.w, (size_t)o.n * k * 2);
    in[nin++] = rng("bias", o.bias, o.bias ? (size_t)o.n * 4 : 0);
    if (o.res) {
      const size_t groups = ((size_t)m - 1) / (size_t)o.rows_per_gate;
      in[nin++] = rng("gate", o.gate, (groups * (size_t)o.gate_ld + o.n) * 2);
      // the residual may be this output itself, and otherwise may not touch it
      if (o.res != o.c) in[nin++] = rng("res", o.res, cbytes);
    }
    out[i] = rng("c", o.c, cbytes);
  }
  dig_status st = check_alias(in, nin, out, n_out);
  if (st != DIG_OK) return st;
  dig::LinearOut lo[DIG_LINEAR_MAX_OUT];
  for (int i = 0; i < n_out; ++i) {
    const dig_linear_out& o = outs[i];
    lo[i] = dig::LinearOut{o.c, o.w, o.bias, o.n, o.act, o.res, o.res ? o.gate : nullptr,
                           (long)o.gate_ld, o.res ? (int)std::min<int64_t>(o.rows_per_gate, m) : 1};
  }
  return check_dev(dig::launch_linear(m, k, a, n_out, lo, stream, ws, ws_bytes),
                   "dig_linear launch");
}

}  // namespace

extern "C" {

dig_status dig_linear(int32_t m, int32_t k, int32_t dtype, const void* a, int32_t n_out,
                      const dig_linear_out* outs, hipStream_t stream) {
  return linear_impl(m, k, dtype, a, n_out, outs, nullptr, 0, stream);
}

size_t dig_linear_workspace_bytes(int32_t m, int32_t k, int32_t n_out, const dig_linear_out* outs) {
  if (m < 1 || k < 1 || n_out != 1 || !outs || outs[0].n < 1) return 0;
  return dig::linear_splitk_bytes(m, k, outs[0].n);
}

dig_status dig_linear_ws(int32_t m, int32_t k, int32_t dtype, const void* a, int32_t n_out,
                         const dig_linear_out* outs, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  const size_t need = dig_linear_workspace_bytes(m, k, n_out, outs);
  if (need == 0) return linear_impl(m, k, dtype, a, n_out, outs, nullptr, 0, stream);
  if (!workspace || workspace_bytes < need)
    return fail(DIG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(DIG_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (outs && a) {  // the workspace may not overlap any argument
    const dig_linear_out& o = outs[0];
    const size_t cb = (size_t)m * o.n * 2;
    const Range in[] = {rng("a", a, (size_t)m * k * 2), rng("w", o.w, (size_t)o.n * k * 2),
                        rng("bias", o.bias, o.bias ? (size_t)o.n * 4 : 0),
                        rng("c", o.c, cb), rng("res", o.res, o.res ? cb : 0),
                        rng("gate", o.gate, o.gate ? 16 : 0)};
    const Range out[] = {rng("workspace", workspace, need)};
    dig_status st = check_alias(in, 6, out, 1);
    if (st != DIG_OK) return st;
  }
  return linear_impl(m, k, dtype, a, n_out, outs, workspace, workspace_bytes, stream);
}

dig_status dig_rmsnorm_modulate(int64_t rows, int32_t dim, int64_t rows_per_group, float eps,
                                const void* x, const void* scale, const void* shift,
                                int64_t mod_ld, void* h, hipStream_t stream) {
  if (rows < 0 || dim < 1 || rows_per_group < 1 || mod_ld < dim)
    return fail(DIG_ERR_SHAPE, "rows >= 0, dim >= 1, rows_per_group >= 1, mod_ld >= dim");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(DIG_ERR_SHAPE, "eps must be finite, >= 0");
  if (dim % 8 || dim > 2048 || mod_ld % 8)
    return fail(DIG_ERR_UNSUPPORTED, "dim and mod_ld must be multiples of 8, dim <= 2048");
  if (rows > (1LL << 32)) return fail(DIG_ERR_UNSUPPORTED, "too many rows");
  if (rows == 0) return ok();
  if (!x || !scale || !shift || !h) return fail(DIG_ERR_NULL, "x, scale, shift and h are required");
  const void* ptrs[] = {x, scale, shift, h};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t bytes = (size_t)rows * dim * 2;
  const size_t mbytes = ((size_t)(rows - 1) / rows_per_group * mod_ld + dim) * 2;
  const Range in[] = {rng("x", x, bytes), rng("scale", scale, mbytes), rng("shift", shift, mbytes)};
  const Range out[] = {rng("h", h, bytes)};
  dig_status st = check_alias(in, 3, out, 1);
  if (st != DIG_OK) return st;
  return check_dev(dig::launch_rmsnorm_modulate(rows, dim, rows_per_group, eps, x, scale, shift,
                                                mod_ld, h, stream),
                   "dig_rmsnorm_modulate launch");
}

size_t dig_block_cond_workspace_bytes(int32_t batch, int32_t dim) {
  if (batch < 0 || dim < 1) return 0;
  return a256((size_t)batch * dim * 2);
}

dig_status dig_block_cond(int32_t batch, int32_t dim, int32_t n_blocks, const void* c,
                          const void* w_ada, const float* b_ada, void* mod, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (batch < 0 || dim < 1 || n_blocks < 1)
    return fail(DIG_ERR_SHAPE, "batch >= 0, dim >= 1 and n_blocks >= 1 are required");
  if (dim % 8) return fail(DIG_ERR_UNSUPPORTED, "dim must be a multiple of 8");
  if ((long long)n_blocks * 6 * dim > (1LL << 30)) return fail(DIG_ERR_UNSUPPORTED, "too large");
  if (batch == 0) return ok();
  if (!c || !w_ada || !mod) return fail(DIG_ERR_NULL, "c, w_ada and mod are required");
  const size_t need = dig_block_cond_workspace_bytes(batch, dim);
  if (!workspace || workspace_bytes < need)
    return fail(DIG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const void* ptrs[] = {c, w_ada, b_ada, mod, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  const size_t nm = (size_t)n_blocks * 6 * dim;
  const Range in[] = {rng("c", c, (size_t)batch * dim * 2), rng("w_ada", w_ada, nm * dim * 2),
                      rng("b_ada", b_ada, b_ada ? nm * 4 : 0)};
  const Range out[] = {rng("mod", mod, (size_t)batch * nm * 2), rng("workspace", workspace, need)};
  dig_status st = check_alias(in, 3, out, 2);
  if (st != DIG_OK) return st;
  st = check_dev(dig::launch_silu((long)batch * dim, c, workspace, stream), "dig_block_cond silu");
  if (st != DIG_OK) return st;
  const dig_linear_out o{mod, w_ada, b_ada, (int32_t)nm, DIG_ACT_NONE, nullptr, nullptr, 0, 1};
  return dig_linear(batch, dim, DIG_BF16, workspace, 1, &o, stream);
}

namespace {

// Carving of dig_block_fwd's workspace (bf16 intermediates, then the GLA call's workspace).
struct BlockWs {
  size_t h, q, k, v, u, r, z, y, x1, hid, split, split_bytes, gla, total;
  bool fused;  // the gate logits are formed inside the mixer's kernels (rank 16)
};

dig_status block_plan(const dig_block_desc* d, dig_gla_desc* g, BlockWs* w) {
  if (!d) return fail(DIG_ERR_NULL, "desc is NULL");
  if (d->batch < 0 || d->grid_h < 0 || d->grid_w < 0)
    return fail(DIG_ERR_SHAPE, "batch, grid_h, grid_w must be >= 0");
  if (d->dim < 1 || d->heads < 1 || d->d_k < 1 || d->d_v < 1 || d->gate_rank < 1 || d->ffn_dim < 1)
    return fail(DIG_ERR_SHAPE, "dim, heads, d_k, d_v, gate_rank, ffn_dim must be >= 1");
  if (d->dim % 8 || d->dim > 2048 || (d->heads * d->d_k) % 8 || (d->heads * d->d_v) % 8 ||
      d->gate_rank % 8 || d->ffn_dim % 8)
    return fail(DIG_ERR_UNSUPPORTED,
                "dim (<= 2048), H*d_k, H*d_v, gate_rank and ffn_dim must be multiples of 8");
  if ((long long)d->grid_h * d->grid_w > (1LL << 31))
    return fail(DIG_ERR_UNSUPPORTED, "grid too large");
  *g = dig_gla_desc{};
  g->batch = d->batch;
  g->seq_len = d->grid_h * d->grid_w;
  g->heads = d->heads;
  g->d_k = d->d_k;
  g->d_v = d->d_v;
  g->chunk = d->chunk;
  g->tau = d->tau;
  g->q_scale = 1.f;
  g->norm_eps = d->norm_eps;
  g->dtype = DIG_BF16;
  g->seg_chunks = 0;
  dig::GlaShape s;
  dig_status st = check_desc(g, &s, kFwd);
  if (st != DIG_OK) return st;
  w->fused = d->gate_rank == dig::kGateRank && check_desc(g, &s, kFwd, true) == DIG_OK;
  const size_t M = (size_t)d->batch * g->seq_len;
  if (M > (size_t)65535 * 256) return fail(DIG_ERR_UNSUPPORTED, "too many tokens");
  const size_t HK = (size_t)d->heads * d->d_k, HV = (size_t)d->heads * d->d_v;
  size_t off = 0;
  auto take = [&](size_t cols) { const size_t o = off; off += a256(M * cols * 2); return o; };
  w->h = take(d->dim);
  w->q = take(HK);
  w->k = take(HK);
  w->v = take(HV);
  w->u = take(d->gate_rank);
  w->r = take(HV);
  w->z = w->fused ? 0 : take(HK);
  w->y = take(HV);
  w->x1 = take(d->dim);
  w->hid = take(d->ffn_dim);
  // fp32 partial sums of the one-output products whose grid would not fill the GPU
  const int m = (int)M;
  size_t sb = dig::linear_splitk_bytes(m, (int)HV, d->dim);
  sb = std::max(sb, dig::linear_splitk_bytes(m, d->dim, d->ffn_dim));
  sb = std::max(sb, dig::linear_splitk_bytes(m, d->ffn_dim, d->dim));
  w->split = off;
  w->split_bytes = sb;
  off += a256(sb);
  w->gla = off;
  off += a256(dig_gla_fwd_workspace_bytes(g));
  w->total = off;
  return DIG_OK;
}

}  // namespace

size_t dig_block_fwd_workspace_bytes(const dig_block_desc* desc) {
  dig_gla_desc g;
  BlockWs w;
  if (block_plan(desc, &g, &w) != DIG_OK) return 0;
  return w.total;
}

dig_status dig_block_fwd(const dig_block_desc* d, const dig_block_weights* wt, const void* mod,
                         int64_t mod_ld, int32_t layout, int32_t out_layout, const void* x,
                         void* x_out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  dig_gla_desc g;
  BlockWs w;
  dig_status st = block_plan(d, &g, &w);
  if (st != DIG_OK) return st;
  if (!valid_scan(layout) || !valid_scan(out_layout))
    return fail(DIG_ERR_SHAPE, "scan direction out of range");
  if (mod_ld < 6LL * d->dim || mod_ld % 8)
    return fail(DIG_ERR_SHAPE, "mod_ld must be >= 6 * dim and a multiple of 8");
  const size_t L = (size_t)d->grid_h * d->grid_w, M = (size_t)d->batch * L;
  if (M == 0) return ok();
  if (!wt) return fail(DIG_ERR_NULL, "weights are required");
  if (!x || !x_out || !mod || !wt->w_in || !wt->w_gate || !wt->w_out || !wt->w_ffn1 ||
      !wt->w_ffn2 || !wt->conv_w)
    return fail(DIG_ERR_NULL, "x, x_out, mod and every weight matrix are required");
  if (!workspace || workspace_bytes < w.total)
    return fail(DIG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", w.total,
                workspace ? workspace_bytes : (size_t)0);
  const int D = d->dim, HK = d->heads * d->d_k, HV = d->heads * d->d_v, R = d->gate_rank;
  const int F = d->ffn_dim, NIN = 2 * HK + 2 * HV + R;
  const void* ptrs[] = {x, x_out, mod, workspace, wt->w_in, wt->b_in, wt->w_gate, wt->b_gate,
                        wt->gla_norm_w, wt->w_out, wt->b_out, wt->w_ffn1, wt->b_ffn1, wt->w_ffn2,
                        wt->b_ffn2, wt->conv_w, wt->conv_b};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  // every bias / row slice handed to the projections must stay 16-byte aligned
  if ((HK % 8) || (HV % 8) || (R % 8))
    return fail(DIG_ERR_UNSUPPORTED, "H*d_k, H*d_v and gate_rank must be multiples of 8");
  const size_t xbytes = M * D * 2;
  const size_t mbytes = ((size_t)(d->batch - 1) * mod_ld + 6 * (size_t)D) * 2;
  const Range in[] = {
      rng("x", x, xbytes), rng("mod", mod, mbytes),
      rng("w_in", wt->w_in, (size_t)NIN * D * 2), rng("b_in", wt->b_in, wt->b_in ? NIN * 4 : 0),
      rng("w_gate", wt->w_gate, (size_t)HK * R * 2),
      rng("b_gate", wt->b_gate, wt->b_gate ? HK * 4 : 0),
      rng("gla_norm_w", wt->gla_norm_w, wt->gla_norm_w ? d->d_v * 4 : 0),
      rng("w_out", wt->w_out, (size_t)D * HV * 2), rng("b_out", wt->b_out, wt->b_out ? D * 4 : 0),
      rng("w_ffn1", wt->w_ffn1, (size_t)F * D * 2),
      rng("b_ffn1", wt->b_ffn1, wt->b_ffn1 ? F * 4 : 0),
      rng("w_ffn2", wt->w_ffn2, (size_t)D * F * 2),
      rng("b_ffn2", wt->b_ffn2, wt->b_ffn2 ? D * 4 : 0),
      rng("conv_w", wt->conv_w, (size_t)D * 36), rng("conv_b", wt->conv_b, wt->conv_b ? D * 4 : 0)};
  const Range out[] = {rng("x_out", x_out, xbytes), rng("workspace", workspace, w.total)};
  st = check_alias(in, 15, out, 2);
  if (st != DIG_OK) return st;

  char* ws = static_cast<char*>(workspace);
  void *h = ws + w.h, *q = ws + w.q, *k = ws + w.k, *v = ws + w.v, *u = ws + w.u, *r = ws + w.r;
  void *z = ws + w.z, *y = ws + w.y, *x1 = ws + w.x1, *hid = ws + w.hid;
  const char* md = static_cast<const char*>(mod);
  const int m = (int)M;
  const float* bi = wt->b_in;
  const char* wi = static_cast<const char*>(wt->w_in);
  auto mcol = [&](int part) { return md + (size_t)part * D * 2; };  // gamma_1 .. alpha_2
  // 1. h = RMSNorm(x) * gamma_1 + beta_1
  st = dig_rmsnorm_modulate((int64_t)M, D, (int64_t)L, d->norm_eps, x, mcol(0), mcol(1), mod_ld, h,
                            stream);
  if (st != DIG_OK) return st;
  // 2. [q | k | v | u | r] = h W_in^T + b_in, one launch
  {
    const int cols[5] = {HK, HK, HV, R, HV};
    void* dst[5] = {q, k, v, u, r};
    dig_linear_out o[5];
    size_t row0 = 0;
    for (int i = 0; i < 5; ++i) {
      o[i] = dig_linear_out{dst[i], wi + row0 * D * 2, bi ? bi + row0 : nullptr, cols[i],
                            DIG_ACT_NONE, nullptr, nullptr, 0, 1};
      row0 += cols[i];
    }
    st = dig_linear(m, D, DIG_BF16, h, 5, o, stream);
    if (st != DIG_OK) return st;
  }
  // 3. z = u W_gate^T + b_gate (rank 16: formed inside the mixer's kernels instead)
  if (!w.fused) {
    const dig_linear_out o{z, wt->w_gate, wt->b_gate, HK, DIG_ACT_NONE, nullptr, nullptr, 0, 1};
    st = dig_linear(m, R, DIG_BF16, u, 1, &o, stream);
    if (st != DIG_OK) return st;
  }
  // 4. the GLA token mixer, eqs. (5)-(10) up to the output projection
  if (w.fused)
    st = dig_gla_fwd_lowrank(&g, q, k, v, u, wt->w_gate, wt->b_gate, R, r, wt->gla_norm_w, y,
                             nullptr, nullptr, ws + w.gla, w.total - w.gla, stream);
  else
    st = dig_gla_fwd(&g, q, k, v, z, r, wt->gla_norm_w, y, nullptr, nullptr, ws + w.gla,
                     w.total - w.gla, stream);
  if (st != DIG_OK) return st;
  // 5. x1 = x + alpha_1 * (y W_out^T + b_out)
  {
    const dig_linear_out o{x1, wt->w_out, wt->b_out, D, DIG_ACT_NONE, x, mcol(2), mod_ld,
                           (int64_t)L};
    st = linear_impl(m, HV, DIG_BF16, y, 1, &o, ws + w.split, w.split_bytes, stream);
    if (st != DIG_OK) return st;
  }
  // 6. h = RMSNorm(x1) * gamma_2 + beta_2
  st = dig_rmsnorm_modulate((int64_t)M, D, (int64_t)L, d->norm_eps, x1, mcol(3), mcol(4), mod_ld,
                            h, stream);
  if (st != DIG_OK) return st;
  // 7. hid = GELU(h W_ffn1^T + b_ffn1)
  {
    const dig_linear_out o{hid, wt->w_ffn1, wt->b_ffn1, F, DIG_ACT_GELU, nullptr, nullptr, 0, 1};
    st = linear_impl(m, D, DIG_BF16, h, 1, &o, ws + w.split, w.split_bytes, stream);
    if (st != DIG_OK) return st;
  }
  // 8. x1 += alpha_2 * (hid W_ffn2^T + b_ffn2)   (in place)
  {
    const dig_linear_out o{x1, wt->w_ffn2, wt->b_ffn2, D, DIG_ACT_NONE, x1, mcol(5), mod_ld,
                           (int64_t)L};
    st = linear_impl(m, F, DIG_BF16, hid, 1, &o, ws + w.split, w.split_bytes, stream);
    if (st != DIG_OK) return st;
  }
  // 9. SREM: 3x3 depthwise conv on the current-order grid, written in the next scan order
  return dig_dwconv3x3(d->batch, d->grid_h, d->grid_w, D, DIG_BF16, layout, out_layout, x1,
                       wt->conv_w, wt->conv_b, x_out, stream);
}

dig_status dig_dwconv3x3_bwd_noalloc(int32_t batch, int32_t grid_h, int32_t grid_w,
                                     int32_t channels, int32_t dtype, int32_t layout,
                                     int32_t out_layout, const void* x, const float* w,
                                     const void* dy, void* dx, float* dw, float* dbias_opt,
                                     hipStream_t stream) {
  bool empty = false;
  dig_status st = check_dwconv_bwd(batch, grid_h, grid_w, channels, dtype, layout, out_layout, x,
                                   w, dy, dx, dw, dbias_opt, stream, &empty);
  if (st != DIG_OK || empty) return st;
  const size_t need = dig_dwconv3x3_bwd_workspace_bytes(batch, grid_h, grid_w, channels);
  if (need > dig::kNoAllocScratchBytes)
    return fail(DIG_ERR_WORKSPACE,
                "the partial sums need %zu bytes; the allocation-free call holds at most %zu "
                "(use dig_dwconv3x3_bwd with a workspace)",
                need, dig::kNoAllocScratchBytes);
  const size_t elt = dtype == DIG_BF16 ? 2 : 4;
  const size_t bytes = (size_t)batch * grid_h * grid_w * channels * elt;
  const Range in[] = {rng("x", x, bytes), rng("w", w, (size_t)channels * 36), rng("dy", dy, bytes)};
  const Range out[] = {rng("dx", dx, bytes), rng("dw", dw, (size_t)channels * 36),
                       rng("dbias", dbias_opt, dbias_opt ? (size_t)channels * 4 : 0)};
  st = check_alias(in, 3, out, 3);
  if (st != DIG_OK) return st;
  return check_dev(dig::launch_dwconv_bwd_noalloc(batch, grid_h, grid_w, channels,
                                                  dtype == DIG_BF16, layout, out_layout, x, w, dy,
                                                  dx, dw, dbias_opt, stream),
                   "dig_dwconv3x3_bwd_noalloc launch");
}

}  // extern "C"
