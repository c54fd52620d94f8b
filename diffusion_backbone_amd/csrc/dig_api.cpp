// dig_api.cpp -- the extern "C" entry points of libdig: argument validation on the host
// (before anything is enqueued), workspace carving, and dispatch to the gfx950 kernels.
#include <hip/hip_runtime.h>

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

dig_status check_desc(const dig_gla_desc* d, dig::GlaShape* s, Pass pass) {
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
  *s = dig::gla_plan(d->batch, d->seq_len, d->heads, d->d_k, d->d_v, d->chunk,
                     d->dtype == DIG_BF16, d->seg_chunks, pass == kBwd);
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

int32_t dig_abi_version(void) { return 100; }

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

dig_status dig_gla_fwd(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                       const void* gate_logit, const void* r, const float* norm_w, void* y,
                       void* o_pre_opt, void* saved_opt, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  dig::GlaShape s;
  dig_status st = check_desc(d, &s, kFwd);
  if (st != DIG_OK) return st;
  if ((long long)d->batch * d->seq_len == 0) return ok();
  if (!q || !k || !v || !gate_logit || !r || !y)
    return fail(DIG_ERR_NULL, "q, k, v, gate_logit, r and y are required");
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
  const size_t sb = dig::gla_states_bytes(s);
  const Range in[] = {rng("q", q, bk), rng("k", k, bk), rng("v", v, bv),
                      rng("gate_logit", gate_logit, bk), rng("r", r, bv),
                      rng("norm_w", norm_w, norm_w ? d->d_v * 4 : 0)};
  const Range out[] = {rng("y", y, bv), rng("o_pre", o_pre_opt, o_pre_opt ? bv : 0),
                       rng("saved", saved_opt, saved_opt ? dig::gla_saved_bytes(s) : 0),
                       rng("workspace", workspace, workspace ? need : 0)};
  st = check_alias(in, 6, out, 4);
  if (st != DIG_OK) return st;

  dig::GlaFwdParams p{};
  p.q = q; p.k = k; p.v = v; p.z = gate_logit; p.r = r; p.norm_w = norm_w;
  p.y = y; p.o_pre = o_pre_opt;
  char* ws = static_cast<char*>(workspace);
  p.states = saved_opt ? static_cast<float*>(saved_opt) : reinterpret_cast<float*>(ws);
  if (saved_opt) {
    p.obar = static_cast<char*>(saved_opt) + dig::gla_saved_obar_offset(s);
    p.rstd = reinterpret_cast<float*>(static_cast<char*>(saved_opt) + dig::gla_saved_rstd_offset(s));
  }
  p.seg_lg = reinterpret_cast<float*>(ws + a256(sb));
  if (s.lookback) {  // chunk contributions, decays and flags
    p.lb_u = reinterpret_cast<float*>(ws);
    p.lb_flag = reinterpret_cast<unsigned*>(ws + a256(sb) + a256(dig::gla_seglg_bytes(s)));
  }
  p.write_states = saved_opt != nullptr;
  p.g2scale = 1.4426950408889634f / d->tau;
  p.q_scale = d->q_scale;
  p.eps = d->norm_eps;
  return check_dev(dig::launch_gla_fwd(s, p, stream), "dig_gla_fwd launch");
}

dig_status dig_gla_bwd(const dig_gla_desc* d, const void* q, const void* k, const void* v,
                       const void* gate_logit, const void* r, const float* norm_w,
                       const void* dy, const void* saved, void* dq, void* dk, void* dv,
                       void* d_gate_logit, void* dr, float* d_norm_w, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  dig::GlaShape s;
  dig_status st = check_desc(d, &s, kBwd);
  if (st != DIG_OK) return st;
  if ((long long)d->batch * d->seq_len == 0) {
    // empty problem: the weight gradient is an empty sum
    if (d_norm_w) {
      if (!aligned16(d_norm_w)) return fail(DIG_ERR_ALIGN, "d_norm_w must be 16-byte aligned");
      return check_dev(dig::launch_fill_zero(d_norm_w, (size_t)d->d_v, stream), "dig_gla_bwd fill");
    }
    return ok();
  }
  if (!q || !k || !v || !gate_logit || !r || !dy || !saved || !dq || !dk || !dv ||
      !d_gate_logit || !dr)
    return fail(DIG_ERR_NULL, "q, k, v, gate_logit, r, dy, saved and all gradients are required");
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
  const Range in[] = {rng("q", q, bk), rng("k", k, bk), rng("v", v, bv),
                      rng("gate_logit", gate_logit, bk), rng("r", r, bv),
                      rng("norm_w", norm_w, norm_w ? d->d_v * 4 : 0), rng("dy", dy, bv),
                      rng("saved", saved, dig::gla_saved_bytes(s))};
  const Range out[] = {rng("dq", dq, bk), rng("dk", dk, bk), rng("dv", dv, bv),
                       rng("d_gate_logit", d_gate_logit, bk), rng("dr", dr, bv),
                       rng("d_norm_w", d_norm_w, d_norm_w ? d->d_v * 4 : 0),
                       rng("workspace", workspace, workspace ? need : 0)};
  st = check_alias(in, 8, out, 7);
  if (st != DIG_OK) return st;

  const size_t BH = (size_t)s.B * s.H;
  char* ws = static_cast<char*>(workspace);
  dig::GlaBwdParams p{};
  p.q = q; p.k = k; p.v = v; p.z = gate_logit; p.r = r; p.norm_w = norm_w; p.dy = dy;
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

dig_status dig_dwconv3x3_bwd(int32_t batch, int32_t grid_h, int32_t grid_w, int32_t channels,
                             int32_t dtype, int32_t layout, int32_t out_layout, const void* x,
                             const float* w, const void* dy, void* dx, float* dw,
                             float* dbias_opt, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  dig_status st = check_srem(batch, grid_h, grid_w, channels, dtype, layout, out_layout);
  if (st != DIG_OK) return st;
  const size_t L = (size_t)grid_h * grid_w;
  if (batch == 0 || L == 0) {
    if (!dw) return fail(DIG_ERR_NULL, "dw is required");
    if (!aligned16(dw) || (dbias_opt && !aligned16(dbias_opt)))
      return fail(DIG_ERR_ALIGN, "dw, dbias must be 16-byte aligned");
    hipError_t e = dig::launch_fill_zero(dw, (size_t)channels * 9, stream);
    if (e == hipSuccess && dbias_opt) e = dig::launch_fill_zero(dbias_opt, (size_t)channels, stream);
    return check_dev(e, "dig_dwconv3x3_bwd fill");
  }
  if (!x || !w || !dy || !dx || !dw) return fail(DIG_ERR_NULL, "x, w, dy, dx and dw are required");
  const void* ptrs[] = {x, w, dy, dx, dw, dbias_opt, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DIG_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
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

}  // extern "C"
