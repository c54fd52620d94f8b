// gla_bwd.hip -- chunkwise backward of DiG's gated linear attention on gfx950.
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
// The last identity carries G backwards; across segments it is scanned like the forward
// state.  The output-stage backward (head-wise RMSNorm x weight x Swish) recomputes o.
#include "dig_device.h"
#include "dig_internal.h"

namespace dig {

constexpr int kBThreads = 256;
constexpr int kBMaxStateTiles = 8;  // state/gradient-state tiles per wave
constexpr int kBMaxPairs = 4;       // (row tile, key tile) pairs per wave for dq/dk
constexpr float kBSlowDecayLog2 = 96.0f;

static int brup(int x, int m) { return (x + m - 1) / m * m; }

GlaBwdLds gla_bwd_lds(const GlaShape& s, bool fin) {
  GlaBwdLds l;
  const int T = s.bf16 ? 2 : 4;
  l.DKP = brup(s.dk, 32);
  l.DK16 = (s.dk + 15) / 16;
  l.DV16 = (s.dv + 15) / 16;
  l.DVP = l.DV16 * 16;
  l.DVK = brup(s.dv, 32);
  l.CK = s.bf16 ? brup(s.C, 32) : s.C;
  int off = 0;
  auto take = [&](int bytes) { int o = off; off += brup(bytes, 16); return o; };
  l.off_q = take(l.CK * l.DKP * T);
  l.off_k = take(l.CK * l.DKP * T);
  l.off_kb = take(fin ? l.CK * l.DKP * T : 0);
  l.off_v = take(l.CK * l.DVK * T);
  l.off_do = take(l.CK * l.DVK * T);
  l.off_s0 = take(l.DKP * l.DVK * T);
  l.off_g = take(fin ? l.DKP * l.DVK * T : 0);
  const int pd = fin ? l.CK * l.CK * T : 0;
  l.off_p = take(pd);
  l.off_d = take(pd);
  l.off_b = take(s.C * s.dk * 4);
  l.off_w = l.off_b;  // q.dq - k.dk reuses the cumsum array once dq, dk are formed
  l.off_raw = take(3 * s.C * s.dk * T);
  l.off_rdy = take(2 * s.C * s.dv * T);
  l.off_part = take(fin ? l.DV16 * l.DKP * 4 : 0);
  l.off_gam = take(l.DKP * 4);
  l.off_misc = take(l.DKP * 4 + 4 * 4 + 4 * l.DVP * 4 + s.C * 4);
  l.bytes = off;
  return l;
}

size_t gla_bwd_workspace(const GlaShape& s) {
  const size_t BH = (size_t)s.B * s.H;
  size_t g = BH * s.nseg * s.dk * s.dv * sizeof(float);
  size_t lg = BH * s.nseg * s.dk * sizeof(float);
  size_t part = BH * s.nseg * s.dv * sizeof(float);
  auto a = [](size_t x) { return (x + 255) / 256 * 256; };
  return a(g) + a(lg) + a(part);
}

template <typename T, int C, bool FIN>
__global__ __launch_bounds__(kBThreads) void gla_bwd_kernel(GlaBwdParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int nseg_launch = FIN ? p.nseg : p.nseg - 1;
  const int seg = (FIN ? 0 : 1) + (int)(blockIdx.x % nseg_launch);
  const int bh = blockIdx.x / nseg_launch;
  const int b = bh / p.H, h = bh - b * p.H;
  const int H = p.H, dk = p.dk, dv = p.dv;
  const GlaBwdLds& Ld = p.lds;
  const int DKP = Ld.DKP, DV16 = Ld.DV16, DVK = Ld.DVK, CK = Ld.CK, DK16 = Ld.DK16,
            DVP = Ld.DVP;
  constexpr int NT = C / 16;

  T* sQ = reinterpret_cast<T*>(smem + Ld.off_q);
  T* sK = reinterpret_cast<T*>(smem + Ld.off_k);
  T* sKb = reinterpret_cast<T*>(smem + Ld.off_kb);
  T* sV = reinterpret_cast<T*>(smem + Ld.off_v);
  T* sdO = reinterpret_cast<T*>(smem + Ld.off_do);
  T* sS0 = reinterpret_cast<T*>(smem + Ld.off_s0);
  T* sG = reinterpret_cast<T*>(smem + Ld.off_g);
  T* sP = reinterpret_cast<T*>(smem + Ld.off_p);
  T* sD = reinterpret_cast<T*>(smem + Ld.off_d);
  float* sW = reinterpret_cast<float*>(smem + Ld.off_w);
  float* sB = reinterpret_cast<float*>(smem + Ld.off_b);
  T* rawq = reinterpret_cast<T*>(smem + Ld.off_raw);
  T* rawk = rawq + C * dk;
  T* rawz = rawk + C * dk;
  T* sRr = reinterpret_cast<T*>(smem + Ld.off_rdy);  // r, then dr
  T* sDy = sRr + C * dv;                               // dy, then dv
  float* sPart = reinterpret_cast<float*>(smem + Ld.off_part);
  float* sGam = reinterpret_cast<float*>(smem + Ld.off_gam);
  float* sLg = reinterpret_cast<float*>(smem + Ld.off_misc);
  float* sMax = sLg + DKP;
  float* sDg = sMax + 4;            // [4][DVP] dgamma partials per wave
  float* sDiag = sDg + 4 * DVP;     // [C] diagonal of dO V^T from the fp32 dO

  for (int i = tid; i < Ld.bytes / 16; i += kBThreads)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  const int c_first = seg * p.sc;
  const int c_end = min(p.NC, c_first + p.sc);
  const int nst = DK16 * DV16;
  const int npair = NT * DK16;
  const long sbase = (long)bh * p.NC;

  // gradient state G (fp32, tile layout: tile u = wave + 4m -> (key tile, value tile))
  f32x4 gacc[kBMaxStateTiles];
#pragma unroll
  for (int m = 0; m < kBMaxStateTiles; ++m) gacc[m] = zero4();
  if (FIN && p.nseg > 1) {
    const float* src = p.gstates + ((long)bh * p.nseg + seg) * dk * dv;
#pragma unroll
    for (int m = 0; m < kBMaxStateTiles; ++m) {
      const int u = wave + 4 * m;
      if (u < nst) {
        const int ct = u / DV16, et = u - ct * DV16;
        const int e = et * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ct * 16 + g4 * 4 + i;
          gacc[m][i] = (c < dk && e < dv) ? src[c * dv + e] : 0.f;
        }
      }
    }
  }
  if (FIN) {
#pragma unroll
    for (int m = 0; m < kBMaxStateTiles; ++m) {
      const int u = wave + 4 * m;
      if (u < nst) {
        const int ct = u / DV16, et = u - ct * DV16;
        const int e = et * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) sG[(ct * 16 + g4 * 4 + i) * DVK + e] = from_f<T>(gacc[m][i]);
      }
    }
  }

  const T* gq = static_cast<const T*>(p.q);
  const T* gk = static_cast<const T*>(p.k);
  const T* gv = static_cast<const T*>(p.v);
  const T* gz = static_cast<const T*>(p.z);
  const T* gr = static_cast<const T*>(p.r);
  const T* gdy = static_cast<const T*>(p.dy);

  float gm[8], dgam[8];
#pragma unroll
  for (int E = 0; E < 8; ++E) {
    const int e = E * 16 + r16;
    gm[E] = (E < DV16 && e < dv && p.norm_w) ? p.norm_w[e] : 1.f;
    dgam[E] = 0.f;
  }
  __syncthreads();

  for (int n = c_end - 1; n >= c_first; --n) {
    const int t0 = n * C;
    const int valid = min(C, p.L - t0);
    const long row0 = ((long)b * p.L + t0) * H + h;

    // ---- stage operands and the saved state entering the chunk
    stage_rows<T>(rawq, dk, gq + row0 * dk, (long)H * dk, C, valid, dk, tid, kBThreads);
    stage_rows<T>(rawk, dk, gk + row0 * dk, (long)H * dk, C, valid, dk, tid, kBThreads);
    stage_rows<T>(rawz, dk, gz + row0 * dk, (long)H * dk, C, valid, dk, tid, kBThreads);
    stage_rows<T>(sV, DVK, gv + row0 * dv, (long)H * dv, C, valid, dv, tid, kBThreads);
    stage_rows<T>(sRr, dv, gr + row0 * dv, (long)H * dv, C, valid, dv, tid, kBThreads);
    stage_rows<T>(sDy, dv, gdy + row0 * dv, (long)H * dv, C, valid, dv, tid, kBThreads);
    f32x4 sacc[kBMaxStateTiles];
    {
      const float* src = p.states + (sbase + n) * dk * dv;
#pragma unroll
      for (int m = 0; m < kBMaxStateTiles; ++m) {
        sacc[m] = zero4();
        const int u = wave + 4 * m;
        if (u < nst) {
          const int ct = u / DV16, et = u - ct * DV16;
          const int e = et * 16 + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = ct * 16 + g4 * 4 + i;
            const float val = (c < dk && e < dv) ? src[c * dv + e] : 0.f;
            sacc[m][i] = val;
            sS0[c * DVK + e] = from_f<T>(val);
          }
        }
      }
    }
    __syncthreads();

    // ---- gate and in-chunk cumsum (log2 domain)
    {
      constexpr int G = 64 / C;
      const int grp = lane / C, tl = lane - grp * C;
      float maxdec = 0.f;
      for (int c0 = wave * G; c0 < dk; c0 += 4 * G) {
        const int c = c0 + grp;
        const bool cv = c < dk;
        const float zf = cv ? to_f(rawz[tl * dk + c]) : 0.f;
        const float g2 = (cv && tl < valid) ? logsigmoid_f(zf) * p.g2scale : 0.f;
        const float bb = group_inclusive_scan(g2, C, tl);
        const float blast = __shfl(bb, C - 1, C);
        if (cv) {
          const float kf = to_f(rawk[tl * dk + c]);
          const float qf = to_f(rawq[tl * dk + c]) * p.q_scale;
          sQ[tl * DKP + c] = from_f<T>(qf * exp2f(bb));
          sK[tl * DKP + c] = from_f<T>(kf * exp2f(-bb));
          if (FIN) sKb[tl * DKP + c] = from_f<T>(kf * exp2f(blast - bb));
          sB[tl * dk + c] = bb;
          if (tl == C - 1) {
            sGam[c] = exp2f(blast);
            if (FIN)
              sLg[c] = blast;  // this chunk's log2 decay, for the e^{b_last - b} factors
            else
              sLg[c] += blast;  // segment's log2 decay
          }
          maxdec = fmaxf(maxdec, -blast);
        }
      }
      maxdec = wave_max(maxdec);
      if (lane == 0) sMax[wave] = maxdec;
    }
    __syncthreads();
    const bool slow = fmaxf(fmaxf(sMax[0], sMax[1]), fmaxf(sMax[2], sMax[3])) > kBSlowDecayLog2;

    // ---- recompute o for row tile I, then the output-stage backward -> dO, dr, dgamma
    for (int I = wave; I < NT; I += 4) {
      f32x4 pt[NT];
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        pt[J] = zero4();
        if (J <= I) {
          if (!slow) {
            pt[J] = Mma<T>::kc(zero4(), sK, DKP, 16 * J, sQ, DKP, 16 * I, DKP, lane);
          } else {
            const int ir = 16 * I + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 16 * J + 4 * g4 + i;
              float acc = 0.f;
              if (j <= ir) {
                for (int c = 0; c < dk; ++c)
                  acc += to_f(rawq[ir * dk + c]) * to_f(rawk[j * dk + c]) *
                         exp2f(sB[ir * dk + c] - sB[j * dk + c]);
                acc *= p.q_scale;
              }
              pt[J][i] = acc;
            }
          }
          if (J == I) {
            // causal mask; the diagonal (gate factor exactly 1) is q_i.k_i formed in fp32 from
            // the unscaled inputs, so a cancelling dot product keeps its relative accuracy
            const int ir = 16 * I + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (4 * g4 + i > r16) pt[J][i] = 0.f;
              if (4 * g4 + i == r16) {
                float acc = 0.f;
                for (int c = 0; c < dk; ++c) acc += to_f(rawq[ir * dk + c]) * to_f(rawk[ir * dk + c]);
                pt[J][i] = acc * p.q_scale;
              }
            }
          }
        }
        // every tile is written, zeros above the diagonal
        if (FIN) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sP[(16 * I + r16) * CK + 16 * J + 4 * g4 + i] = from_f<T>(pt[J][i]);
        }
      }
      f32x4 oacc[8];
#pragma unroll
      for (int E = 0; E < 8; ++E) oacc[E] = zero4();
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int pp = 0; pp < (NT + 1) / 2; ++pp) {
          if (2 * pp <= I) {
            const int J0 = 2 * pp, J1 = 2 * pp + 1;
            bf16x8 a;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              a[i] = from_f<bf16>(pt[J0][i]);
              a[4 + i] = from_f<bf16>((J1 < NT && J1 <= I) ? pt[J1 < NT ? J1 : 0][i] : 0.f);
            }
#pragma unroll
            for (int E = 0; E < 8; ++E) {
              if (E < DV16) {
                const int e = E * 16 + r16;
                bf16x8 bv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  bv[i] = sV[(32 * pp + 4 * g4 + i) * DVK + e];
                  bv[4 + i] = sV[(32 * pp + 16 + 4 * g4 + i) * DVK + e];
                }
                oacc[E] = mfma_bf16(a, bv, oacc[E]);
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int J = 0; J < NT; ++J) {
          if (J <= I) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
              for (int E = 0; E < 8; ++E) {
                if (E < DV16) {
                  const float bv = to_f(sV[(16 * J + 4 * g4 + s4) * DVK + E * 16 + r16]);
                  oacc[E] = mfma_f32(pt[J][s4], bv, oacc[E]);
                }
              }
            }
          }
        }
      }
#pragma unroll
      for (int E = 0; E < 8; ++E)
        if (E < DV16)
          oacc[E] = Mma<T>::template mm<true, false>(oacc[E], sQ, DKP, 16 * I, sS0, DVK, 16 * E,
                                                     DKP, lane);

      float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int E = 0; E < 8; ++E)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss[i] += oacc[E][i] * oacc[E][i];
      float rstd[4], md[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) rstd[i] = rsqrtf(sum16(ss[i]) / (float)dv + p.eps);
      float dn[8][4];
#pragma unroll
      for (int E = 0; E < 8; ++E) {
        const int e = E * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dn[E][i] = 0.f;
          if (E < DV16 && e < dv) {
            const int row = 16 * I + 4 * g4 + i;
            const float nv = oacc[E][i] * rstd[i];
            const float rv = to_f(sRr[row * dv + e]);
            const float dyv = to_f(sDy[row * dv + e]);
            const float sg = sigmoid_f(rv);
            const float sw = rv * sg;
            if (FIN) {
              dgam[E] += dyv * nv * sw;
              sRr[row * dv + e] = from_f<T>(dyv * nv * gm[E] * sg * (1.f + rv * (1.f - sg)));
            }
            dn[E][i] = dyv * gm[E] * sw;
            md[i] += dn[E][i] * nv;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) md[i] = sum16(md[i]) / (float)dv;
      float dvd[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int E = 0; E < 8; ++E) {
        const int e = E * 16 + r16;
        if (E < DV16 && e < dv) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * I + 4 * g4 + i;
            const float nv = oacc[E][i] * rstd[i];
            const float dov = rstd[i] * (dn[E][i] - nv * md[i]);
            sdO[row * DVK + e] = from_f<T>(dov);
            dvd[i] += dov * to_f(sV[row * DVK + e]);
          }
        }
      }
      // do_i is orthogonal to the normalised o_i (up to eps); when o_i is parallel to v_i
      // (the first token) do_i.v_i cancels, so it is formed here from the fp32 do_i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dd = sum16(dvd[i]);
        if (FIN && r16 == 0) sDiag[16 * I + 4 * g4 + i] = dd;
      }
    }
    __syncthreads();

    if (FIN) {
      // ---- D = dO V^T (causal), S_end and the boundary term sum_e S_end (.) G
      // every tile is written, zeros above the diagonal
      for (int q = wave; q < NT * NT; q += 4) {
        const int I = q / NT, J = q - I * NT;
        f32x4 d = zero4();
        if (J <= I) d = Mma<T>::kc(zero4(), sdO, DVK, 16 * I, sV, DVK, 16 * J, DVK, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ii = 16 * I + 4 * g4 + i, jj = 16 * J + r16;
          sD[ii * CK + jj] = from_f<T>(jj < ii ? d[i] : (jj == ii ? sDiag[ii] : 0.f));
        }
      }
#pragma unroll
      for (int m = 0; m < kBMaxStateTiles; ++m) {
        const int u = wave + 4 * m;
        if (u < nst) {
          const int ct = u / DV16, et = u - ct * DV16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = ct * 16 + g4 * 4 + i;
            sacc[m][i] *= (c < dk) ? sGam[c] : 1.f;
          }
          sacc[m] = Mma<T>::template mm<false, false>(sacc[m], sKb, DKP, 16 * ct, sV, DVK,
                                                      16 * et, CK, lane);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float part = sum16(sacc[m][i] * gacc[m][i]);
            if (r16 == 0) sPart[et * DKP + ct * 16 + g4 * 4 + i] = part;
          }
        }
      }
      __syncthreads();

      // ---- dq, dk (kept in registers), dv (staged over dy)
      f32x4 dqa[kBMaxPairs], dka[kBMaxPairs];
#pragma unroll
      for (int m = 0; m < kBMaxPairs; ++m) {
        dqa[m] = zero4();
        dka[m] = zero4();
        const int u = wave + 4 * m;
        if (u < npair) {
          const int I = u / DK16, ct = u - I * DK16;
          f32x4 a1 = Mma<T>::kc(zero4(), sdO, DVK, 16 * I, sS0, DVK, 16 * ct, DVK, lane);
          f32x4 a3 = Mma<T>::kc(zero4(), sV, DVK, 16 * I, sG, DVK, 16 * ct, DVK, lane);
          f32x4 a2, a4;
          if (!slow) {
            a2 = Mma<T>::template mm<true, false>(zero4(), sD, CK, 16 * I, sK, DKP, 16 * ct, CK,
                                                  lane);
            a4 = Mma<T>::template mm<false, false>(zero4(), sD, CK, 16 * I, sQ, DKP, 16 * ct, CK,
                                                   lane);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * I + 4 * g4 + i, c = ct * 16 + r16;
            float dq = 0.f, dkk = 0.f;
            if (c < dk) {
              const float bt = sB[t * dk + c];
              const float blast = sLg[c];
              if (!slow) {
                dq = exp2f(bt) * (a1[i] + a2[i]);
                dkk = exp2f(-bt) * a4[i] + exp2f(blast - bt) * a3[i];
              } else {
                float s1 = 0.f, s2 = 0.f;
                for (int j = 0; j <= t && j < C; ++j)
                  s1 += to_f(sD[t * CK + j]) * to_f(rawk[j * dk + c]) * exp2f(bt - sB[j * dk + c]);
                for (int i2 = t; i2 < C; ++i2)
                  s2 += to_f(sD[i2 * CK + t]) * to_f(rawq[i2 * dk + c]) * p.q_scale *
                        exp2f(sB[i2 * dk + c] - bt);
                dq = exp2f(bt) * a1[i] + s1;
                dkk = s2 + exp2f(blast - bt) * a3[i];
              }
            }
            dqa[m][i] = dq;
            dka[m][i] = dkk;
          }
        }
      }
      for (int q = wave; q < NT * DV16; q += 4) {
        const int J = q / DV16, et = q - J * DV16;
        f32x4 a = Mma<T>::template mm<false, false>(zero4(), sP, CK, 16 * J, sdO, DVK, 16 * et, CK,
                                                    lane);
        a = Mma<T>::template mm<true, false>(a, sKb, DKP, 16 * J, sG, DVK, 16 * et, DKP, lane);
        const int e = et * 16 + r16;
        if (e < dv) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sDy[(16 * J + 4 * g4 + i) * dv + e] = from_f<T>(a[i]);
        }
      }
      __syncthreads();

      // ---- q.dq - k.dk into sW; dq, dk staged over raw q, k; gradient state update
#pragma unroll
      for (int m = 0; m < kBMaxPairs; ++m) {
        const int u = wave + 4 * m;
        if (u < npair) {
          const int I = u / DK16, ct = u - I * DK16;
          const int c = ct * 16 + r16;
          if (c < dk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = 16 * I + 4 * g4 + i;
              const float qf = to_f(rawq[t * dk + c]) * p.q_scale;
              const float kf = to_f(rawk[t * dk + c]);
              sW[t * dk + c] = qf * dqa[m][i] - kf * dka[m][i];
              rawq[t * dk + c] = from_f<T>(p.q_scale * dqa[m][i]);
              rawk[t * dk + c] = from_f<T>(dka[m][i]);
            }
          }
        }
      }
    }

    // gradient state: G <- diag(e^{b_last}) G + (q e^{b})^T dO
#pragma unroll
    for (int m = 0; m < kBMaxStateTiles; ++m) {
      const int u = wave + 4 * m;
      if (u < nst) {
        const int ct = u / DV16, et = u - ct * DV16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ct * 16 + g4 * 4 + i;
          gacc[m][i] *= (c < dk) ? sGam[c] : 1.f;
        }
        gacc[m] = Mma<T>::template mm<false, false>(gacc[m], sQ, DKP, 16 * ct, sdO, DVK, 16 * et,
                                                    CK, lane);
        if (FIN) {
          const int e = et * 16 + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) sG[(ct * 16 + g4 * 4 + i) * DVK + e] = from_f<T>(gacc[m][i]);
        }
      }
    }
    __syncthreads();

    if (FIN) {
      // ---- dlog(alpha): in-chunk suffix sum + boundary term; dz = dlog(alpha) sigmoid(-z)/tau
      constexpr int G = 64 / C;
      const int grp = lane / C, tl = lane - grp * C;
      for (int c0 = wave * G; c0 < dk; c0 += 4 * G) {
        const int c = c0 + grp;
        const bool cv = c < dk;
        const float w = (cv && tl < valid) ? sW[tl * dk + c] : 0.f;
        const float suf = group_inclusive_suffix(w, C, tl);
        if (cv) {
          float bterm = 0.f;
          for (int et = 0; et < DV16; ++et) bterm += sPart[et * DKP + c];
          float dla = suf + bterm;
          if (n == 0 && tl == 0) dla = 0.f;  // alpha_0 multiplies the zero initial state
          const float zf = to_f(rawz[tl * dk + c]);
          rawz[tl * dk + c] = from_f<T>(dla * sigmoid_f(-zf) * p.inv_tau);
        }
      }
      __syncthreads();
      T* gdq = static_cast<T*>(p.dq);
      T* gdk = static_cast<T*>(p.dk_);
      T* gdz = static_cast<T*>(p.dz);
      T* gdv = static_cast<T*>(p.dv_);
      T* gdr = static_cast<T*>(p.dr);
      store_rows<T>(gdq + row0 * dk, (long)H * dk, rawq, dk, valid, dk, tid, kBThreads);
      store_rows<T>(gdk + row0 * dk, (long)H * dk, rawk, dk, valid, dk, tid, kBThreads);
      store_rows<T>(gdz + row0 * dk, (long)H * dk, rawz, dk, valid, dk, tid, kBThreads);
      store_rows<T>(gdv + row0 * dv, (long)H * dv, sDy, dv, valid, dv, tid, kBThreads);
      store_rows<T>(gdr + row0 * dv, (long)H * dv, sRr, dv, valid, dv, tid, kBThreads);
      __syncthreads();
    }
  }

  if (FIN) {
    // per-workgroup partial of dgamma, reduced in a fixed order
#pragma unroll
    for (int E = 0; E < 8; ++E) {
      float v = dgam[E];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (g4 == 0 && E < DV16) sDg[wave * DVP + E * 16 + r16] = v;
    }
    __syncthreads();
    for (int e = tid; e < dv; e += kBThreads)
      p.dgamma_part[(long)blockIdx.x * dv + e] =
          ((sDg[e] + sDg[DVP + e]) + sDg[2 * DVP + e]) + sDg[3 * DVP + e];
  } else {
    float* dst = p.gstates + ((long)bh * p.nseg + seg) * dk * dv;
#pragma unroll
    for (int m = 0; m < kBMaxStateTiles; ++m) {
      const int u = wave + 4 * m;
      if (u < nst) {
        const int ct = u / DV16, et = u - ct * DV16;
        const int e = et * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ct * 16 + g4 * 4 + i;
          if (c < dk && e < dv) dst[c * dv + e] = gacc[m][i];
        }
      }
    }
    for (int c = tid; c < dk; c += kBThreads) p.seg_lg[((long)bh * p.nseg + seg) * dk + c] = sLg[c];
  }
}

// Reverse exclusive scan over segments, in place: slot(p) <- gradient reaching the end of
// segment p from later segments.  G(nseg-1) = 0, G(p-1) = 2^{lg(p)} G(p) + dG(p).
__global__ __launch_bounds__(kBThreads) void gla_gstate_scan(float* gst, const float* seg_lg,
                                                            int BH, int nseg, int dk, int dv) {
  const long idx = (long)blockIdx.x * kBThreads + threadIdx.x;
  const long per = (long)dk * dv;
  if (idx >= (long)BH * per) return;
  const long bh = idx / per, ce = idx - bh * per;
  const int c = (int)(ce / dv);
  float* base = gst + bh * nseg * per + ce;
  const float* lg = seg_lg + bh * nseg * dk + c;
  float G = 0.f;
  for (int ps = nseg - 1; ps >= 1; --ps) {
    const float d = base[(long)ps * per];
    base[(long)ps * per] = G;
    G = exp2f(lg[ps * dk]) * G + d;
  }
  base[0] = G;
}

__global__ __launch_bounds__(kBThreads) void gla_dgamma_reduce(const float* part, int nparts,
                                                              int dv, float* out) {
  const int e = blockIdx.x * kBThreads + threadIdx.x;
  if (e >= dv) return;
  float s = 0.f;
  for (int i = 0; i < nparts; ++i) s += part[(long)i * dv + e];
  out[e] = s;
}

template <typename T, int C>
static hipError_t launch_bt(const GlaShape& s, GlaBwdParams p, hipStream_t st) {
  const long BH = (long)s.B * s.H;
  if (s.nseg > 1) {
    GlaBwdParams pa = p;
    pa.lds = gla_bwd_lds(s, false);
    hipLaunchKernelGGL((gla_bwd_kernel<T, C, false>), dim3((unsigned)(BH * (s.nseg - 1))),
                       dim3(kBThreads), pa.lds.bytes, st, pa);
    const long nthreads = BH * s.dk * s.dv;
    hipLaunchKernelGGL(gla_gstate_scan, dim3((unsigned)((nthreads + kBThreads - 1) / kBThreads)),
                       dim3(kBThreads), 0, st, p.gstates, p.seg_lg, (int)BH, s.nseg, s.dk, s.dv);
  }
  p.lds = gla_bwd_lds(s, true);
  hipLaunchKernelGGL((gla_bwd_kernel<T, C, true>), dim3((unsigned)(BH * s.nseg)),
                     dim3(kBThreads), p.lds.bytes, st, p);
  if (p.d_norm_w)
    hipLaunchKernelGGL(gla_dgamma_reduce, dim3((s.dv + kBThreads - 1) / kBThreads),
                       dim3(kBThreads), 0, st, p.dgamma_part, (int)(BH * s.nseg), s.dv,
                       p.d_norm_w);
  return hipGetLastError();
}

hipError_t launch_gla_bwd(const GlaShape& s, GlaBwdParams p, hipStream_t st) {
  p.B = s.B; p.L = s.L; p.H = s.H; p.dk = s.dk; p.dv = s.dv;
  p.NC = s.NC; p.sc = s.sc; p.nseg = s.nseg;
  if (s.bf16) {
    switch (s.C) {
      case 16: return launch_bt<bf16, 16>(s, p, st);
      case 32: return launch_bt<bf16, 32>(s, p, st);
      default: return launch_bt<bf16, 64>(s, p, st);
    }
  }
  switch (s.C) {
    case 16: return launch_bt<float, 16>(s, p, st);
    case 32: return launch_bt<float, 32>(s, p, st);
    default: return launch_bt<float, 64>(s, p, st);
  }
}

}  // namespace dig
