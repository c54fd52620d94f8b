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
// The last identity carries G backwards.  A segment's incoming G comes either from
// recomputing it over all later chunks in the same workgroup (short sequences), or from
// pass A (per-segment local G from zero) + a reverse scan over segments.  The output-stage
// backward (head-wise RMSNorm x weight x Swish) recomputes o from the saved S0.
#include <type_traits>

#include "dig_device.h"
#include "dig_internal.h"

namespace dig {

constexpr int kBThreads = 256;
constexpr float kBSlowDecayLog2 = 96.0f;

static int brup(int x, int m) { return (x + m - 1) / m * m; }

// LDS carve-up; matrix-core operands use rows padded by 8 elements (bank spread).
GlaBwdLds gla_bwd_lds(const GlaShape& s, bool fin) {
  GlaBwdLds l;
  const int T = s.bf16 ? 2 : 4;
  l.DKP = brup(16 * s.ndk, 32);
  l.DK16 = s.ndk;
  l.DV16 = s.ndv;
  l.DVP = 16 * s.ndv;
  l.DVK = brup(16 * s.ndv, 32);
  l.CK = s.bf16 ? brup(s.C, 32) : s.C;
  const int QP = l.DKP + 8, VP = l.DVK + 8, PP = l.CK + 8;
  const int cpad = s.ndk <= 2 ? 32 : 64;
  int off = 0;
  auto take = [&](int bytes) { int o = off; off += brup(bytes, 16); return o; };
  l.off_q = take(l.CK * QP * T);                     // q e^{b}          [CK][QP]
  l.off_k = take(l.CK * QP * T);                     // k e^{-b}         [CK][QP]
  l.off_kb = take(fin ? l.CK * QP * T : 0);          // k e^{blast-b}    [CK][QP]
  l.off_v = take(l.CK * VP * T);                     // v                [CK][VP]
  l.off_do = take(l.CK * VP * T);                    // dO               [CK][VP]
  l.off_s0 = take(l.DKP * VP * T);                   // S0               [DKP][VP]
  l.off_g = take(fin ? l.DKP * VP * T : 0);          // G                [DKP][VP]
  const int pd = fin ? l.CK * PP * T : 0;
  l.off_p = take(pd);                                // P                [CK][PP]
  l.off_d = take(pd);                                // dO V^T           [CK][PP]
  l.off_b = take(s.C * s.dk * 4);                    // log2 cumsum b    [C][dk] fp32
  l.off_w = l.off_b;  // q.dq - k.dk reuses the cumsum array once dq, dk are formed
  l.off_raw = take(3 * s.C * s.dk * T);              // raw q, k, z (packed rows, LDS DMA)
  l.off_rdy = take(3 * s.C * s.dv * T);              // raw r, dy, v
  l.off_qk = take((256 / cpad) * cpad * 4);          // per-segment gate sums [seg][col]
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

template <typename T, int NDK, int NDV, bool FIN>
__global__ __launch_bounds__(kBThreads) void gla_bwd_kernel(GlaBwdParams p) {
  constexpr int DKP = ((NDK * 16 + 31) / 32) * 32;
  constexpr int DVP = NDV * 16;
  constexpr int DVK = ((NDV * 16 + 31) / 32) * 32;
  constexpr int QP = DKP + 8, VP = DVK + 8;  // padded row pitches
  constexpr int NST = NDK * NDV;
  constexpr int STW = (NST + 3) / 4;
  constexpr int CPAD = NDK <= 2 ? 32 : 64;   // gate pass: lanes over key columns
  constexpr int NSEGT = kBThreads / CPAD;    // ... and token segments
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int C = p.C, NT = C >> 4;
  const int nseg_launch = FIN ? p.nseg : p.nseg - 1;
  const int seg = (FIN ? 0 : 1) + (int)(blockIdx.x % nseg_launch);
  const int bh = blockIdx.x / nseg_launch;
  const int b = bh / p.H, h = bh - b * p.H;
  const int H = p.H, dk = p.dk, dv = p.dv;
  const GlaBwdLds& Ld = p.lds;
  const int CK = Ld.CK, PP = CK + 8;
  const int npair = NT * NDK;  // (row tile, key tile) pairs of dq / dk

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
  T* rawv = sDy + C * dv;
  float* sTot = reinterpret_cast<float*>(smem + Ld.off_qk);
  float* sPart = reinterpret_cast<float*>(smem + Ld.off_part);
  float* sGam = reinterpret_cast<float*>(smem + Ld.off_gam);
  float* sLg = reinterpret_cast<float*>(smem + Ld.off_misc);
  float* sMax = sLg + DKP;
  float* sDg = sMax + 4;         // [4][DVP] dgamma partials per wave
  float* sDiag = sDg + 4 * DVP;  // [C] diagonal of dO V^T from the fp32 dO

  for (int i = tid; i < Ld.bytes / 16; i += kBThreads)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  const int c_first = seg * p.sc;
  const int c_end = min(p.NC, c_first + p.sc);
  const int n_top = (FIN && p.prefix) ? p.NC : c_end;  // later chunks recomputed for G
  const bool scanned = !p.prefix && p.nseg > 1;
  const long sbase = (long)bh * p.NC;
  const DmaMap mk = dma_map<T>(dk, lane), mv = dma_map<T>(dv, lane);
  const int gc = tid % CPAD, gs = tid / CPAD, TL = C / NSEGT;

  // gradient state G (fp32, tile layout: tile u = wave + 4m -> (key tile, value tile))
  f32x4 gacc[STW];
#pragma unroll
  for (int m = 0; m < STW; ++m) gacc[m] = zero4();
  if (FIN && scanned) {
    const float* src = p.gstates + ((long)bh * p.nseg + seg) * dk * dv;
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave + 4 * m;
      if (u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
        const int e = et * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ct * 16 + g4 * 4 + i;
          gacc[m][i] = (c < dk && e < dv) ? src[c * dv + e] : 0.f;
        }
      }
    }
  }

  const T* gq = static_cast<const T*>(p.q);
  const T* gk = static_cast<const T*>(p.k);
  const T* gv = static_cast<const T*>(p.v);
  const T* gz = static_cast<const T*>(p.z);
  const T* gr = static_cast<const T*>(p.r);
  const T* gdy = static_cast<const T*>(p.dy);

  float gm[NDV], dgam[NDV];
#pragma unroll
  for (int E = 0; E < NDV; ++E) {
    const int e = E * 16 + r16;
    gm[E] = (e < dv && p.norm_w) ? p.norm_w[e] : 1.f;
    dgam[E] = 0.f;
  }

  for (int n = n_top - 1; n >= c_first; --n) {
    const bool own = FIN && n < c_end;  // gradients of this chunk are this workgroup's output
    const int t0 = n * C;
    const int valid = min(C, p.L - t0);
    const long row0 = ((long)b * p.L + t0) * H + h;
    const float* s0src = p.states + (sbase + n) * dk * dv;

    // ---- stage the raw operands (asynchronous global->LDS copies, one round trip), the
    // saved state entering the chunk and the current G
    dma_rows<T>(mk, rawq, gq + row0 * dk, (long)H * dk, valid, wave, 4, lane);
    dma_rows<T>(mk, rawk, gk + row0 * dk, (long)H * dk, valid, wave, 4, lane);
    dma_rows<T>(mk, rawz, gz + row0 * dk, (long)H * dk, valid, wave, 4, lane);
    dma_rows<T>(mv, rawv, gv + row0 * dv, (long)H * dv, valid, wave, 4, lane);
    dma_rows<T>(mv, sRr, gr + row0 * dv, (long)H * dv, valid, wave, 4, lane);
    dma_rows<T>(mv, sDy, gdy + row0 * dv, (long)H * dv, valid, wave, 4, lane);
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave + 4 * m;
      if (u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
        const int e = et * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ct * 16 + g4 * 4 + i;
          sS0[c * VP + e] = from_f<T>((c < dk && e < dv) ? s0src[c * dv + e] : 0.f);
          if (own) sG[c * VP + e] = from_f<T>(gacc[m][i]);
        }
      }
    }
    dma_wait();
    __syncthreads();
    if (valid < C) {  // ragged last chunk: rows past the sequence are zero
      zero_rows<T>(rawq, valid, C, dk, tid, kBThreads);
      zero_rows<T>(rawk, valid, C, dk, tid, kBThreads);
      zero_rows<T>(rawz, valid, C, dk, tid, kBThreads);
      zero_rows<T>(rawv, valid, C, dv, tid, kBThreads);
      zero_rows<T>(sRr, valid, C, dv, tid, kBThreads);
      zero_rows<T>(sDy, valid, C, dv, tid, kBThreads);
      __syncthreads();
    }

    // ---- gate, pass 1: g = log2(sigmoid(z))/tau and its running sum along each column's
    // token segment (lanes over key columns); V into its padded layout
    {
      float run = 0.f;
      if (gc < dk) {
        for (int j = 0; j < TL; ++j) {
          const int t = gs * TL + j;
          const float g2 = t < valid ? Fm<T>::lsig2(to_f(rawz[t * dk + gc])) * p.inv_tau : 0.f;
          run += g2;
          sB[t * dk + gc] = run;
        }
      }
      sTot[gs * CPAD + gc] = run;
      for (int i = tid; i < C * DVP; i += kBThreads) {
        const int e = i % DVP, t = i / DVP;
        if (e < dv) sV[t * VP + e] = rawv[t * dv + e];
      }
    }
    __syncthreads();

    // ---- gate, pass 2: segment offsets complete b; scaled operands
    {
      float off = 0.f, blast = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < NSEGT; ++s2) {
        const float tv = sTot[s2 * CPAD + gc];
        if (s2 < gs) off += tv;
        blast += tv;
      }
      if (gc < dk) {
        for (int j = 0; j < TL; ++j) {
          const int t = gs * TL + j;
          const float bb = sB[t * dk + gc] + off;
          const float kf = to_f(rawk[t * dk + gc]);
          const float qf = to_f(rawq[t * dk + gc]) * p.q_scale;
          sQ[t * QP + gc] = from_f<T>(qf * Fm<T>::exp2(bb));
          sK[t * QP + gc] = from_f<T>(kf * Fm<T>::exp2(-bb));
          if (own) sKb[t * QP + gc] = from_f<T>(kf * Fm<T>::exp2(blast - bb));
          sB[t * dk + gc] = bb;
        }
        if (gs == 0) {
          sGam[gc] = Fm<T>::exp2(blast);
          if (FIN)
            sLg[gc] = blast;  // this chunk's log2 decay, for the e^{b_last - b} factors
          else
            sLg[gc] += blast;  // segment's log2 decay
        }
      }
      if (wave == 0) {  // wave 0 holds segment 0 of every column
        const float md = wave_max((gs == 0 && gc < dk) ? -blast : 0.f);
        if (lane == 0) sMax[0] = md;
      }
    }
    __syncthreads();
    const bool slow = sMax[0] > kBSlowDecayLog2;

    // ---- recompute o for row tile I, then the output-stage backward -> dO, dr, dgamma
    if (wave < NT) {
      const int I = wave;
      float diag;  // exact q_i.k_i from the unscaled inputs (gate factor 1)
      {
        const int ir = 16 * I + r16, cq = (dk + 3) >> 2;
        // fp32 I/O accumulates in fp64: the sum can cancel far below its terms
        using Acc = typename std::conditional<sizeof(T) == 4, double, float>::type;
        Acc acc = 0;
        for (int c = g4 * cq; c < min(dk, g4 * cq + cq); ++c)
          acc += (Acc)to_f(rawq[ir * dk + c]) * (Acc)to_f(rawk[ir * dk + c]);
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        diag = (float)acc * p.q_scale;
      }
      f32x4 pt[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        pt[J] = zero4();
        if (J <= I) {
          if (!slow) {
            pt[J] = Mma<T>::kc(zero4(), sK, QP, 16 * J, sQ, QP, 16 * I, DKP, lane);
          } else {
            const int ir = 16 * I + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 16 * J + 4 * g4 + i;
              float acc = 0.f;
              if (j <= ir) {
                for (int c = 0; c < dk; ++c)
                  acc += to_f(rawq[ir * dk + c]) * to_f(rawk[j * dk + c]) *
                         Fm<T>::exp2(sB[ir * dk + c] - sB[j * dk + c]);
                acc *= p.q_scale;
              }
              pt[J][i] = acc;
            }
          }
          if (J == I) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (4 * g4 + i > r16) pt[J][i] = 0.f;
              if (4 * g4 + i == r16) pt[J][i] = diag;
            }
          }
          // P kept for dv (tiles up to the diagonal; the rest of sP stays zero)
          if (own) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sP[(16 * I + r16) * PP + 16 * J + 4 * g4 + i] = from_f<T>(pt[J][i]);
          }
        }
      }
      f32x4 oacc[NDV];
#pragma unroll
      for (int E = 0; E < NDV; ++E) oacc[E] = zero4();
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          if (2 * pp <= I) {
            const bool hi_on = 2 * pp + 1 <= I;
            bf16x8 a;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              a[i] = from_f<bf16>(pt[2 * pp][i]);
              a[4 + i] = from_f<bf16>(hi_on ? pt[2 * pp + 1][i] : 0.f);
            }
#pragma unroll
            for (int E = 0; E < NDV; ++E) {
              const int e = E * 16 + r16;
              bf16x8 bv;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                bv[i] = sV[(32 * pp + 4 * g4 + i) * VP + e];
                bv[4 + i] = sV[(32 * pp + 16 + 4 * g4 + i) * VP + e];
              }
              oacc[E] = mfma_bf16(a, bv, oacc[E]);
            }
          }
        }
      } else {
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          if (J <= I) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
              for (int E = 0; E < NDV; ++E) {
                const float bv = to_f(sV[(16 * J + 4 * g4 + s4) * VP + E * 16 + r16]);
                oacc[E] = mfma_f32(pt[J][s4], bv, oacc[E]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int E = 0; E < NDV; ++E)
        oacc[E] = Mma<T>::template mm<true, false>(oacc[E], sQ, QP, 16 * I, sS0, VP, 16 * E,
                                                   DKP, lane);

      float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int E = 0; E < NDV; ++E)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss[i] += oacc[E][i] * oacc[E][i];
      float rstd[4], md[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) rstd[i] = rsqrtf(sum16(ss[i]) / (float)dv + p.eps);
      // oacc becomes the normalised output n, dn holds dy * w * swish(r)
      float dn[NDV][4];
#pragma unroll
      for (int E = 0; E < NDV; ++E) {
        const int e = E * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dn[E][i] = 0.f;
          oacc[E][i] *= rstd[i];
          if (e < dv) {
            const int row = 16 * I + 4 * g4 + i;
            const float nv = oacc[E][i];
            const float rv = to_f(sRr[row * dv + e]);
            const float dyv = to_f(sDy[row * dv + e]);
            const float sg = Fm<T>::sig(rv);
            const float sw = rv * sg;
            if (own) {
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
      using Acc = typename std::conditional<sizeof(T) == 4, double, float>::type;
      Acc dvd[4] = {0, 0, 0, 0};
#pragma unroll
      for (int E = 0; E < NDV; ++E) {
        const int e = E * 16 + r16;
        if (e < dv) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * I + 4 * g4 + i;
            const float dov = rstd[i] * (dn[E][i] - oacc[E][i] * md[i]);
            sdO[row * VP + e] = from_f<T>(dov);
            dvd[i] += (Acc)dov * (Acc)to_f(sV[row * VP + e]);
          }
        }
      }
      // do_i is orthogonal to the normalised o_i (up to eps); when o_i is parallel to v_i
      // (the first token) do_i.v_i cancels, so it is formed here from the fp32 do_i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Acc dd = dvd[i];
        dd += __shfl_xor(dd, 1);
        dd += __shfl_xor(dd, 2);
        dd += __shfl_xor(dd, 4);
        dd += __shfl_xor(dd, 8);
        if (own && r16 == 0) sDiag[16 * I + 4 * g4 + i] = (float)dd;
      }
    }
    __syncthreads();

    if (own) {
      // ---- D = dO V^T (causal), S_end and the boundary term sum_e S_end (.) G
      for (int q = wave; q < NT * NT; q += 4) {
        const int I = q / NT, J = q - I * NT;
        if (J <= I) {
          f32x4 d = Mma<T>::kc(zero4(), sdO, VP, 16 * I, sV, VP, 16 * J, DVK, lane);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ii = 16 * I + 4 * g4 + i, jj = 16 * J + r16;
            sD[ii * PP + jj] = from_f<T>(jj < ii ? d[i] : (jj == ii ? sDiag[ii] : 0.f));
          }
        }
      }
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        const int u = wave + 4 * m;
        if (u < NST) {
          const int ct = u / NDV, et = u - ct * NDV;
          const int e = et * 16 + r16;
          f32x4 se;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = ct * 16 + g4 * 4 + i;
            se[i] = (c < dk && e < dv) ? s0src[c * dv + e] * sGam[c] : 0.f;
          }
          se = Mma<T>::template mm<false, false>(se, sKb, QP, 16 * ct, sV, VP, 16 * et, CK, lane);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float part = sum16(se[i] * gacc[m][i]);
            if (r16 == 0) sPart[et * DKP + ct * 16 + g4 * 4 + i] = part;
          }
        }
      }
      __syncthreads();

      // ---- dq, dk (kept in registers), dv (staged over dy)
      f32x4 dqa[NDK], dka[NDK];
#pragma unroll
      for (int m = 0; m < NDK; ++m) {
        dqa[m] = zero4();
        dka[m] = zero4();
        const int u = wave + 4 * m;
        if (u < npair) {
          const int I = u / NDK, ct = u - I * NDK;
          const f32x4 a1 = Mma<T>::kc(zero4(), sdO, VP, 16 * I, sS0, VP, 16 * ct, DVK, lane);
          const f32x4 a3 = Mma<T>::kc(zero4(), sV, VP, 16 * I, sG, VP, 16 * ct, DVK, lane);
          f32x4 a2 = zero4(), a4 = zero4();
          if (!slow) {
            a2 = Mma<T>::template mm<true, false>(zero4(), sD, PP, 16 * I, sK, QP, 16 * ct, CK,
                                                  lane);
            a4 = Mma<T>::template mm<false, false>(zero4(), sD, PP, 16 * I, sQ, QP, 16 * ct, CK,
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
                dq = Fm<T>::exp2(bt) * (a1[i] + a2[i]);
                dkk = Fm<T>::exp2(-bt) * a4[i] + Fm<T>::exp2(blast - bt) * a3[i];
              } else {
                float s1 = 0.f, s2 = 0.f;
                for (int j = 0; j <= t && j < C; ++j)
                  s1 += to_f(sD[t * PP + j]) * to_f(rawk[j * dk + c]) * Fm<T>::exp2(bt - sB[j * dk + c]);
                for (int i2 = t; i2 < C; ++i2)
                  s2 += to_f(sD[i2 * PP + t]) * to_f(rawq[i2 * dk + c]) * p.q_scale *
                        Fm<T>::exp2(sB[i2 * dk + c] - bt);
                dq = Fm<T>::exp2(bt) * a1[i] + s1;
                dkk = s2 + Fm<T>::exp2(blast - bt) * a3[i];
              }
            }
            dqa[m][i] = dq;
            dka[m][i] = dkk;
          }
        }
      }
      for (int q = wave; q < NT * NDV; q += 4) {
        const int J = q / NDV, et = q - J * NDV;
        f32x4 a = Mma<T>::template mm<false, false>(zero4(), sP, PP, 16 * J, sdO, VP, 16 * et, CK,
                                                    lane);
        a = Mma<T>::template mm<true, false>(a, sKb, QP, 16 * J, sG, VP, 16 * et, DKP, lane);
        const int e = et * 16 + r16;
        if (e < dv) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sDy[(16 * J + 4 * g4 + i) * dv + e] = from_f<T>(a[i]);
        }
      }
      __syncthreads();

      // ---- q.dq - k.dk into sW; dq, dk staged over raw q, k
#pragma unroll
      for (int m = 0; m < NDK; ++m) {
        const int u = wave + 4 * m;
        if (u < npair) {
          const int I = u / NDK, ct = u - I * NDK;
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
    for (int m = 0; m < STW; ++m) {
      const int u = wave + 4 * m;
      if (u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ct * 16 + g4 * 4 + i;
          gacc[m][i] *= (c < dk) ? sGam[c] : 1.f;
        }
        gacc[m] = Mma<T>::template mm<false, false>(gacc[m], sQ, QP, 16 * ct, sdO, VP, 16 * et,
                                                    CK, lane);
      }
    }
    __syncthreads();

    if (own) {
      // ---- dlog(alpha): in-chunk suffix sum + boundary term; dz = dlog(alpha) sigmoid(-z)/tau
      // (lanes over key columns; each column's suffix sums run along its token segment)
      float run = 0.f;
      if (gc < dk) {
        for (int j = TL - 1; j >= 0; --j) {
          const int t = gs * TL + j;
          run += t < valid ? sW[t * dk + gc] : 0.f;
        }
      }
      sTot[gs * CPAD + gc] = run;
      __syncthreads();
      if (gc < dk) {
        float off = 0.f, bterm = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < NSEGT; ++s2)
          if (s2 > gs) off += sTot[s2 * CPAD + gc];
        for (int et = 0; et < NDV; ++et) bterm += sPart[et * DKP + gc];
        float suf = off + bterm;
        for (int j = TL - 1; j >= 0; --j) {
          const int t = gs * TL + j;
          suf += t < valid ? sW[t * dk + gc] : 0.f;
          float dla = suf;
          if (n == 0 && t == 0) dla = 0.f;  // alpha_0 multiplies the zero initial state
          const float zf = to_f(rawz[t * dk + gc]);
          rawz[t * dk + gc] = from_f<T>(dla * Fm<T>::sig(-zf) * p.inv_tau);
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
    for (int E = 0; E < NDV; ++E) {
      float v = dgam[E];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (g4 == 0) sDg[wave * DVP + E * 16 + r16] = v;
    }
    __syncthreads();
    for (int e = tid; e < dv; e += kBThreads)
      p.dgamma_part[(long)blockIdx.x * dv + e] =
          ((sDg[e] + sDg[DVP + e]) + sDg[2 * DVP + e]) + sDg[3 * DVP + e];
  } else {
    float* dst = p.gstates + ((long)bh * p.nseg + seg) * dk * dv;
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave + 4 * m;
      if (u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
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

// out[e] = sum over parts of part[i][e]: one block per column e, a fixed-order tree (the
// same bits on every run).
__global__ __launch_bounds__(kBThreads) void gla_dgamma_reduce(const float* part, int nparts,
                                                              int dv, float* out) {
  __shared__ float red[kBThreads];
  const int e = blockIdx.x, tid = threadIdx.x;
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

template <typename T, int NDK, int NDV>
static hipError_t launch_bt(const GlaShape& s, GlaBwdParams p, hipStream_t st) {
  const long BH = (long)s.B * s.H;
  if (!s.prefix && s.nseg > 1) {
    GlaBwdParams pa = p;
    pa.lds = gla_bwd_lds(s, false);
    hipLaunchKernelGGL((gla_bwd_kernel<T, NDK, NDV, false>), dim3((unsigned)(BH * (s.nseg - 1))),
                       dim3(kBThreads), pa.lds.bytes, st, pa);
    const long nthreads = BH * s.dk * s.dv;
    hipLaunchKernelGGL(gla_gstate_scan, dim3((unsigned)((nthreads + kBThreads - 1) / kBThreads)),
                       dim3(kBThreads), 0, st, p.gstates, p.seg_lg, (int)BH, s.nseg, s.dk, s.dv);
  }
  p.lds = gla_bwd_lds(s, true);
  hipLaunchKernelGGL((gla_bwd_kernel<T, NDK, NDV, true>), dim3((unsigned)(BH * s.nseg)),
                     dim3(kBThreads), p.lds.bytes, st, p);
  if (p.d_norm_w)
    hipLaunchKernelGGL(gla_dgamma_reduce, dim3(s.dv), dim3(kBThreads), 0, st, p.dgamma_part,
                       (int)(BH * s.nseg), s.dv, p.d_norm_w);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bcls(const GlaShape& s, GlaBwdParams p, hipStream_t st) {
  switch (s.ndk * 16 + s.ndv) {
    case 1 * 16 + 2: return launch_bt<T, 1, 2>(s, p, st);
    case 2 * 16 + 4: return launch_bt<T, 2, 4>(s, p, st);
    case 3 * 16 + 5: return launch_bt<T, 3, 5>(s, p, st);
    case 4 * 16 + 8: return launch_bt<T, 4, 8>(s, p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gla_bwd(const GlaShape& s, GlaBwdParams p, hipStream_t st) {
  p.B = s.B; p.L = s.L; p.H = s.H; p.dk = s.dk; p.dv = s.dv;
  p.NC = s.NC; p.sc = s.sc; p.nseg = s.nseg;
  p.C = s.C; p.prefix = s.prefix;
  return s.bf16 ? launch_bcls<bf16>(s, p, st) : launch_bcls<float>(s, p, st);
}

}  // namespace dig
