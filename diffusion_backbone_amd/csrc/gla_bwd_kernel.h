// gla_bwd_kernel.h -- the chunk kernel of the GLA backward on gfx950 (included by the
// per-element-type translation units gla_bwd_bf16.hip and gla_bwd_f32.hip).
//
// Gradients of <dy, y> through the forward (DiG study-group slides, eqs. (5)-(10), by the
// chain rule).  Per image and head, with do the gradient at the pre-norm output o, S_t the
// state after token t and dS_t the gradient flowing into S_t:
//   dq_t = S_t do_t,   dk_t = dS_t v_t,   dv_t = k_t dS_t,
//   dlog(alpha_u) = sum_{t >= u} (q_t.dq_t - k_t.dk_t)          (elementwise per key dim)
// Chunk form: b = in-chunk inclusive cumsum of log(alpha), S0 = state entering the chunk
// (saved by the forward), G = gradient reaching the chunk's end state from later chunks,
// D = dO V^T and P = gated Q K^T (both causal inside the chunk):
//   dq_i = e^{b_i} (do_i S0^T + sum_{j<=i} D_ij k_j e^{-b_j})
//   dk_j = e^{-b_j} sum_{i>=j} D_ij q_i e^{b_i} + e^{b_last-b_j} (G v_j)
//   dv_j = sum_{i>=j} P_ij do_i + (k_j e^{-b_j}) (e^{b_last} G)
//   dlog(alpha_u) = sum_{t>=u in chunk} (q.dq - k.dk)_t + sum_e (S_end (.) G)[:, e]
//   G_prev = diag(e^{b_last}) G + sum_i (q_i e^{b_i})^T do_i
// S_end, the state leaving the chunk, is the saved state entering the next chunk (and G is
// zero after the last chunk).  The output-stage backward (head-wise RMSNorm x weight x
// Swish) recomputes o from S0.
//
// Phases of one chunk (four waves, barriers between):
//   gate      lanes = tokens: log-sigmoid, DPP cumulative sum, q e^{b}, k e^{-b} in row and
//             transposed layouts, V in a padded row layout;
//   recompute wave I: gated Q K^T rows 16I.., o = P V + (q e^b) S0, RMSNorm x Swish
//             backward -> dO (row and transposed), dr, dgamma;
//   D         dO V^T tiles (row and transposed), the boundary term of dlog(alpha);
//   grads     dq, dk (row tile x key tile pairs), dv, and the carried G;
//   dlog      lanes = tokens in reverse: suffix sums of q.dq - k.dk as a DPP scan -> dz.
// Pass A of the three-pass scheme (chunks that only carry G) runs gate, recompute and the G
// update only.  Exact head shapes load the next chunk's raw rows into registers while the
// current one is processed; tile classes copy them global->LDS after the chunk is done.
#pragma once

#include <type_traits>

#include "dig_device.h"
#include "dig_internal.h"

namespace dig {

#ifndef DIG_BWD_WAVES8
#define DIG_BWD_WAVES8 8
#endif
constexpr float kBwdSlowDecayLog2 = 96.0f;

constexpr int bal16(int x) { return (x + 15) / 16 * 16; }


// LDS layout (compile time).  LEAN drops the row-layout copies of dO, S0 and D (their
// products then read the transposed copies with strided fragments) when the full layout
// would not fit.  PAD gives the raw staging rows pitches at which the gate pass (one lane
// per token) reads without bank conflicts (register-staged rows only; LDS DMA writes rows
// packed).  The fp32 per-token rows (b, q.dq - k.dk) have an odd pitch for the same reason.
// LR: the key gate is the rank-16 product formed in the kernel (factor rows staged beside the
// others, the head's slice of the up-projection in an LDS table; the z rows stage dz only).
template <typename T, int DK, int DV, int C, bool FIN, bool LEAN, int NW = 4, bool PAD = false,
          bool LR = false>
struct BwdLayout {
  static constexpr int SZ = (int)sizeof(T);
  static constexpr int NDK = (DK + 15) / 16, NDV = (DV + 15) / 16;
  static constexpr int DKP = 16 * NDK, DVP = 16 * NDV;           // contraction pads (K 16)
  static constexpr int QP = DKP + 8, VP = DVP + 8, TP = C + 8;    // padded row pitches
  // gate columns per lane: the key tiles' columns over the lanes' column groups, rounded up
  // (short chunks have more groups than columns: the groups past the tiles do nothing)
  static constexpr int NGRP = 64 * NW / C;
  static constexpr int NCL = (DKP + NGRP - 1) / NGRP;
  static constexpr int NEL = (DVP + NGRP - 1) / NGRP;  // value columns per lane (V rows)
  // the row layouts of q e^{b}, k e^{-b} are fp32 for either element type (bf16 I/O splits
  // them into hi + lo bf16 fragments for the gated Q K^T): QKC stored columns (d_k rounded up
  // to 4) at pitch QKP floats; the transposed copies are of the element type
  static constexpr int QKC = SZ == 2 ? (DK + 3) / 4 * 4 : DKP;
  static constexpr int QKP = SZ == 2 ? (QKC % 32 == 0 ? QKC + 4 : QKC) : QP;
  static constexpr int KPE = PAD ? row_pitch(DK * SZ, NCL * SZ) / SZ : DK;  // raw k pitch
  static constexpr int VPE = PAD ? row_pitch(DV * SZ, NEL * SZ) / SZ : DV;  // raw v pitch
  static constexpr int DKB = DK % 2 ? DK : DK + 1;                // fp32 row pitch (odd)
  // row layouts [token][dim]
  static constexpr int O_Q = 0;                                          // q e^{b}  [C][QKP]
  static constexpr int O_K = O_Q + bal16(C * QKP * 4);                   // k e^{-b} [C][QKP]
  static constexpr int O_V = O_K + bal16(C * QKP * 4);                   // v         [C][VP]
  static constexpr int O_DO = O_V + bal16(C * VP * SZ);                  // dO        [C][VP]
  static constexpr int O_S0 = O_DO + bal16(LEAN ? 0 : C * VP * SZ);      // S0      [DKP][VP]
  static constexpr int O_D = O_S0 + bal16(LEAN ? 0 : DKP * VP * SZ);     // dO V^T    [C][TP]
  // transposed layouts [dim][token] and [value][key]
  static constexpr int O_QT = O_D + bal16(FIN && !LEAN ? C * TP * SZ : 0);  // (q e^b)^T [DKP][TP]
  static constexpr int O_KT = O_QT + bal16(DKP * TP * SZ);               // (k e^-b)^T [DKP][TP]
  static constexpr int O_DOT = O_KT + bal16(FIN ? DKP * TP * SZ : 0);    // dO^T     [DVP][TP]
  static constexpr int O_S0T = O_DOT + bal16(DVP * TP * SZ);             // S0^T     [DVP][QP]
  static constexpr int O_GT = O_S0T + bal16(DVP * QP * SZ);              // G^T      [DVP][QP]
  static constexpr int O_PT = O_GT + bal16(FIN ? DVP * QP * SZ : 0);     // P^T        [C][TP]
  // D^T [C][TP]; during the recompute phase the strong-decay P rows [4][16][C] live here
  static constexpr int DT_BYTES = (FIN ? C * TP * SZ : 0) > 4 * 16 * C * SZ
                                      ? (FIN ? C * TP * SZ : 0) : 4 * 16 * C * SZ;
  static constexpr int O_DT = O_PT + bal16(FIN ? C * TP * SZ : 0);
  // fp32 scratch
  static constexpr int O_B = O_DT + bal16(DT_BYTES);                 // b        [C][DKB]
  static constexpr int O_W = O_B + bal16(C * DKB * 4);               // q.dq-k.dk [C][DKB]
  static constexpr int O_GAM = O_W + bal16(FIN ? C * DKB * 4 : 0);   // e^{b_last}  [DKP]
  static constexpr int O_LG = O_GAM + bal16(DKP * 4);                // b_last / segment decay
  static constexpr int O_MAX = O_LG + bal16(DKP * 4);                // per-wave decay [NW]
  static constexpr int O_PART = O_MAX + 64;                          // [DKP][8]
  static constexpr int O_DG = O_PART + bal16(DKP * 8 * 4);           // [NW][DVP]
  static constexpr int O_DIAG = O_DG + bal16(NW * DVP * 4);          // [2][C] (halves)
  static constexpr int O_XCH = O_DIAG + bal16(2 * C * 4);            // [4][C] row sums
  static constexpr int O_ZT = O_XCH + bal16(4 * C * 4);              // low-rank gate table
  static constexpr int O_RAW = O_ZT + bal16(LR ? lowrank_table_bytes(DKP) : 0);
  // raw staging: q, k, z (pitch KPE, or the runtime d_k when packed), v, r, dy (pitch VPE)
  static constexpr int R_Q = 0;
  static constexpr int R_K = R_Q + bal16(C * KPE * SZ);
  static constexpr int R_Z = R_K + bal16(C * KPE * SZ);
  static constexpr int R_V = R_Z + bal16(C * KPE * SZ);
  // r then dr, dy then dv: rows at a pitch that is a multiple of four elements when
  // register-staged (the recompute phase reads them through the transpose load; the gate pass
  // does not read them)
  static constexpr int RPE = PAD ? (DV + 3) / 4 * 4 : DV;
  static constexpr int R_R = R_V + bal16(C * (VPE > 2 * KPE ? VPE : 2 * KPE) * SZ);  // v; dq|dk
  static constexpr int R_DY = R_R + bal16(C * RPE * SZ);
  // factor rows (LR): 16 elements, packed (the final pass has no LDS left for a padded pitch)
  static constexpr int ZPE = kGateRank;
  static constexpr int R_F = R_DY + bal16(C * RPE * SZ);
  static constexpr int SLOT = R_F + bal16(LR ? C * ZPE * SZ : 0);
  static constexpr int bytes = O_RAW + SLOT;
};
constexpr int kBwdLdsBudget = 160 * 1024;
template <typename T, int DK, int DV, int C, bool FIN, int NW = 4, bool PAD = false,
          bool LR = false>
constexpr bool bwd_lean() {
  return BwdLayout<T, DK, DV, C, FIN, false, NW, PAD, LR>::bytes > kBwdLdsBudget;
}

// Register prefetch of the next chunk's raw rows (exact head shapes).  The recomputing final
// pass drops it when a wave holds more than one state tile: those registers then go to the
// tiles (with the prefetch the compiler spills inside the chunk loop).  The final pass that
// reads pass A's dO (RD) has the registers to keep it.
template <int DK, int DV, bool EXACT, bool FIN, int NW, bool RD = false>
constexpr bool bwd_prefetch() {
  constexpr int stw = ((DK + 15) / 16 * ((DV + 15) / 16) + NW - 1) / NW;
  return EXACT && !(FIN && !RD && stw > 1);
}

// Reuse of pass A's output-stage backward (RU, three-pass calls): pass A stores dO in its
// register-fragment order (Vec4 per lane, [chunk][wave][value tile][lane]), the rows' exact
// dO.v diagonal and dr; the final pass then reads dO and the diagonal instead of recomputing
// o = P V + (q e^b) S0 and the RMSNorm x Swish backward, and reads neither r nor dy.  Needs
// every wave in the recompute phase (row tiles x value halves = waves).
template <int C, int NW>
constexpr int bwd_spl() {
  return NW >= 2 * (C / 16) ? 2 : 1;
}
template <int DK, int DV, bool EXACT, int C, int NW>
constexpr bool bwd_reuse_ok() {
  return EXACT && (C / 16) * bwd_spl<C, NW>() == NW;
}
template <typename T, int DV, int C, int NW>
constexpr size_t bwd_reuse_chunk_bytes() {
  constexpr int NDVH = ((DV + 15) / 16 + bwd_spl<C, NW>() - 1) / bwd_spl<C, NW>();
  return (size_t)NW * NDVH * 64 * 4 * sizeof(T) + 2 * C * sizeof(float);
}

// Look-back (LB, short sequences, one chunk per workgroup, one launch): each workgroup
// publishes its chunk's own contribution to the gradient state, U = (q e^b)^T dO, with the
// chunk's log2 decay and its dgamma partial, then raises its flag; the gradient reaching its
// chunk's end is the decayed sum of the later chunks' U:
//   G(n) = U(n+1) + diag(e^{b_last(n+1)}) U(n+2) + diag(e^{b_last(n+1) + b_last(n+2)}) U(n+3) ...
// Later chunks get lower workgroup indices, so every workgroup waited on was dispatched
// before the waiter (in-order dispatch): the waits cannot deadlock.  The last workgroup
// reduces the dgamma partials in a fixed order once every flag is up.  Flags hold this
// call's tag, so values left by earlier calls never match; each wait is bounded.
template <typename T, int DK, int DV, bool EXACT, int C, bool FIN, int NW, bool RU = false,
          bool LB = false, bool LR = false>
__global__ __launch_bounds__(64 * NW) void gla_bwd_kernel(GlaBwdParams p) {
  static_assert(!LR || sizeof(T) == 2, "the low-rank gate is bf16");
  static_assert(!RU || bwd_reuse_ok<DK, DV, EXACT, C, NW>(), "reuse needs every wave in the recompute phase");
  static_assert(!LB || (FIN && !RU), "the look-back runs the recomputing final pass");
  constexpr bool RD = FIN && RU;  // the final pass reads dO (skips the output-stage backward)
  constexpr bool PF = bwd_prefetch<DK, DV, EXACT, FIN, NW, RD>();
  constexpr bool LEAN = bwd_lean<T, DK, DV, C, FIN, NW, PF, LR>();
  using Lo = BwdLayout<T, DK, DV, C, FIN, LEAN, NW, PF, LR>;
  constexpr int ZPE = Lo::ZPE, RPE = Lo::RPE;
  constexpr int KPE = Lo::KPE, VPE = Lo::VPE, DKB = Lo::DKB;
  constexpr int NTH = 64 * NW;  // NW waves
  constexpr bool kBf = sizeof(T) == 2;
  constexpr int NDK = Lo::NDK, NDV = Lo::NDV, DKP = Lo::DKP, DVP = Lo::DVP;
  constexpr int QP = Lo::QP, VP = Lo::VP, TP = Lo::TP;
  constexpr int QKC = Lo::QKC, QKP = Lo::QKP;  // fp32 q e^{b}, k e^{-b} row tiles
  constexpr int NT = C / 16;
  constexpr int NST = NDK * NDV, STW = (NST + NW - 1) / NW;
  constexpr int NPAIR = NT * NDK, PRW = (NPAIR + NW - 1) / NW;  // dq/dk (row tile, key tile)
  constexpr int NDVT = NT * NDV, DVW = (NDVT + NW - 1) / NW;    // dv (row tile, value tile)
  constexpr int NCL = Lo::NCL;                               // gate: key columns per lane
  constexpr int NEL = Lo::NEL;                               // gate: value columns per lane
  constexpr bool FULLK = EXACT && DK == DKP, FULLV = EXACT && DV == DVP;
  static_assert(NCL >= 1 && NEL >= 1, "tile split");
  static_assert(NCL * (NTH / C) >= DKP && NEL * (NTH / C) >= DVP, "the gate pass covers every column");
  constexpr bool KOVER = NCL * (NTH / C) > DKP;  // column groups past the key tiles (short chunks)
  static_assert(QKC % NCL == 0 || QKC >= DKP, "gate column runs end at the stored columns");
  using Acc = typename std::conditional<kBf, float, double>::type;
  constexpr int RNDVH = (NDV + bwd_spl<C, NW>() - 1) / bwd_spl<C, NW>();  // reuse fragments

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  // pass A covers every segment: segment 0's G is not needed, but its dgamma partial is (with
  // more than one segment the dgamma partials come from pass A and the scan reduces them)
  // (look-back: later segments first, so that a workgroup waits only on earlier ones)
  const int seg = LB ? p.nseg - 1 - (int)(blockIdx.x % p.nseg) : (int)(blockIdx.x % p.nseg);
  const int bh = blockIdx.x / p.nseg;
  const bool dg_here = FIN ? (p.nseg == 1 || LB) : true;
  const int b = bh / p.H, h = bh - b * p.H;
  const int H = p.H;
  const int dk = EXACT ? DK : p.dk, dv = EXACT ? DV : p.dv;

  float* sQ = reinterpret_cast<float*>(smem + Lo::O_Q);
  float* sK = reinterpret_cast<float*>(smem + Lo::O_K);
  T* sV = reinterpret_cast<T*>(smem + Lo::O_V);
  T* sdO = reinterpret_cast<T*>(smem + Lo::O_DO);
  T* sS0 = reinterpret_cast<T*>(smem + Lo::O_S0);
  T* sD = reinterpret_cast<T*>(smem + Lo::O_D);
  T* sQt = reinterpret_cast<T*>(smem + Lo::O_QT);
  T* sKt = reinterpret_cast<T*>(smem + Lo::O_KT);
  T* sdOt = reinterpret_cast<T*>(smem + Lo::O_DOT);
  T* sS0t = reinterpret_cast<T*>(smem + Lo::O_S0T);
  T* sGt = reinterpret_cast<T*>(smem + Lo::O_GT);
  T* sPt = reinterpret_cast<T*>(smem + Lo::O_PT);
  T* sDt = reinterpret_cast<T*>(smem + Lo::O_DT);
  float* sB = reinterpret_cast<float*>(smem + Lo::O_B);
  float* sW = reinterpret_cast<float*>(smem + Lo::O_W);  // q.dq - k.dk [C][DK]
  float* sGam = reinterpret_cast<float*>(smem + Lo::O_GAM);
  float* sLg = reinterpret_cast<float*>(smem + Lo::O_LG);
  float* sMax = reinterpret_cast<float*>(smem + Lo::O_MAX);
  float* sPart = reinterpret_cast<float*>(smem + Lo::O_PART);
  float* sDg = reinterpret_cast<float*>(smem + Lo::O_DG);
  float* sDiag = reinterpret_cast<float*>(smem + Lo::O_DIAG);
  float* sXch = reinterpret_cast<float*>(smem + Lo::O_XCH);
  T* sSlow = reinterpret_cast<T*>(smem + Lo::O_DT);  // strong-decay P rows (recompute only)
  T* rawq = reinterpret_cast<T*>(smem + Lo::O_RAW + Lo::R_Q);
  T* rawk = reinterpret_cast<T*>(smem + Lo::O_RAW + Lo::R_K);
  T* rawz = reinterpret_cast<T*>(smem + Lo::O_RAW + Lo::R_Z);  // then dz
  const bf16* rawf = reinterpret_cast<const bf16*>(smem + Lo::O_RAW + Lo::R_F);  // factor (LR)
  T* rawv = reinterpret_cast<T*>(smem + Lo::O_RAW + Lo::R_V);  // then dq | dk
  // raw row pitches: padded for register-staged rows, the runtime widths for DMA-staged ones
  const int kp = PF ? KPE : dk, vp = PF ? VPE : dv, rp = PF ? RPE : dv;
  T* sdqs = rawv;
  T* sdks = rawv + C * kp;
  T* sRr = reinterpret_cast<T*>(smem + Lo::O_RAW + Lo::R_R);   // r, then dr
  T* sDy = reinterpret_cast<T*>(smem + Lo::O_RAW + Lo::R_DY);  // dy, then dv

  const int c_first = seg * p.sc;
  const int c_end = min(p.NC, c_first + p.sc);
  const int n_top = c_end;
  const bool scanned = p.nseg > 1;  // G entering the segment's end comes from the scan
  const long sbase = (long)bh * p.NC;
  const float inv_tau = p.g2scale * 0.69314718055994531f;  // g2scale = log2(e) / tau

  const T* gq = static_cast<const T*>(p.q);
  const T* gk = static_cast<const T*>(p.k);
  const T* gv = static_cast<const T*>(p.v);
  const T* gz = static_cast<const T*>(p.z);
  const T* gr = static_cast<const T*>(p.r);
  const T* gdy = static_cast<const T*>(p.dy);

  auto issue = [&](int n) {
    unsigned char* base = smem + Lo::O_RAW;
    const int t0 = n * C, valid = min(C, p.L - t0);
    const long row0 = ((long)b * p.L + t0) * H + h;
    const long gsk = (long)H * dk * sizeof(T), gsv = (long)H * dv * sizeof(T);
    const int rbk = dk * (int)sizeof(T), rbv = dv * (int)sizeof(T);
    dma_rows_c(base + Lo::R_Q, reinterpret_cast<const unsigned char*>(gq + row0 * dk), gsk, rbk,
               valid, wave, NW, lane);
    if constexpr (FIN)  // pass A forms no P: no k
      dma_rows_c(base + Lo::R_K, reinterpret_cast<const unsigned char*>(gk + row0 * dk), gsk,
                 rbk, valid, wave, NW, lane);
    if constexpr (LR)
      dma_rows_c(base + Lo::R_F,
                 reinterpret_cast<const unsigned char*>(gz + ((long)b * p.L + t0) * kGateRank),
                 kGateRank * sizeof(T), kGateRank * (int)sizeof(T), valid, wave, NW, lane);
    else
      dma_rows_c(base + Lo::R_Z, reinterpret_cast<const unsigned char*>(gz + row0 * dk), gsk,
                 rbk, valid, wave, NW, lane);
    dma_rows_c(base + Lo::R_V, reinterpret_cast<const unsigned char*>(gv + row0 * dv), gsv, rbv,
               valid, wave, NW, lane);
    if constexpr (!RD) {
      dma_rows_c(base + Lo::R_R, reinterpret_cast<const unsigned char*>(gr + row0 * dv), gsv,
                 rbv, valid, wave, NW, lane);
      dma_rows_c(base + Lo::R_DY, reinterpret_cast<const unsigned char*>(gdy + row0 * dv), gsv,
                 rbv, valid, wave, NW, lane);
    }
  };
  // this lane's elements of the fp32 state tiles of chunk n (the saved forward states)
  // (exact shapes: branch-free, padding positions hold clamped copies that are masked where
  // the state becomes an MFMA operand; they only meet zeros elsewhere)
  auto load_state = [&](int n, f32x4 (&dst)[STW]) {
    const float* src = p.states + (sbase + n) * dk * dv;
    if constexpr (PF && DK % 4 == 0) {
      // A lane's four rows lie all inside d_k or all in the padding (where any rows do): one
      // 32-bit offset per tile, the rows at immediate offsets from it.
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        const int u = min(wave + NW * m, NST - 1);
        const int ct = u / NDV, et = u - ct * NDV;
        const int e = min(et * 16 + r16, DV - 1);
        const unsigned off = (unsigned)((min(ct * 16 + g4 * 4, DK - 4) * DV + e) * (int)sizeof(float));
        const char* sp = reinterpret_cast<const char*>(src) + off;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[m][i] = *reinterpret_cast<const float*>(sp + i * DV * (int)sizeof(float));
      }
      return;
    } else if constexpr (PF) {
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        const int u = min(wave + NW * m, NST - 1);
        const int ct = u / NDV, et = u - ct * NDV;
        const int e = min(et * 16 + r16, DV - 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[m][i] = src[min(ct * 16 + g4 * 4 + i, DK - 1) * DV + e];
      }
      return;
    }
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      dst[m] = zero4();
      const int u = wave + NW * m;
      if (u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
        const int e = et * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ct * 16 + g4 * 4 + i;
          if ((FULLK || c < dk) && (FULLV || e < dv)) dst[m][i] = src[c * dv + e];
        }
      }
    }
  };

  RowRegs<DK * (int)sizeof(T), C, NTH, KPE * (int)sizeof(T)> pq, pk;
  RowRegs<(LR ? kGateRank : DK) * (int)sizeof(T), C, NTH, (LR ? ZPE : KPE) * (int)sizeof(T)> pz;
  RowRegs<DV * (int)sizeof(T), C, NTH, VPE * (int)sizeof(T)> pv;
  RowRegs<DV * (int)sizeof(T), C, NTH, RPE * (int)sizeof(T)> pr, pdy;
  auto pf_load = [&](int n) {
    const int t0 = n * C, valid = min(C, p.L - t0);
    const long row0 = ((long)b * p.L + t0) * H + h;
    const long gsk = (long)H * DK * sizeof(T), gsv = (long)H * DV * sizeof(T);
    pq.load(reinterpret_cast<const unsigned char*>(gq + row0 * DK), gsk, valid, tid);
    if constexpr (FIN) pk.load(reinterpret_cast<const unsigned char*>(gk + row0 * DK), gsk, valid, tid);
    if constexpr (LR)
      pz.load(reinterpret_cast<const unsigned char*>(gz + ((long)b * p.L + t0) * kGateRank),
              kGateRank * sizeof(T), valid, tid);
    else
      pz.load(reinterpret_cast<const unsigned char*>(gz + row0 * DK), gsk, valid, tid);
    pv.load(reinterpret_cast<const unsigned char*>(gv + row0 * DV), gsv, valid, tid);
    if constexpr (!RD) {
      pr.load(reinterpret_cast<const unsigned char*>(gr + row0 * DV), gsv, valid, tid);
      pdy.load(reinterpret_cast<const unsigned char*>(gdy + row0 * DV), gsv, valid, tid);
    }
  };
  auto pf_put = [&](int n) {
    unsigned char* base = smem + Lo::O_RAW;
    const int valid = min(C, p.L - n * C);
    pq.put(base + Lo::R_Q, valid, tid);
    if constexpr (FIN) pk.put(base + Lo::R_K, valid, tid);
    pz.put(base + (LR ? Lo::R_F : Lo::R_Z), valid, tid);
    pv.put(base + Lo::R_V, valid, tid);
    if constexpr (!RD) {
      pr.put(base + Lo::R_R, valid, tid);
      pdy.put(base + Lo::R_DY, valid, tid);
    }
  };
  if constexpr (PF) pf_load(n_top - 1);
  else issue(n_top - 1);
  // the look-back's single chunk: its saved o rstd and rstd are loaded with its rows (where
  // a wave holds one state tile: with two, the registers are not there)
  constexpr bool LBPF = LB && STW == 1;
  Quad<float> obr_lb[LBPF ? RNDVH : 1];
  float4 rsv_lb = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (LBPF) {
    const int I = wave % NT, E0 = (wave / NT) * RNDVH;
    const Quad<float>* ob = static_cast<const Quad<float>*>(p.obar) + ((sbase + n_top - 1) * NT + I) * NDV * 64 + lane;
#pragma unroll
    for (int Eh = 0; Eh < RNDVH; ++Eh) obr_lb[Eh] = ob[min(E0 + Eh, NDV - 1) * 64];
    rsv_lb = *reinterpret_cast<const float4*>(p.rstd + (sbase + n_top - 1) * C + 16 * I + 4 * g4);
  }
  for (int i = tid; i < Lo::O_RAW / 16; i += NTH)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();  // the zero fill is complete before anything below writes LDS
  if constexpr (LR)  // read from the first chunk's gate pass on (behind the loop's barrier)
    lowrank_table_fill<DKP, NTH>(smem + Lo::O_ZT, static_cast<const bf16*>(p.zw), p.zb, h, dk,
                                 tid);

  // gradient state G (fp32, tile u = wave + 4m -> (key tile, value tile))
  f32x4 gacc[STW];
#pragma unroll
  for (int m = 0; m < STW; ++m) gacc[m] = zero4();
  if (FIN && scanned && !LB) {
    const float* src = p.gstates + ((long)bh * p.nseg + seg) * dk * dv;
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave + NW * m;
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
  // sum_e S_end (.) G per key column, the boundary term of dlog(alpha) of the chunk about to
  // be processed: S_end is the saved state entering the next chunk up, G the gradient
  // carried into the chunk's end (zero after the last chunk)
  auto write_part = [&](const f32x4 (&se)[STW]) {
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave + NW * m;
      if (u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float part = row_sum16(se[m][i] * gacc[m][i]);
          if (r16 == 0) sPart[(ct * 16 + g4 * 4 + i) * 8 + et] = part;  // (key, value tile)
        }
      }
    }
  };
  // look-back: S_end waits for G (the look-back below); loaded here where a wave holds one
  // state tile, after the look-back where it holds two (registers)
  f32x4 se_lb[LB ? STW : 1];
  if (FIN && n_top < p.NC) {
    if constexpr (LB) {
      if constexpr (STW == 1) load_state(n_top, se_lb);
    } else {
      f32x4 se[STW];
      load_state(n_top, se);
      write_part(se);
    }
  }
  f32x4 s0c[STW];  // S0 of the current chunk (the final pass: pass A forms no o, dq or dk)
  if constexpr (FIN) load_state(n_top - 1, s0c);

  // dgamma partial sums of this wave's value tiles E0 + Eh of its row tiles (E0 fixed per
  // wave: the accumulators take compile-time indices only)
  float gm[NDV], dgl[RNDVH];
#pragma unroll
  for (int E = 0; E < NDV; ++E) {
    const int e = E * 16 + r16;
    gm[E] = (e < dv && p.norm_w) ? p.norm_w[e] : 1.f;
  }
#pragma unroll
  for (int Eh = 0; Eh < RNDVH; ++Eh) dgl[Eh] = 0.f;
  // this wave's column-tile partial of dgamma for tile E (zero outside its tiles)
  auto dgam_of = [&](int E) {
    float v = 0.f;
    if (wave < NT * bwd_spl<C, NW>()) {
      const int E0w = (wave / NT) * RNDVH;
#pragma unroll
      for (int Eh = 0; Eh < RNDVH; ++Eh)
        if (E0w + Eh == E) v = dgl[Eh];
    }
    return v;
  };
  const int tg = tid % C, cg = tid / C;
  const int c0 = cg * NCL, e0 = cg * NEL;
  // Every load above has landed before the loop: otherwise the compiler's wait for them,
  // placed inside the loop, would also wait for the prefetch.
  if constexpr (PF) dma_wait();

  for (int n = n_top - 1; n >= c_first; --n) {
    // per-iteration copies of the lane-dependent indices (see opaque())
    const int lane = opaque(tid & 63);
    const int r16 = lane & 15, g4 = lane >> 4;
    const int tg = (wave * 64 + lane) % C, cg = (wave * 64 + lane) / C;
    const int c0 = cg * NCL, e0 = cg * NEL;
    constexpr bool own = FIN;  // the final pass emits every chunk it walks
    const int t0 = n * C;
    const int valid = min(C, p.L - t0);
    const long row0 = ((long)b * p.L + t0) * H + h;
    if constexpr (PF) {
      if (n < n_top - 1) __syncthreads();  // the single staging slot is free again
      pf_put(n);
    } else if (n < n_top - 1) {
      __syncthreads();  // the single staging slot is free again
      issue(n);
    }

    // ---- S0 (transposed, and row unless LEAN) as bf16 operands; G^T follows the gate
#pragma unroll
    for (int m = 0; m < (FIN ? STW : 0); ++m) {
      const int u = wave + NW * m;
      if (u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
        const int e = et * 16 + r16;
        T sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool in = FULLK && FULLV ? true : (ct * 16 + g4 * 4 + i < dk && e < dv);
          sv[i] = from_f<T>(in ? s0c[m][i] : 0.f);
          if constexpr (!LEAN) sS0[(ct * 16 + g4 * 4 + i) * VP + e] = sv[i];
        }
        lds_row_write<T, 4>(sS0t + e * QP, ct * 16 + g4 * 4, sv);
      }
    }
    if constexpr (!PF) dma_wait();
    __syncthreads();
    // the reading final pass: this chunk's dO fragments and diagonal from pass A (consumed in
    // the recompute phase, after the gate phase has covered their latency)
    Quad<T> dofr[RD ? RNDVH : 1];
    float dgw = 0.f;
    // the passes that form dO: this chunk's normalised output o rstd and rstd as the forward
    // saved them (the recompute phase's row tile I, value tiles E0.. of half hh)
    Quad<float> obr[RD ? 1 : RNDVH];
    float4 rsv = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (LBPF) {
#pragma unroll
      for (int Eh = 0; Eh < RNDVH; ++Eh) obr[Eh] = obr_lb[Eh];
      rsv = rsv_lb;
    } else if constexpr (!RD) {
      const int I = wave % NT, E0 = (wave / NT) * RNDVH;
      const Quad<float>* ob = static_cast<const Quad<float>*>(p.obar) + ((sbase + n) * NT + I) * NDV * 64 + lane;
#pragma unroll
      for (int Eh = 0; Eh < RNDVH; ++Eh) obr[Eh] = ob[min(E0 + Eh, NDV - 1) * 64];
      rsv = *reinterpret_cast<const float4*>(p.rstd + (sbase + n) * C + 16 * I + 4 * g4);
    }
    if constexpr (RD) {
      const Quad<T>* fb = static_cast<const Quad<T>*>(p.dofrag) +
                          ((sbase + n) * NW + wave) * RNDVH * 64 + lane;
#pragma unroll
      for (int Eh = 0; Eh < RNDVH; ++Eh) dofr[Eh] = fb[Eh * 64];
      dgw = p.diagws[(sbase + n) * 2 * C + min(tid, 2 * C - 1)];
    }
    f32x4 s0p[STW];  // prefetch S0 of the next chunk down (consumed at the next top)
    // the next chunk's rows and S0 are loaded after the gate phase: issued here, in one burst
    // with the loads above from every wave, they held the gate phase up
    // Issued on every chunk (the last one loads its own chunk again, unused): fixed load counts
    // keep the compiler's waits for the loads issued before exact, where a conditional
    // prefetch made them wait for everything outstanding, the prefetch included.
    auto prefetch_next = [&]() {
      if constexpr (!LB) {  // (the look-back's workgroups hold one chunk)
        const int nn = max(n - 1, c_first);
        if constexpr (PF) pf_load(nn);
        if constexpr (FIN) load_state(nn, s0p);
      }
    };

    // ---------------------------------------------------------------- gate phase
    {
      const bool tv = tg < valid;
      T zr[NCL], kr[NCL], qr[NCL], vr[NEL];
      float zf[NCL], bb[NCL], bl[NCL];  // gate logits, log2 gates
      if constexpr (LR) {  // formed and turned into log gates before the other rows are read
        lowrank_logits<DKP, NCL>(zf, rawf + tg * ZPE, smem + Lo::O_ZT, c0);
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
          const bool on = FULLK ? tv : (tv && c0 + j < dk);
          bb[j] = keep_if(on, Fm<T>::lsig2(zf[j]) * inv_tau);
          pin(bb[j]);
        }
        // sigmoid(-z) for dz, in the z rows (which stage nothing else until dz replaces it)
        if constexpr (FIN) {
#pragma unroll
          for (int j = 0; j < NCL; ++j)
            if (FULLK || c0 + j < dk) rawz[tg * kp + c0 + j] = from_f<T>(Fm<T>::sig(-zf[j]));
        }
      } else if constexpr (FULLK) {
        lds_row_read_k<T, NCL, KPE>(zr, rawz + tg * KPE, c0, tv);
      } else {
        lds_row_read<T, NCL>(zr, rawz + tg * kp, c0, dk, tv, kp);
      }
      if constexpr (FULLK) {
        if constexpr (FIN) lds_row_read_k<T, NCL, KPE>(kr, rawk + tg * KPE, c0, tv);
        lds_row_read_k<T, NCL, KPE>(qr, rawq + tg * KPE, c0, tv);
      } else {
        if constexpr (FIN) lds_row_read<T, NCL>(kr, rawk + tg * kp, c0, dk, tv, kp);
        lds_row_read<T, NCL>(qr, rawq + tg * kp, c0, dk, tv, kp);
      }
      if constexpr (FULLV) lds_row_read_k<T, NEL, VPE>(vr, rawv + tg * VPE, e0, tv);
      else lds_row_read<T, NEL>(vr, rawv + tg * vp, e0, dv, tv, vp);
      if constexpr (!LR) {
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
          const bool on = FULLK ? tv : (tv && c0 + j < dk);
          bb[j] = keep_if(on, Fm<T>::lsig2(to_f(zr[j])) * inv_tau);
        }
      }

#pragma unroll
      for (int j = 0; j < NCL; ++j) bb[j] = scan_dpp<C>(bb[j]);
#pragma unroll
      for (int j = 0; j < NCL; ++j) bl[j] = group_last<C>(bb[j], lane);
      float qf[NCL], kf[NCL];
      T qs[NCL], ks[NCL];
#pragma unroll
      for (int j = 0; j < NCL; ++j) {
        qf[j] = to_f(qr[j]) * p.q_scale * Fm<T>::exp2(bb[j]);
        qs[j] = from_f<T>(qf[j]);
        if constexpr (FIN) {
          kf[j] = to_f(kr[j]) * Fm<T>::exp2(-bb[j]);
          ks[j] = from_f<T>(kf[j]);
        }
      }
      float md = 0.f;
#pragma unroll
      for (int j = 0; j < NCL; ++j) md = fmaxf(md, -bl[j]);
      md = wave_max_dpp(md);

      if (FIN && c0 < QKC) {  // a lane's column run lies wholly inside or past the stored
                              // columns (fp32 q e^b, k e^-b: the split products of P)
        lds_row_write<float, NCL>(sQ + tg * QKP, c0, qf);
        lds_row_write<float, NCL>(sK + tg * QKP, c0, kf);
      }
      if constexpr (NEL * (NTH / C) == DVP) {
        lds_row_write<T, NEL>(sV + tg * VP, e0, vr);
      } else {  // more column groups than value columns (short chunks): up to the tiles' end
#pragma unroll
        for (int j = 0; j < NEL; ++j)
          if (e0 + j < DVP) sV[tg * VP + e0 + j] = vr[j];
      }
#pragma unroll
      for (int j = 0; j < NCL; ++j) {
        if ((FULLK && !KOVER) || c0 + j < DKP) {  // (groups past the key tiles: nothing)
          sQt[(c0 + j) * TP + tg] = qs[j];
          if constexpr (FIN) sKt[(c0 + j) * TP + tg] = ks[j];
        }
        if (FIN && (FULLK || c0 + j < dk)) sB[tg * DKB + c0 + j] = bb[j];
      }
      if (lane == 0) sMax[wave] = md;
      if (tg == C - 1) {
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
          if (!KOVER || c0 + j < DKP) {
            sGam[c0 + j] = Fm<T>::exp2(bl[j]);
            if (FIN)
              sLg[c0 + j] = bl[j];  // this chunk's log2 decay, for the e^{b_last - b} factors
            else
              sLg[c0 + j] += bl[j];  // segment's log2 decay
          }
        }
      }
    }
    __syncthreads();
    prefetch_next();
    float mxa = sMax[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) mxa = fmaxf(mxa, sMax[w]);
    const bool slow = mxa > kBwdSlowDecayLog2;

    // G^T as (e^{b_last} G)^T: it enters dv as k e^{-b} (e^{b_last} G) and dk as
    // e^{-b} V (e^{b_last} G)^T; with strong decay (elementwise paths) G itself
    auto write_gt = [&]() {
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        const int u = wave + NW * m;
        if (u < NST) {
          const int ct = u / NDV, et = u - ct * NDV;
          const int e = et * 16 + r16;
          const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + ct * 16 + g4 * 4);
          T gv4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) gv4[i] = from_f<T>(slow ? gacc[m][i] : gacc[m][i] * gam[i]);
          lds_row_write<T, 4>(sGt + e * QP, ct * 16 + g4 * 4, gv4);
        }
      }
    };
    if (own && !LB) write_gt();  // the look-back writes it once G is known

    // ------------------------------------------------------------ recompute phase
    // Row tile I = wave % NT; with at least twice as many waves as row tiles, the two waves
    // of a row tile split its value tiles (half h = wave / NT) and exchange the RMSNorm row
    // sums through LDS (two extra barriers); the gated Q K^T tile is formed by both.
    constexpr int SPL = NW >= 2 * NT ? 2 : 1;
    constexpr int NDVH = (NDV + SPL - 1) / SPL;            // value tiles per half
    const bool part = wave < NT * SPL;
    const int I = wave % NT, hh = wave / NT;
    const int E0 = hh * NDVH;
    f32x4 pt[NT];  // pt[J][i] = P[16I + r16][16J + 4 g4 + i]
    f32x4 oacc[NDVH];
    T rr[NDVH][4], dyr[NDVH][4];
    float ss[4] = {0.f, 0.f, 0.f, 0.f}, md[4] = {0.f, 0.f, 0.f, 0.f}, rstd[4];
    float dn[NDVH][4];
    if (FIN && slow) {  // strong decay: P rows elementwise, one copy per row tile (uniform branch)
      if (part && hh == 0) {
        T* sPw = sSlow + I * 16 * C;
        for (int idx = lane; idx < 16 * C; idx += 64) {
          const int rq = idx / C, j = idx - rq * C, ir = 16 * I + rq;
          float acc = 0.f;
          if (j <= ir && ir < valid) {
#pragma unroll 1
            for (int c = 0; c < dk; ++c)
              acc += to_f(rawq[ir * kp + c]) * to_f(rawk[j * kp + c]) *
                     Fm<T>::exp2(sB[ir * DKB + c] - sB[j * DKB + c]);
            acc *= p.q_scale;
          }
          sPw[idx] = from_f<T>(acc);
        }
      }
      __syncthreads();
    }
    // the reading final pass needs P only for P^T (dv): where two waves share a row tile they
    // form alternate column tiles of it; the recomputing passes need whole rows (o = P V)
    auto mine = [&](int J) { return !RD || SPL == 1 || (J & 1) == hh; };
    if (part) {
      if constexpr (FIN) {  // P (for dv) in the final pass only
      float diag = 0.f;  // exact q_i.k_i from the unscaled inputs (gate factor 1)
      if (mine(I)) {
        constexpr int DQ = DKP / 4;
        const int ir = 16 * I + r16;
        T qd[DQ], kd[DQ];
        if constexpr (FULLK) {
          lds_row_read_k<T, DQ, KPE>(qd, rawq + ir * KPE, g4 * DQ, true);
          lds_row_read_k<T, DQ, KPE>(kd, rawk + ir * KPE, g4 * DQ, true);
        } else {
          lds_row_read<T, DQ>(qd, rawq + ir * kp, g4 * DQ, dk, true, kp);
          lds_row_read<T, DQ>(kd, rawk + ir * kp, g4 * DQ, dk, true, kp);
        }
        Acc acc = 0;
#pragma unroll
        for (int j = 0; j < DQ; ++j) acc += (Acc)to_f(qd[j]) * (Acc)to_f(kd[j]);
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        // rows past the sequence end hold stale staging data: they must stay exactly zero
        diag = ir < valid ? (float)acc * p.q_scale : 0.f;
      }
      if (!slow) {
        // bf16 I/O: split operands (dv takes P_ij times do_i, which is large where rstd_i is,
        // so P_ij is needed to the accuracy of its own magnitude there); the row tile's side
        // is split once for every column tile
        if constexpr (kBf) {
          const auto bq = split_b<QKC, QKP>(sQ, 16 * I, lane);
#pragma unroll
          for (int J = 0; J < NT; ++J)
            pt[J] = J <= I && mine(J) ? mm_split_pre<QKC, QKP, QKP>(zero4(), sK, 16 * J, bq, lane)
                                      : zero4();
        } else {
#pragma unroll
          for (int J = 0; J < NT; ++J)
            pt[J] = J <= I && mine(J) ? Mma<T>::kc(zero4(), sK, QKP, 16 * J, sQ, QKP, 16 * I, DKP, lane)
                                      : zero4();
        }
      } else {
        const T* sPw = sSlow + I * 16 * C;
#pragma unroll
        for (int J = 0; J < NT; ++J)
#pragma unroll
          for (int i = 0; i < 4; ++i) pt[J][i] = to_f(sPw[r16 * C + 16 * J + 4 * g4 + i]);
      }
#pragma unroll
      for (int J = 0; J < NT; ++J) {
        if (J == I) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (4 * g4 + i > r16) pt[J][i] = 0.f;
            if (4 * g4 + i == r16) pt[J][i] = diag;
          }
        }
        if (own && (RD ? mine(J) : hh == 0) && J <= I) {  // P^T for dv (tiles above the
                                                           // diagonal stay zero)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sPt[(16 * J + 4 * g4 + i) * TP + 16 * I + r16] = from_f<T>(pt[J][i]);
        }
      }
      }  // FIN
      if constexpr (!RD) {  // the reading final pass skips the output-stage backward
      // o rstd as the forward saved it (its rows are the rows of this tile); rows past the
      // sequence end hold whatever the forward formed from stale staging rows: zero here
#pragma unroll
      for (int Eh = 0; Eh < NDVH; ++Eh)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[Eh][i] = 16 * I + 4 * g4 + i < valid ? obr[Eh].v[i] : 0.f;

      // output-stage backward: r, dy first (one LDS round trip); value tiles past this
      // half's range (an odd tile count) count as zero columns.  Register-staged bf16 rows
      // (pitch a multiple of 4): a tile whose 16 columns all lie inside the row comes through
      // the transpose load (the lane's four rows of its column in one 8-byte read)
#pragma unroll
      for (int Eh = 0; Eh < NDVH; ++Eh) {
        if constexpr (kBf && PF) {
          if (16 * (E0 + Eh) + 16 <= DV) {
            const bf16x4 r4 = lds_tr4(sRr, RPE, 16 * (E0 + Eh), 16 * I + 4 * g4, r16);
            const bf16x4 y4 = lds_tr4(sDy, RPE, 16 * (E0 + Eh), 16 * I + 4 * g4, r16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool on = 16 * I + 4 * g4 + i < valid;  // stale rows: 0
              rr[Eh][i] = on ? r4[i] : from_f<T>(0.f);
              dyr[Eh][i] = on ? y4[i] : from_f<T>(0.f);
            }
            continue;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = (E0 + Eh) * 16 + r16, row = 16 * I + 4 * g4 + i;
          const bool on = E0 + Eh < NDV && (FULLV || e < dv) && row < valid;  // stale rows: 0
          rr[Eh][i] = on ? sRr[row * rp + e] : from_f<T>(0.f);
          dyr[Eh][i] = on ? sDy[row * rp + e] : from_f<T>(0.f);
          if (E0 + Eh >= NDV) oacc[Eh][i] = 0.f;
        }
      }
      }  // !RD
    }
    if (part && !RD) {
      rstd[0] = rsv.x; rstd[1] = rsv.y; rstd[2] = rsv.z; rstd[3] = rsv.w;
#pragma unroll
      for (int i = 0; i < 4; ++i)  // (rows past the sequence end: see oacc)
        if (16 * I + 4 * g4 + i >= valid) rstd[i] = 0.f;
      // oacc is the normalised output, dn = dy * w * swish(r)
#pragma unroll
      for (int Eh = 0; Eh < NDVH; ++Eh) {
        const int E = min(E0 + Eh, NDV - 1), e = (E0 + Eh) * 16 + r16;
        const bool col_on = E0 + Eh < NDV && (FULLV || e < dv);
        float gmE = gm[0];
#pragma unroll
        for (int k = 1; k < NDV; ++k) gmE = k == E ? gm[k] : gmE;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * I + 4 * g4 + i;
          const float nv = oacc[Eh][i], rv = to_f(rr[Eh][i]), dyv = to_f(dyr[Eh][i]);
          const float sg = Fm<T>::sig(rv), sw = rv * sg;
          if (col_on) {
            if (dg_here) dgl[Eh] += dyv * nv * sw;
            if (own || RU) sRr[row * rp + e] = from_f<T>(dyv * nv * gmE * sg * (1.f + rv * (1.f - sg)));
          }
          dn[Eh][i] = dyv * gmE * sw;
          md[i] += dn[Eh][i] * nv;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) md[i] = row_sum16(md[i]);
      if constexpr (SPL > 1) {
        if (r16 == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sXch[(2 + hh) * C + 16 * I + 4 * g4 + i] = md[i];
        }
      }
    }
    if constexpr (SPL > 1 && !RD) __syncthreads();  // dn.o row sums of both halves
    if (part && RD) {
      // dO and the dO.v diagonal as pass A formed them
#pragma unroll
      for (int Eh = 0; Eh < NDVH; ++Eh) {
        if (E0 + Eh < NDV) {
          const int e = (E0 + Eh) * 16 + r16;
          T dov4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dov4[i] = dofr[Eh].v[i];
            if constexpr (!LEAN) sdO[(16 * I + 4 * g4 + i) * VP + e] = dov4[i];
          }
          lds_row_write<T, 4>(sdOt + e * TP, 16 * I + 4 * g4, dov4);
        }
      }
      if (tid < 2 * C) sDiag[tid] = dgw;
    } else if (part) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float tot = md[i];
        if constexpr (SPL > 1) {
          const int row = 16 * I + 4 * g4 + i;
          tot = sXch[2 * C + row] + sXch[3 * C + row];
        }
        md[i] = tot / (float)dv;
      }
      Acc dvd[4] = {0, 0, 0, 0};
      Quad<T> dof[NDVH];  // pass A with reuse: dO in fragment order for the final pass
#pragma unroll
      for (int Eh = 0; Eh < NDVH; ++Eh) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dof[Eh].v[i] = from_f<T>(0.f);
        if (E0 + Eh < NDV) {
          const int e = (E0 + Eh) * 16 + r16;
          T dov4[4], v4[4];
          if constexpr (kBf) {  // the lane's four rows of v in one transpose load
            const bf16x4 t4 = lds_tr4(reinterpret_cast<const bf16*>(sV), VP, 16 * (E0 + Eh),
                                      16 * I + 4 * g4, r16);
#pragma unroll
            for (int i = 0; i < 4; ++i) v4[i] = t4[i];
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v4[i] = sV[(16 * I + 4 * g4 + i) * VP + e];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * I + 4 * g4 + i;
            const float dov =
                (FULLV || e < dv) ? rstd[i] * (dn[Eh][i] - oacc[Eh][i] * md[i]) : 0.f;
            dov4[i] = from_f<T>(dov);
            dof[Eh].v[i] = dov4[i];
            if constexpr (!LEAN && FIN) sdO[row * VP + e] = dov4[i];  // for D = dO V^T
            dvd[i] += (Acc)dov * (Acc)to_f(v4[i]);
          }
          lds_row_write<T, 4>(sdOt + e * TP, 16 * I + 4 * g4, dov4);
        }
      }
      if constexpr (RU && !FIN) {
        Quad<T>* fb = static_cast<Quad<T>*>(p.dofrag) + ((sbase + n) * NW + wave) * NDVH * 64 + lane;
#pragma unroll
        for (int Eh = 0; Eh < NDVH; ++Eh) fb[Eh * 64] = dof[Eh];
      }
      // do_i is orthogonal to the normalised o_i (up to eps); when o_i is parallel to v_i
      // (the first token) do_i.v_i cancels, so it is formed here from the fp32 do_i; the
      // halves' partial sums are added where the diagonal is used
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Acc dd = dvd[i];
        if constexpr (kBf) {
          dd = row_sum16(dd);  // DPP within the row of 16 lanes (no LDS permute)
        } else {
          dd += __shfl_xor(dd, 1);
          dd += __shfl_xor(dd, 2);
          dd += __shfl_xor(dd, 4);
          dd += __shfl_xor(dd, 8);
        }
        if ((own || RU) && r16 == 0) sDiag[hh * C + 16 * I + 4 * g4 + i] = (float)dd;
      }
    }
    if constexpr (LB) {  // the dgamma partial is complete: per-wave sums
#pragma unroll
      for (int E = 0; E < NDV; ++E) {
        float v = dgam_of(E);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (g4 == 0) sDg[wave * DVP + E * 16 + r16] = v;
      }
    }
    __syncthreads();
    if constexpr (RU && !FIN) {
      if (tid < 2 * C) p.diagws[(sbase + n) * 2 * C + tid] = sDiag[tid];
    }
    if constexpr (LB) {
      // publish this chunk's U = (q e^b)^T dO, its log2 decay and the dgamma partial (the
      // flag follows the D phase, which covers the stores' latency)
      const long slot = (long)bh * p.nseg + seg;
      float* dst = p.gstates + slot * dk * dv;
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        const int u = wave + NW * m;
        if (u < NST) {
          const int ct = u / NDV, et = u - ct * NDV;
          const f32x4 ua = Mma<T>::kc(zero4(), sQt, TP, 16 * ct, sdOt, TP, 16 * et, C, lane);
          const int e = et * 16 + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = ct * 16 + g4 * 4 + i;
            if ((FULLK || c < dk) && (FULLV || e < dv)) st_dev(dst + c * dv + e, ua[i]);
          }
        }
      }
      for (int c = tid; c < dk; c += NTH) st_dev(p.seg_lg + slot * dk + c, sLg[c]);
      for (int e = tid; e < dv; e += NTH) {
        float sum = sDg[e];  // waves in order
        for (int w = 1; w < NW; ++w) sum += sDg[w * DVP + e];
        st_dev(p.dgamma_part + (long)blockIdx.x * dv + e, sum);
      }
    }

    if (own) {
      // ---- D = dO V^T (causal, row and transposed) and the dlog(alpha) boundary term
      for (int q = wave; q < NT * NT; q += NW) {
        const int I = q / NT, J = q - I * NT;
        if (J <= I) {
          f32x4 d;
          if constexpr (LEAN)
            d = Mma<T>::template mm<false, true>(zero4(), sdOt, TP, 16 * I, sV, VP, 16 * J, DVP,
                                                 lane);
          else
            d = Mma<T>::kc(zero4(), sdO, VP, 16 * I, sV, VP, 16 * J, DVP, lane);
          T dt4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ii = 16 * I + 4 * g4 + i, jj = 16 * J + r16;
            const float dg = NW >= 2 * NT ? sDiag[ii] + sDiag[C + ii] : sDiag[ii];
            dt4[i] = from_f<T>(jj < ii ? d[i] : (jj == ii ? dg : 0.f));
            if constexpr (!LEAN) sD[ii * TP + jj] = dt4[i];
          }
          lds_row_write<T, 4>(sDt + (16 * J + r16) * TP, 16 * I + 4 * g4, dt4);
        }
      }
      if constexpr (LB) __builtin_amdgcn_s_waitcnt(0);  // the values published above are out
      __syncthreads();
      if constexpr (LB) {
        const long slot0 = (long)bh * p.nseg;
        if (tid == 0)
          __hip_atomic_store(p.lb_flag + slot0 + seg, p.lb_tag, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        // G reaching this chunk's end: the later chunks' U, each decayed by the chunks
        // between (gacc is zero here)
        float fac[STW][4];
#pragma unroll
        for (int m = 0; m < STW; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) fac[m][i] = 1.f;
        const bool expired =
            lb_wait_all(p.lb_flag + slot0 + seg + 1, p.nseg - 1 - seg, p.lb_wait_tag, lane, p.lb_spins);
        // LBU later segments per step, their loads in flight together (a step past the
        // last segment re-reads it and adds nothing)
        constexpr int LBU = STW == 1 ? 4 : 1;
        for (int s0 = seg + 1; s0 < p.nseg; s0 += LBU) {
          float uv[LBU][STW][4], gv[LBU][STW][4];
#pragma unroll
          for (int a = 0; a < LBU; ++a) {
            const long sl = slot0 + min(s0 + a, p.nseg - 1);
            const float* src = p.gstates + sl * dk * dv;
            const float* lg = p.seg_lg + sl * dk;
#pragma unroll
            for (int m = 0; m < STW; ++m) {
              const int u = min(wave + NW * m, NST - 1);
              const int ct = u / NDV, et = u - ct * NDV;
              const int e = min(et * 16 + r16, dv - 1);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int c = min(ct * 16 + g4 * 4 + i, dk - 1);
                uv[a][m][i] = ld_dev(src + c * dv + e);
                gv[a][m][i] = ld_dev(lg + c);
              }
            }
          }
#pragma unroll
          for (int a = 0; a < LBU; ++a) {
            const bool on = s0 + a < p.nseg;
#pragma unroll
            for (int m = 0; m < STW; ++m) {
              const int u = wave + NW * m;
              const int ct = u / NDV, et = u - ct * NDV;
              const int e = et * 16 + r16;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int c = ct * 16 + g4 * 4 + i;
                const bool in = on && u < NST && (FULLK || c < dk) && (FULLV || e < dv);
                gacc[m][i] += in ? fac[m][i] * uv[a][m][i] : 0.f;
                fac[m][i] *= on ? Fm<T>::exp2(gv[a][m][i]) : 1.f;
              }
            }
          }
        }
        if (expired) {  // a later chunk's contribution never arrived: poison G, record it
#pragma unroll
          for (int m = 0; m < STW; ++m) gacc[m] = f32x4{__builtin_nanf(""), __builtin_nanf(""),
                                                        __builtin_nanf(""), __builtin_nanf("")};
          if (lane == 0) lb_fail(p.lb_status);
        }
        write_gt();
        if (n_top < p.NC) {
          if constexpr (STW > 1) load_state(n_top, se_lb);
          write_part(se_lb);
        }
        __syncthreads();
        if (tid == 0) lb_raise(p.lb_flag + (long)gridDim.x + slot0 + seg, p.lb_tag);  // done
      }

      // ---- dq, dk, q.dq - k.dk (staged as soon as each (row tile, key tile) pair is done:
      // dq | dk over the raw v rows, which are no longer read) and dv (over dy, read only in
      // the recompute phase)
#pragma unroll
      for (int m = 0; m < PRW; ++m) {
        // one pair at a time: keeps later pairs' operand fragments from being hoisted
        __builtin_amdgcn_sched_barrier(0);
        const int u = wave + NW * m;
        if (u < NPAIR) {
          const int I = u / NDK, ct = u - I * NDK;
          f32x4 a1, a2 = zero4(), a4 = zero4();
          if constexpr (LEAN)
            a1 = Mma<T>::template mm<false, false>(zero4(), sdOt, TP, 16 * I, sS0t, QP, 16 * ct,
                                                   DVP, lane);
          else
            a1 = Mma<T>::kc(zero4(), sdO, VP, 16 * I, sS0, VP, 16 * ct, DVP, lane);
          const f32x4 a3 = Mma<T>::template mm<true, false>(zero4(), sV, VP, 16 * I, sGt, QP,
                                                            16 * ct, DVP, lane);
          if (!slow) {
            if constexpr (LEAN)
              a2 = Mma<T>::template mm<false, true>(zero4(), sDt, TP, 16 * I, sKt, TP, 16 * ct, C,
                                                    lane);
            else
              a2 = Mma<T>::kc(zero4(), sD, TP, 16 * I, sKt, TP, 16 * ct, C, lane);
            a4 = Mma<T>::kc(zero4(), sDt, TP, 16 * I, sQt, TP, 16 * ct, C, lane);
          }
          const int c = ct * 16 + r16;
          if (FULLK || c < dk) {
            const float blast = sLg[c];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = 16 * I + 4 * g4 + i;
              const float bt = sB[t * DKB + c];
              float dq, dkk;
              if (!slow) {  // a3 holds V (e^{b_last} G)^T here
                dq = Fm<T>::exp2(bt) * (a1[i] + a2[i]);
                dkk = Fm<T>::exp2(-bt) * (a4[i] + a3[i]);
              } else {  // a3 holds V G^T here
                float s1 = 0.f, s2 = 0.f;
#pragma unroll 1
                for (int j = 0; j <= t && j < valid; ++j)
                  s1 += to_f(LEAN ? sDt[j * TP + t] : sD[t * TP + j]) * to_f(rawk[j * kp + c]) *
                        Fm<T>::exp2(bt - sB[j * DKB + c]);
#pragma unroll 1
                for (int i2 = t; i2 < valid; ++i2)
                  s2 += to_f(sDt[t * TP + i2]) * to_f(rawq[i2 * kp + c]) * p.q_scale *
                        Fm<T>::exp2(sB[i2 * DKB + c] - bt);
                dq = Fm<T>::exp2(bt) * a1[i] + s1;
                dkk = s2 + Fm<T>::exp2(blast - bt) * a3[i];
              }
              const float qf = to_f(rawq[t * kp + c]) * p.q_scale, kf = to_f(rawk[t * kp + c]);
              sW[t * DKB + c] = qf * dq - kf * dkk;
              sdqs[t * kp + c] = from_f<T>(p.q_scale * dq);
              sdks[t * kp + c] = from_f<T>(dkk);
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < DVW; ++m) {
        __builtin_amdgcn_sched_barrier(0);
        const int u = wave + NW * m;
        if (u < NDVT) {
          const int J = u / NDV, et = u - J * NDV;
          f32x4 dva = Mma<T>::kc(zero4(), sPt, TP, 16 * J, sdOt, TP, 16 * et, C, lane);
          const int e = et * 16 + r16;
          if (!slow) {
            if constexpr (kBf)
              dva = mm_split_b<QKC, QKP, QP>(dva, sK, 16 * J, sGt, 16 * et, lane);
            else
              dva = Mma<T>::kc(dva, sK, QKP, 16 * J, sGt, QP, 16 * et, DKP, lane);
          } else {  // k_j e^{b_last - b_j} G elementwise (no overflow)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 16 * J + 4 * g4 + i;
              float acc = 0.f;
#pragma unroll 1
              for (int c = 0; c < dk; ++c)
                acc += to_f(rawk[j * kp + c]) * Fm<T>::exp2(sLg[c] - sB[j * DKB + c]) *
                       to_f(sGt[e * QP + c]);
              dva[i] += acc;
            }
          }
          if (FULLV || e < dv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sDy[(16 * J + 4 * g4 + i) * rp + e] = from_f<T>(dva[i]);
          }
        }
      }
    }

    // gradient state: G <- diag(e^{b_last}) G + (q e^{b})^T dO (the look-back's single chunk
    // has no chunk below it)
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave + NW * m;
      if (!LB && u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
        const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + ct * 16 + g4 * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) gacc[m][i] *= gam[i];
        gacc[m] = Mma<T>::kc(gacc[m], sQt, TP, 16 * ct, sdOt, TP, 16 * et, C, lane);
      }
    }
    __syncthreads();
    if constexpr (RU && !FIN) {  // pass A emits dr (the reading final pass has no r)
      T* gdr = static_cast<T*>(p.dr);
      if constexpr (PF) {
        constexpr int RV = DV * (int)sizeof(T), LV = RPE * (int)sizeof(T);
        store_rows_fixed<RV, C, NTH, LV>(reinterpret_cast<unsigned char*>(gdr + row0 * DV),
                                         (long)H * RV, reinterpret_cast<const unsigned char*>(sRr),
                                         valid, tid);
      } else {
        store_rows<T>(gdr + row0 * dv, (long)H * dv, sRr, dv, valid, dv, tid, NTH);
      }
    }

    if (own) {
      if constexpr (PF) {
        // dq, dk, dv (and dr) are complete in LDS (the barrier above): their stores go out
        // first and overlap the dlog(alpha) phase, which writes only the z rows
        T* gdq = static_cast<T*>(p.dq);
        T* gdk = static_cast<T*>(p.dk_);
        T* gdv = static_cast<T*>(p.dv_);
        T* gdr = static_cast<T*>(p.dr);
        constexpr int RK = DK * (int)sizeof(T), RV = DV * (int)sizeof(T);
        using UC = unsigned char;
        constexpr int LK = KPE * (int)sizeof(T), LV = RPE * (int)sizeof(T);
        store_rows_fixed<RK, C, NTH, LK>(reinterpret_cast<UC*>(gdq + row0 * DK), (long)H * RK,
                                         reinterpret_cast<const UC*>(sdqs), valid, tid);
        store_rows_fixed<RK, C, NTH, LK>(reinterpret_cast<UC*>(gdk + row0 * DK), (long)H * RK,
                                         reinterpret_cast<const UC*>(sdks), valid, tid);
        store_rows_fixed<RV, C, NTH, LV>(reinterpret_cast<UC*>(gdv + row0 * DV), (long)H * RV,
                                         reinterpret_cast<const UC*>(sDy), valid, tid);
        if constexpr (!RD)
          store_rows_fixed<RV, C, NTH, LV>(reinterpret_cast<UC*>(gdr + row0 * DV), (long)H * RV,
                                           reinterpret_cast<const UC*>(sRr), valid, tid);
      }
      // ---- dlog(alpha) = suffix sums of q.dq - k.dk (lanes = tokens in reverse order, DPP
      // prefix scan) + the boundary term; dz = dlog(alpha) sigmoid(-z) / tau, over raw z
      const int tr = C - 1 - tg;
      const bool tv = tr < valid;
      float w[NCL], zg[NCL];  // q.dq - k.dk; z (low-rank gate: sigmoid(-z), from the gate pass)
#pragma unroll
      for (int j = 0; j < NCL; ++j) {
        const int c = c0 + j;
        const bool on = tv && (FULLK || c < dk);
        w[j] = on ? sW[tr * DKB + c] : 0.f;
        zg[j] = on ? to_f(rawz[tr * kp + c]) : 0.f;
      }
      float bterm[NCL];
#pragma unroll
      for (int j = 0; j < NCL; ++j) {
        float s = 0.f;
#pragma unroll
        for (int et = 0; et < NDV; ++et) s += sPart[(c0 + j) * 8 + et];  // one row of 8
        bterm[j] = s;
      }
#pragma unroll
      for (int j = 0; j < NCL; ++j) w[j] = scan_dpp<C>(w[j]);
#pragma unroll
      for (int j = 0; j < NCL; ++j) {
        const int c = c0 + j;
        if (tv && (FULLK || c < dk)) {
          float dla = w[j] + bterm[j];
          if (n == 0 && tr == 0) dla = 0.f;  // alpha_0 multiplies the zero initial state
          const float sgm = LR ? zg[j] : Fm<T>::sig(-zg[j]);
          rawz[tr * kp + c] = from_f<T>(dla * sgm * inv_tau);
        }
      }
      __syncthreads();
      T* gdz = static_cast<T*>(p.dz);
      T* gdq = static_cast<T*>(p.dq);
      T* gdk = static_cast<T*>(p.dk_);
      T* gdv = static_cast<T*>(p.dv_);
      T* gdr = static_cast<T*>(p.dr);
      if constexpr (PF) {
        constexpr int RK = DK * (int)sizeof(T);
        using UC = unsigned char;
        constexpr int LK = KPE * (int)sizeof(T);
        store_rows_fixed<RK, C, NTH, LK>(reinterpret_cast<UC*>(gdz + row0 * DK), (long)H * RK,
                                         reinterpret_cast<const UC*>(rawz), valid, tid);
      } else {
        store_rows<T>(gdq + row0 * dk, (long)H * dk, sdqs, dk, valid, dk, tid, NTH);
        store_rows<T>(gdk + row0 * dk, (long)H * dk, sdks, dk, valid, dk, tid, NTH);
        store_rows<T>(gdz + row0 * dk, (long)H * dk, rawz, dk, valid, dk, tid, NTH);
        store_rows<T>(gdv + row0 * dv, (long)H * dv, sDy, dv, valid, dv, tid, NTH);
        if constexpr (!RD) store_rows<T>(gdr + row0 * dv, (long)H * dv, sRr, dv, valid, dv, tid, NTH);
      }
    }
    // one chunk down: its boundary term (this chunk's S0 is its S_end, G is updated), and
    // its S0 (read by nobody before the next top barrier; sPart's last reader, this chunk's
    // dlog phase, is behind the barrier above)
    if (FIN && !LB && n > c_first) {
      write_part(s0c);
#pragma unroll
      for (int m = 0; m < STW; ++m) s0c[m] = s0p[m];
    }
  }

  if (dg_here && !LB) {
    // per-workgroup partial of dgamma, reduced in a fixed order by a later kernel
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      float v = dgam_of(E);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (g4 == 0) sDg[wave * DVP + E * 16 + r16] = v;
    }
    __syncthreads();
    for (int e = tid; e < dv; e += NTH) {
      float sum = sDg[e];  // waves in order (waves past the row tiles add exact zeros)
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += sDg[w * DVP + e];
      p.dgamma_part[((long)bh * p.nseg + seg) * dv + e] = sum;
    }
  }
  if (!FIN) {
    float* dst = p.gstates + ((long)bh * p.nseg + seg) * dk * dv;
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave + NW * m;
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
    __syncthreads();
    for (int c = tid; c < dk; c += NTH)
      p.seg_lg[((long)bh * p.nseg + seg) * dk + c] = sLg[c];
  }
  if constexpr (LB) {
    // the last workgroup: once every workgroup is done with its waits (each had published
    // before), d_norm_w = the partials added in a fixed order (parts strided over NG groups per
    // column, then the groups in order), and the flags are cleared for the next launch
    bool partial = false;  // some workgroup's done flag never arrived
    if (blockIdx.x == gridDim.x - 1) {
      const int nparts = (int)gridDim.x;
      const bool ex = lb_wait_each(p.lb_flag + nparts, nparts, p.lb_wait_tag, tid, NTH, p.lb_spins);
      if (ex) lb_fail(p.lb_status);
      partial = __syncthreads_or(ex) != 0;
      for (int i = tid; i < 2 * nparts; i += NTH) lb_raise(p.lb_flag + i, 0u);
    }
    if (p.d_norm_w && blockIdx.x == gridDim.x - 1) {
      const int nparts = (int)gridDim.x;
      constexpr int NG = NTH / DVP < NW ? NTH / DVP : NW;
      const int g = tid / DVP, e = tid - g * DVP;
      if (g < NG && e < dv) {
        // parts g, g + NG, ... in increasing order, eight loads in flight at a time
        constexpr int U8 = 8;
        float sum = 0.f;
        for (int i0 = g; i0 < nparts; i0 += U8 * NG) {
          float v8[U8];
#pragma unroll
          for (int j = 0; j < U8; ++j)
            v8[j] = ld_dev(p.dgamma_part + (long)min(i0 + j * NG, nparts - 1) * dv + e);
#pragma unroll
          for (int j = 0; j < U8; ++j) sum += i0 + j * NG < nparts ? v8[j] : 0.f;
        }
        sDg[g * DVP + e] = sum;
      }
      __syncthreads();
      for (int e2 = tid; e2 < dv; e2 += NTH) {
        float sum = sDg[e2];
#pragma unroll
        for (int g2 = 1; g2 < NG; ++g2) sum += sDg[g2 * DVP + e2];
        p.d_norm_w[e2] = partial ? __builtin_nanf("") : sum;
      }
    }
  }
}

// Waves per workgroup: eight where the head shape leaves every phase at least one column per
// lane and the registers fit two waves per SIMD, else four.
template <typename T, int DK, int DV, bool EXACT>
constexpr int bwd_waves() {
  return (EXACT && sizeof(T) == 2 && ((DK == 32 && DV == 64) || (DK == 36 && DV == 72))) ? DIG_BWD_WAVES8 : 4;
}

template <typename T, int DK, int DV, bool EXACT, int C, bool LR>
static hipError_t launch_bwd_c(const GlaShape& s, GlaBwdParams p, hipStream_t st, int* lds_out,
                               size_t* ru_out) {
  const long BH = (long)s.B * s.H;
  constexpr int NW = bwd_waves<T, DK, DV, EXACT>();
  constexpr bool RU = bwd_reuse_ok<DK, DV, EXACT, C, NW>();
  const bool lb = RU && s.lookback;  // the look-back shares the reuse condition
  const bool three = !s.bprefix && s.nseg > 1 && !lb;
  if (ru_out) {  // reuse buffers: dO fragments of every chunk, then the diagonals
    ru_out[0] = RU && three ? (size_t)BH * s.NC * (bwd_reuse_chunk_bytes<T, DV, C, NW>() - 2 * C * sizeof(float)) : 0;
    ru_out[1] = RU && three ? (size_t)BH * s.NC * 2 * C * sizeof(float) : 0;
    return hipSuccess;
  }
  constexpr bool PF_FIN = bwd_prefetch<DK, DV, EXACT, true, NW>();
  constexpr bool PF_RD = bwd_prefetch<DK, DV, EXACT, true, NW, true>();
  constexpr bool PF_A = bwd_prefetch<DK, DV, EXACT, false, NW>();
  constexpr int fin_bytes =
      BwdLayout<T, DK, DV, C, true, bwd_lean<T, DK, DV, C, true, NW, PF_FIN, LR>(), NW, PF_FIN,
                LR>::bytes;
  constexpr int rd_bytes =
      BwdLayout<T, DK, DV, C, true, bwd_lean<T, DK, DV, C, true, NW, PF_RD, LR>(), NW, PF_RD,
                LR>::bytes;
  constexpr int a_bytes =
      BwdLayout<T, DK, DV, C, false, bwd_lean<T, DK, DV, C, false, NW, PF_A, LR>(), NW, PF_A,
                LR>::bytes;
  if (lds_out) {
    *lds_out = RU && three && rd_bytes > fin_bytes ? rd_bytes : fin_bytes;
    return hipSuccess;
  }
  if constexpr (RU) {
    if (lb) {
      if (!p.lb_flag) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gla_bwd_kernel<T, DK, DV, EXACT, C, true, NW, false, true, LR>),
                         dim3((unsigned)(BH * s.nseg)), dim3(64 * NW), fin_bytes, st, p);
      return hipGetLastError();
    }
  }
  if (three) {
    if constexpr (RU) {
      if (!p.dofrag || !p.diagws) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gla_bwd_kernel<T, DK, DV, EXACT, C, false, NW, true, false, LR>),
                         dim3((unsigned)(BH * s.nseg)), dim3(64 * NW), a_bytes, st, p);
    } else {
      hipLaunchKernelGGL((gla_bwd_kernel<T, DK, DV, EXACT, C, false, NW, false, false, LR>),
                         dim3((unsigned)(BH * s.nseg)), dim3(64 * NW), a_bytes, st, p);
    }
    const hipError_t e = launch_gla_gstate_scan(s, p, st);
    if (e != hipSuccess) return e;
    if constexpr (RU) {
      hipLaunchKernelGGL((gla_bwd_kernel<T, DK, DV, EXACT, C, true, NW, true, false, LR>),
                         dim3((unsigned)(BH * s.nseg)), dim3(64 * NW), rd_bytes, st, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gla_bwd_kernel<T, DK, DV, EXACT, C, true, NW, false, false, LR>),
                     dim3((unsigned)(BH * s.nseg)), dim3(64 * NW), fin_bytes, st, p);
  return hipGetLastError();
}

template <typename T, int DK, int DV, bool EXACT, bool LR>
static hipError_t launch_bwd_dims(const GlaShape& s, GlaBwdParams p, hipStream_t st,
                                  int* lds_out, size_t* ru_out) {
  switch (s.C) {
    case 16: return launch_bwd_c<T, DK, DV, EXACT, 16, LR>(s, p, st, lds_out, ru_out);
    case 32: return launch_bwd_c<T, DK, DV, EXACT, 32, LR>(s, p, st, lds_out, ru_out);
    case 64: return launch_bwd_c<T, DK, DV, EXACT, 64, LR>(s, p, st, lds_out, ru_out);
    default: return hipErrorInvalidValue;
  }
}

// Same shape dispatch as the forward.  Queries: lds_out != nullptr reports the final pass's
// LDS bytes, ru_out != nullptr the reuse buffers' bytes ({dO fragments, diagonals}).
template <typename T, bool LR>
hipError_t launch_gla_bwd_t(const GlaShape& s, GlaBwdParams p, hipStream_t st, int* lds_out,
                            size_t* ru_out) {
  if (s.dk == 32 && s.dv == 64) return launch_bwd_dims<T, 32, 64, true, LR>(s, p, st, lds_out, ru_out);
  if (s.dk == 36 && s.dv == 72) return launch_bwd_dims<T, 36, 72, true, LR>(s, p, st, lds_out, ru_out);
  if (s.dk == 16 && s.dv == 32) return launch_bwd_dims<T, 16, 32, true, LR>(s, p, st, lds_out, ru_out);
  switch (s.ndk * 16 + s.ndv) {
    case 1 * 16 + 2: return launch_bwd_dims<T, 16, 32, false, LR>(s, p, st, lds_out, ru_out);
    case 2 * 16 + 4: return launch_bwd_dims<T, 32, 64, false, LR>(s, p, st, lds_out, ru_out);
    case 3 * 16 + 5: return launch_bwd_dims<T, 48, 80, false, LR>(s, p, st, lds_out, ru_out);
    case 4 * 16 + 8: return launch_bwd_dims<T, 64, 128, false, LR>(s, p, st, lds_out, ru_out);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dig
