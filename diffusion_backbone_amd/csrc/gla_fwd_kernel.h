// gla_fwd_kernel.h -- the chunk kernel of the GLA forward on gfx950 (included by the
// per-element-type translation units gla_fwd_bf16.hip and gla_fwd_f32.hip).
//
// What is computed (DiG study-group slides, eqs. (5)-(10); write-up section 3,
// "Efficiency Analysis": chunks of M tokens computed on-chip), per image b and head h:
//   g_t = logsigmoid(z_t)/tau,  S_t = diag(exp g_t) S_{t-1} + k_t^T v_t,  o_t = q_t S_t,
//   y_t = RMSNorm_head(o_t) * w * Swish(r_t).
// Chunk form, with b_i = sum of g over the chunk up to token i (inclusive) and S0 the state
// entering the chunk:
//   o_i = sum_{j<=i} [sum_c q_ic e^{b_ic} k_jc e^{-b_jc}] v_j + (q_i e^{b_i}) S0
//   S_next = diag(e^{b_last}) S0 + sum_j (k_j e^{b_last - b_j})^T v_j
// The bracket (the gated Q K^T of the chunk) and both products with V/S run on matrix cores
// (bf16 16x16x32 or fp32 16x16x4, fp32 accumulation).  Gates live in log2 space in fp32.
// When a chunk's total decay is so strong that k e^{-b} could overflow, that chunk's gated
// Q K^T is evaluated elementwise as sum_c q_ic k_jc exp(b_ic - b_jc) instead.
//
// Per chunk, one workgroup of four waves runs two phases separated by barriers:
//   gate    lanes = tokens of the chunk, each lane a run of key columns: log-sigmoid, the
//           in-chunk cumulative sum as a DPP lane scan, the scaled operands q e^{b},
//           k e^{-b}, (k e^{b_last-b})^T and V^T written to LDS;
//   product every wave advances its share of the fp32 state tiles; wave I owns query rows
//           16I..16I+15: gated Q K^T (kept in registers), P V, (q e^{b}) S0, the RMSNorm x
//           Swish epilogue, y stored straight from the accumulators.
// Exact head shapes load the raw rows of the next chunk into registers while the current one
// is processed and write them to the one staging slot at the top of the next iteration (an
// LDS DMA would make every LDS read of the current chunk wait for the copy).  Tile classes
// copy global->LDS by DMA (two staging slots when LDS allows).
//
// Head dims: DK x DV is either the exact shape (compile-time dims, no guards) or a 16-wide
// tile class holding any smaller runtime shape (EXACT = false), zero-padded inside LDS.
// The LDS layout is a compile-time function of the template parameters.
#pragma once

#include <type_traits>

#include "dig_device.h"
#include "dig_internal.h"

namespace dig {

#ifndef DIG_FWD_WAVES8
#define DIG_FWD_WAVES8 8
#endif
constexpr float kSlowDecayLog2 = 96.0f;  // e^{-b} factors up to 2^96 stay finite in bf16/fp32
constexpr int kFwdLdsBudget = 160 * 1024;

constexpr int al16(int x) { return (x + 15) / 16 * 16; }

// PAD: raw staging rows at pitches the gate pass (one lane per token) reads without bank
// conflicts (register-staged rows; LDS DMA writes them packed).
// LR: the key gate is the rank-16 product formed in the gate pass (the staged z rows are the
// 16-element factor rows; the head's slice of the up-projection sits in an LDS table).
template <typename T, int DK, int DV, int C, bool OUT, int NW = 4, bool PAD = false,
          bool LR = false>
struct FwdLayout {
  static constexpr int SZ = (int)sizeof(T);
  static constexpr int NDK = (DK + 15) / 16, NDV = (DV + 15) / 16;
  static constexpr int DKP = ((NDK * 16 + 31) / 32) * 32;  // key dim padded to the K step
  static constexpr int DVP = NDV * 16;
  static constexpr int CK = SZ == 2 ? ((C + 31) / 32) * 32 : C;  // token dim padded
  static constexpr int QP = DKP + 8, TP = CK + 8;              // padded LDS row pitches
  // gate columns per lane: the key columns up to the last 16-wide tile (the K-step padding
  // past it stays zero and is never touched), the value columns
  // (exact head shapes whose d_k splits evenly over the lanes cover the true columns only: the
  // padding columns of the key tiles stay at their zero fill)
  static constexpr int GCOLS = PAD && (DK * C) % (64 * NW) == 0 ? DK : 16 * NDK;
  static constexpr int NCL = GCOLS * C / (64 * NW), NEL = DVP * C / (64 * NW);
  // q e^{b} and k e^{-b} are kept in fp32 for either element type (bf16 I/O splits them into
  // hi + lo bf16 fragments for the gated Q K^T): QKC stored columns (the true d_k for exact
  // head shapes, the 16-wide tile class otherwise) at pitch QKP floats
  static constexpr int QKC = SZ == 2 ? (PAD ? (DK + 3) / 4 * 4 : 16 * NDK) : DKP;
  static constexpr int QKP = SZ == 2 ? (QKC % 32 == 0 ? QKC + 4 : QKC) : QP;
  // byte offsets: operands, state copy, gates, misc; the raw staging slots come last
  static constexpr int O_Q = 0;                                         // q e^{b}  [C][QKP]
  static constexpr int O_K = O_Q + al16(OUT ? C * QKP * 4 : 0);          // k e^{-b} [C][QKP]
  static constexpr int O_KBT = O_K + al16(OUT ? C * QKP * 4 : 0);        // kbar^T [16NDK][TP]
  // VTR: the products read V from the staged rows through the transpose load (register-staged
  // bf16 rows, padded to DVP zero columns), so the gate pass writes no V^T copy; the token
  // dimension is a contraction over whole 32-token steps, so the chunk must hold them (32, 64)
  static constexpr bool VTR = PAD && SZ == 2 && C % 32 == 0;
  static constexpr int O_VT = O_KBT + al16(16 * NDK * TP * SZ);          // v^T    [DVP][TP]
  static constexpr int O_S = O_VT + al16(VTR ? 0 : DVP * TP * SZ);       // S^T    [DVP][QP]
  // b fp32 [C][DK], written only for strong-decay chunks, which do not read k e^{-b}: it
  // takes that tile's place when it fits there
  static constexpr bool B_IN_K = C * DK * 4 <= C * QKP * 4;
  static constexpr int O_B = B_IN_K ? O_K : O_S + al16(OUT ? DVP * QP * SZ : 0);
  static constexpr int O_GAM = O_S + al16(OUT ? DVP * QP * SZ : 0) +
                               al16(OUT && !B_IN_K ? C * DK * 4 : 0);  // e^{b_last} [DKP]
  static constexpr int O_LG = O_GAM + al16(DKP * 4);                     // segment decay
  static constexpr int O_MAX = O_LG + al16(DKP * 4);                     // per-wave decay
  static constexpr int O_ZT = O_MAX + 64;                 // low-rank gate table (LR)
  static constexpr int O_RAW = O_ZT + al16(LR ? lowrank_table_bytes(16 * NDK) : 0);
  // factor rows (LR): 16 elements at a 48-byte pitch when register-staged (conflict-free
  // 16-byte reads, one lane per token), packed when DMA-staged
  static constexpr int ZPE = PAD ? 24 : kGateRank;
  // one staging slot: raw k, z, v (+ q, r) rows at pitches KPE, VPE (elements; the runtime
  // widths when DMA-staged).  A padded pitch is kept only if it does not cost the second
  // workgroup per CU.
  static constexpr int slot_bytes(int kpe, int vpe) {
    return al16(C * kpe * SZ) + al16(C * (LR ? ZPE : kpe) * SZ) + al16(C * vpe * SZ) +
           (OUT ? al16(C * kpe * SZ) + al16(C * vpe * SZ) : 0);
  }
  static constexpr int HALF_CU = 80 * 1024;
  static constexpr bool fits(int kpe, int vpe) {
    return O_RAW + slot_bytes(kpe, vpe) <= HALF_CU || O_RAW + slot_bytes(DK, DV) > HALF_CU;
  }
  static constexpr int KPAD = row_pitch(DK * SZ, NCL * SZ) / SZ;
  static constexpr int VPAD = row_pitch(DV * SZ, NEL * SZ) / SZ;
  static constexpr int KPE = PAD && fits(KPAD, DV) ? KPAD : DK;
  static constexpr int VPE = VTR ? DVP : (PAD && fits(KPE, VPAD) ? VPAD : DV);
  static constexpr int R_K = 0;
  static constexpr int R_Z = R_K + al16(C * KPE * SZ);
  static constexpr int R_V = R_Z + al16(C * (LR ? ZPE : KPE) * SZ);
  static constexpr int R_Q = R_V + al16(C * VPE * SZ);
  static constexpr int R_R = R_Q + al16(OUT ? C * KPE * SZ : 0);
  static constexpr int SLOT = R_R + al16(OUT ? C * VPE * SZ : 0);
  static constexpr int bytes(int nbuf) { return O_RAW + nbuf * SLOT; }
};

// Look-back (LB: short sequences, one chunk per workgroup, one launch).  The state waves form
// the chunk's own contribution U = Kbar^T V (the carry from a zero state), publish it with the
// chunk's decay factors and raise the chunk's flag, while the query-row waves form P V; then
// the state waves wait for the earlier chunks' flags of the sequence and sum
//   S0(n) = U(n-1) + diag(e^{b_last(n-1)}) U(n-2) + diag(e^{b_last(n-1) + b_last(n-2)}) U(n-3) ...
// which the query-row waves then use for (q e^b) S0.  Earlier chunks have lower workgroup
// indices (dispatched first), every wait is bounded, and flags carry a per-call tag.
template <typename T, int DK, int DV, bool EXACT, int C, bool OUT, int NW, bool LB = false,
          bool LR = false>
__global__ __launch_bounds__(64 * NW) void gla_fwd_kernel(GlaFwdParams p, int nbuf) {
  static_assert(!LB || OUT, "the look-back runs the output kernel");
  static_assert(!LR || sizeof(T) == 2, "the low-rank gate is bf16");
  constexpr int NTH = 64 * NW;  // NW waves
  using Lo = FwdLayout<T, DK, DV, C, OUT, NW, EXACT, LR>;
  constexpr int ZPE = Lo::ZPE;
  constexpr bool VTR = Lo::VTR;  // V through the transpose load from the staged rows
  constexpr int KPE = Lo::KPE, VPE = Lo::VPE;
  constexpr bool kBf = sizeof(T) == 2;
  constexpr int NDK = Lo::NDK, NDV = Lo::NDV, DKP = Lo::DKP, DVP = Lo::DVP, CK = Lo::CK;
  constexpr int QP = Lo::QP, TP = Lo::TP;
  constexpr int QKC = Lo::QKC, QKP = Lo::QKP;  // fp32 q e^{b}, k e^{-b} tiles
  constexpr int NT = C / 16;                            // query row tiles
  constexpr int NST = NDK * NDV;                        // fp32 state tiles
  // state tiles are owned by waves SW0..NW-1: the waves past the query row tiles when there
  // are more waves than row tiles (they advance the state while the others form outputs)
  constexpr int SW0 = (OUT && NW > NT) ? NT : 0, NSW = NW - SW0;
  constexpr int STW = (NST + NSW - 1) / NSW;            // state tiles per owning wave
  constexpr int NCL = Lo::NCL;                          // gate pass: key columns per lane
  constexpr int NEL = Lo::NEL;                          // V transpose: value columns per lane
  // every gate/transpose column is a real one: no per-column guards
  constexpr bool FULLK = EXACT && DK == DKP, FULLV = EXACT && DV == DVP;
  static_assert(NCL >= 1 && NEL >= 1, "tile split");
  static_assert(QKC % NCL == 0 || QKC >= 16 * NDK, "gate column runs end at the stored columns");
  using Acc = typename std::conditional<kBf, float, double>::type;
  constexpr bool PF = EXACT;  // register prefetch (one staging slot) for exact head shapes

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  // Workgroups are handed to the 8 XCDs (each with its own L2) in turn, workgroup i to XCD
  // i mod 8.  A head's rows are d_k- or d_v-wide slices of each token row that share 128-byte
  // lines with the neighbouring heads.  The output pass numbers workgroups head x segments +
  // segment.  Pass A launches one segment fewer per head (the last segment's state is never
  // needed), which in that numbering would spread a segment's heads over the XCDs: its work
  // items are numbered segment-major (heads fastest) and XCD x takes the x-th contiguous
  // eighth of them, so the heads of a segment meet in one L2.
  int seg, bh;
  if constexpr (OUT) {
    seg = blockIdx.x % p.nseg;
    bh = blockIdx.x / p.nseg;
  } else {
    const int nbh = p.B * p.H;
    const int item = xcd_item((int)blockIdx.x, (int)gridDim.x);
    seg = item / nbh;
    bh = item - seg * nbh;
  }
  const int b = bh / p.H, h = bh - b * p.H;
  const int H = p.H;
  const int dk = EXACT ? DK : p.dk, dv = EXACT ? DV : p.dv;

  float* sQ = reinterpret_cast<float*>(smem + Lo::O_Q);
  float* sK = reinterpret_cast<float*>(smem + Lo::O_K);
  T* sKbT = reinterpret_cast<T*>(smem + Lo::O_KBT);
  T* sVt = reinterpret_cast<T*>(smem + Lo::O_VT);
  T* sS = reinterpret_cast<T*>(smem + Lo::O_S);
  float* sB = reinterpret_cast<float*>(smem + Lo::O_B);
  float* sGam = reinterpret_cast<float*>(smem + Lo::O_GAM);
  float* sLg = reinterpret_cast<float*>(smem + Lo::O_LG);
  float* sMax = reinterpret_cast<float*>(smem + Lo::O_MAX);

  const int c_first = seg * p.sc;
  const int c_end = min(p.NC, c_first + p.sc);
  const int n_begin = (OUT && p.prefix) ? 0 : c_first;
  const bool scanned = !LB && !p.prefix && p.nseg > 1;  // incoming state comes from pass B
  const long sbase = (long)bh * p.NC;             // chunk-slot base for this (b,h)
  const float inv_tau = p.g2scale * 0.69314718055994531f;  // g2scale = log2(e) / tau

  const T* gq = static_cast<const T*>(p.q);
  const T* gk = static_cast<const T*>(p.k);
  const T* gv = static_cast<const T*>(p.v);
  const T* gz = static_cast<const T*>(p.z);
  const T* gr = static_cast<const T*>(p.r);
  T* gy = static_cast<T*>(p.y);
  T* gop = static_cast<T*>(p.o_pre);

  // staging slot s: k, z, v, then q, r (output chunks only)
  auto issue = [&](int n, int s) {
    unsigned char* base = smem + Lo::O_RAW + s * Lo::SLOT;
    const int t0 = n * C, valid = min(C, p.L - t0);
    const long row0 = ((long)b * p.L + t0) * H + h;
    const long gsk = (long)H * dk * sizeof(T), gsv = (long)H * dv * sizeof(T);
    const int rbk = dk * (int)sizeof(T), rbv = dv * (int)sizeof(T);
    dma_rows_c(base + Lo::R_K, reinterpret_cast<const unsigned char*>(gk + row0 * dk), gsk, rbk,
               valid, wave, NW, lane);
    if constexpr (LR)
      dma_rows_c(base + Lo::R_Z,
                 reinterpret_cast<const unsigned char*>(gz + ((long)b * p.L + t0) * kGateRank),
                 kGateRank * sizeof(T), kGateRank * (int)sizeof(T), valid, wave, NW, lane);
    else
      dma_rows_c(base + Lo::R_Z, reinterpret_cast<const unsigned char*>(gz + row0 * dk), gsk,
                 rbk, valid, wave, NW, lane);
    dma_rows_c(base + Lo::R_V, reinterpret_cast<const unsigned char*>(gv + row0 * dv), gsv, rbv,
               valid, wave, NW, lane);
    if (OUT && n >= c_first) {
      dma_rows_c(base + Lo::R_Q, reinterpret_cast<const unsigned char*>(gq + row0 * dk), gsk,
                 rbk, valid, wave, NW, lane);
      dma_rows_c(base + Lo::R_R, reinterpret_cast<const unsigned char*>(gr + row0 * dv), gsv,
                 rbv, valid, wave, NW, lane);
    }
  };
  // exact shapes: the raw rows of a chunk in registers (loaded one iteration ahead)
  RowRegs<DK * (int)sizeof(T), C, NTH, KPE * (int)sizeof(T)> pk, pq;
  RowRegs<(LR ? kGateRank : DK) * (int)sizeof(T), C, NTH, (LR ? ZPE : KPE) * (int)sizeof(T)> pz;
  RowRegs<DV * (int)sizeof(T), C, NTH, VPE * (int)sizeof(T)> pv, pr;
  auto pf_load = [&](int n) {
    const int t0 = n * C, valid = min(C, p.L - t0);
    const long row0 = ((long)b * p.L + t0) * H + h;
    const long gsk = (long)H * DK * sizeof(T), gsv = (long)H * DV * sizeof(T);
    pk.load(reinterpret_cast<const unsigned char*>(gk + row0 * DK), gsk, valid, tid);
    if constexpr (LR)
      pz.load(reinterpret_cast<const unsigned char*>(gz + ((long)b * p.L + t0) * kGateRank),
              kGateRank * sizeof(T), valid, tid);
    else
      pz.load(reinterpret_cast<const unsigned char*>(gz + row0 * DK), gsk, valid, tid);
    pv.load(reinterpret_cast<const unsigned char*>(gv + row0 * DV), gsv, valid, tid);
    if (OUT && n >= c_first) {
      pq.load(reinterpret_cast<const unsigned char*>(gq + row0 * DK), gsk, valid, tid);
      pr.load(reinterpret_cast<const unsigned char*>(gr + row0 * DV), gsv, valid, tid);
    }
  };
  auto pf_put = [&](int n, unsigned char* base) {
    const int valid = min(C, p.L - n * C);
    pk.put(base + Lo::R_K, valid, tid);
    pz.put(base + Lo::R_Z, valid, tid);
    pv.put(base + Lo::R_V, valid, tid);
    if (OUT && n >= c_first) {
      pq.put(base + Lo::R_Q, valid, tid);
      pr.put(base + Lo::R_R, valid, tid);
    }
  };
  if constexpr (PF) pf_load(n_begin);
  else issue(n_begin, 0);  // the first chunk's copy overlaps the set-up below

  // zero everything but the staging slots (with VTR the slot too: the V rows' padding columns
  // are operands): padding rows/columns of the MFMA operands must read as zero and are never
  // written afterwards
  for (int i = tid; i < (VTR ? Lo::bytes(1) : Lo::O_RAW) / 16; i += NTH)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();  // the zero fill is complete before anything below writes LDS
  if constexpr (LR)  // read from the first chunk's gate pass on (behind the loop's barrier)
    lowrank_table_fill<16 * NDK, NTH>(smem + Lo::O_ZT, static_cast<const bf16*>(p.zw), p.zb, h,
                                      dk, tid);

  f32x4 sacc[STW];
#pragma unroll
  for (int m = 0; m < STW; ++m) sacc[m] = zero4();
  if (OUT && scanned && seg > 0) {  // (never with the look-back: scanned is false there)
    const float* src = p.states + (sbase + c_first) * dk * dv;
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave - SW0 + NSW * m;
      if (wave >= SW0 && u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
        const int e = et * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ct * 16 + g4 * 4 + i;
          sacc[m][i] = (c < dk && e < dv) ? src[c * dv + e] : 0.f;
        }
      }
    }
  }

  float gm[NDV];  // norm weight of the output column this lane touches in tile E
#pragma unroll
  for (int E = 0; E < NDV; ++E) {
    const int e = E * 16 + r16;
    gm[E] = (OUT && e < dv && p.norm_w) ? p.norm_w[e] : 1.f;
  }
  // oacc += (q e^{b}) S0 for query rows 16I..: S0 is the bf16 copy in sS; q e^{b} enters as
  // hi + lo parts (bf16 I/O)
  auto q_s0 = [&](f32x4 (&oacc)[NDV], int I) {
    const int l = opaque(tid & 63);
    if constexpr (kBf) {
#pragma unroll
      for (int E = 0; E < NDV; ++E)
        oacc[E] = mm_split_b<QKC, QKP, QP>(oacc[E], sQ, 16 * I, reinterpret_cast<const bf16*>(sS),
                                           16 * E, l);
    } else {
#pragma unroll
      for (int E = 0; E < NDV; ++E)
        oacc[E] = Mma<T>::kc(oacc[E], sQ, QKP, 16 * I, sS, QP, 16 * E, DKP, l);
    }
  };

  // Every load above (and the first chunk's rows) has landed before the loop: otherwise the
  // compiler's wait for them, placed inside the loop, would also wait for the prefetch.
  if constexpr (PF) dma_wait();

  // gate-pass lane roles: token tg of the chunk, key columns c0.., value columns e0..
  const int tg = tid % C, cg = tid / C;
  const int c0 = cg * NCL, e0 = cg * NEL;

  for (int n = n_begin; n < c_end; ++n) {
    // per-iteration copies of the lane-dependent indices (see opaque())
    const int lane = opaque(tid & 63);
    const int r16 = lane & 15, g4 = lane >> 4;
    const int tg = (wave * 64 + lane) % C, cg = (wave * 64 + lane) / C;
    const int c0 = cg * NCL, e0 = cg * NEL;
    const int it = n - n_begin;
    const int slot = nbuf == 2 ? (it & 1) : 0;
    unsigned char* raw = smem + Lo::O_RAW + slot * Lo::SLOT;
    const T* rawk = reinterpret_cast<const T*>(raw + Lo::R_K);
    const T* rawz = reinterpret_cast<const T*>(raw + Lo::R_Z);
    const T* rawv = reinterpret_cast<const T*>(raw + Lo::R_V);
    const T* rawq = reinterpret_cast<const T*>(raw + Lo::R_Q);
    const T* sR = reinterpret_cast<const T*>(raw + Lo::R_R);
    // raw row pitches: padded for register-staged rows, the runtime widths for DMA-staged ones
    const int kp = PF ? KPE : dk, vp = PF ? VPE : dv;
    const bool emit = OUT && n >= c_first;
    const int t0 = n * C;
    const int valid = min(C, p.L - t0);
    const long row0 = ((long)b * p.L + t0) * H + h;  // (b, t0, h) as a token-head row

    if constexpr (PF) {
      pf_put(n, raw);  // the previous chunk's last reads of the slot preceded the last barrier
    } else if (nbuf == 1 && it > 0) {  // single slot: wait until the previous chunk left it
      __syncthreads();
      issue(n, 0);
    }
    // the state entering this chunk: saved for the backward, bf16 copy for (q e^b) S0
    if (!LB && emit && p.write_states && !(scanned && n == c_first)) {
      float* dst = p.states + (sbase + n) * dk * dv;
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        const int u = wave - SW0 + NSW * m;
        if (wave >= SW0 && u < NST) {
          const int ct = u / NDV, et = u - ct * NDV;
          const int e = et * 16 + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = ct * 16 + g4 * 4 + i;
            if (c < dk && e < dv) dst[c * dv + e] = sacc[m][i];
          }
        }
      }
    }
    if (!LB && emit) {
#pragma unroll
      for (int m = 0; m < STW; ++m) {
        const int u = wave - SW0 + NSW * m;
        if (wave >= SW0 && u < NST) {
          const int ct = u / NDV, et = u - ct * NDV;
          const int e = et * 16 + r16;
          T s4[4];  // the lane's four key rows of column e: one 8-byte write
#pragma unroll
          for (int i = 0; i < 4; ++i) s4[i] = from_f<T>(sacc[m][i]);
          lds_row_write<T, 4>(sS + e * QP, ct * 16 + g4 * 4, s4);
        }
      }
    }
    if constexpr (!PF) dma_wait();
    __syncthreads();
    if constexpr (PF) {
      if (n + 1 < c_end) pf_load(n + 1);
    } else if (nbuf == 2 && n + 1 < c_end) {
      issue(n + 1, slot ^ 1);
    }

    // ---------------------------------------------------------------- gate phase
    // (every LDS read first, then the arithmetic, then every write: one LDS round trip)
    float bb[NCL];  // in-chunk cumulative log2 gates of token tg, key columns c0..
    {
      const bool tv = tg < valid;
      T zr[NCL], kr[NCL], qr[NCL], vr[NEL];
      float zf[NCL];  // gate logits
      if constexpr (LR) {  // formed and turned into log gates before the other rows are read
        lowrank_logits<16 * NDK, NCL>(zf, reinterpret_cast<const bf16*>(rawz) + tg * ZPE,
                                      smem + Lo::O_ZT, c0);
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
          const bool on = FULLK ? tv : (tv && c0 + j < dk);
          bb[j] = keep_if(on, Fm<T>::lsig2(zf[j]) * inv_tau);
          pin(bb[j]);
        }
      } else if constexpr (FULLK) {
        lds_row_read_k<T, NCL, KPE>(zr, rawz + tg * KPE, c0, tv);
      } else {
        lds_row_read<T, NCL>(zr, rawz + tg * kp, c0, dk, tv, kp);
      }
      if constexpr (FULLK) {
        lds_row_read_k<T, NCL, KPE>(kr, rawk + tg * KPE, c0, tv);
        if (emit) lds_row_read_k<T, NCL, KPE>(qr, rawq + tg * KPE, c0, tv);
      } else {
        lds_row_read<T, NCL>(kr, rawk + tg * kp, c0, dk, tv, kp);
        if (emit) lds_row_read<T, NCL>(qr, rawq + tg * kp, c0, dk, tv, kp);
      }
      if constexpr (VTR) {
      } else if constexpr (FULLV) {
        lds_row_read_k<T, NEL, VPE>(vr, rawv + tg * VPE, e0, tv);
      } else {
        lds_row_read<T, NEL>(vr, rawv + tg * vp, e0, dv, tv, vp);
      }
      if constexpr (!LR) {
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
          const bool on = FULLK ? tv : (tv && c0 + j < dk);
          bb[j] = keep_if(on, Fm<T>::lsig2(to_f(zr[j])) * inv_tau);
        }
      }

      float bl[NCL];
#pragma unroll
      for (int j = 0; j < NCL; ++j) bb[j] = scan_dpp<C>(bb[j]);
#pragma unroll
      for (int j = 0; j < NCL; ++j) bl[j] = group_last<C>(bb[j], lane);
      T kb[NCL];
      float qs[NCL], ks[NCL];
#pragma unroll
      for (int j = 0; j < NCL; ++j) {
        const float kf = to_f(kr[j]);
        kb[j] = from_f<T>(kf * Fm<T>::exp2(bl[j] - bb[j]));
        if (emit) {
          qs[j] = to_f(qr[j]) * p.q_scale * Fm<T>::exp2(bb[j]);
          ks[j] = kf * Fm<T>::exp2(-bb[j]);
        }
      }
      float md = 0.f;  // strongest decay over this wave's columns -> slow-path test
#pragma unroll
      for (int j = 0; j < NCL; ++j) md = fmaxf(md, -bl[j]);
      if (emit) md = wave_max_dpp(md);

#pragma unroll
      for (int j = 0; j < NCL; ++j)
        if (FULLK || c0 + j < 16 * NDK) sKbT[(c0 + j) * TP + tg] = kb[j];
      if constexpr (!VTR) {
#pragma unroll
        for (int j = 0; j < NEL; ++j) sVt[(e0 + j) * TP + tg] = vr[j];  // V^T, zero past the end
      }
      if (emit) {
        if (c0 < QKC) {  // a lane's column run lies wholly inside or past the stored columns
          lds_row_write<float, NCL>(sQ + tg * QKP, c0, qs);
          lds_row_write<float, NCL>(sK + tg * QKP, c0, ks);
        }
        if (lane == 0) sMax[wave] = md;
      }
      if (tg == C - 1) {
#pragma unroll
        for (int j = 0; j < NCL; ++j) {
          sGam[c0 + j] = Fm<T>::exp2(bl[j]);
          if (!OUT) sLg[c0 + j] += bl[j];
        }
      }
    }
    __syncthreads();

    // strong decay somewhere in the chunk (uniform over the workgroup): the gated Q K^T is
    // evaluated elementwise from b, which is written now (over k e^{-b} when it fits there)
    bool slow = false;
    if (emit) {
      float mxa = sMax[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) mxa = fmaxf(mxa, sMax[w]);
      slow = mxa > kSlowDecayLog2;
    }
    if (slow) {
#pragma unroll
      for (int j = 0; j < NCL; ++j)
        if (FULLK || c0 + j < dk) sB[tg * DK + c0 + j] = bb[j];
      __syncthreads();
    }

    // ------------------------------------------------------------- product phase
    // state carry first (independent of the outputs): S = diag(e^{b_last}) S + Kbar^T V
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave - SW0 + NSW * m;
      if (wave >= SW0 && u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
        const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + ct * 16 + g4 * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[m][i] *= gam[i];
        if constexpr (VTR)
          sacc[m] = Mma<T>::template mm<true, false>(sacc[m], sKbT, TP, 16 * ct, rawv, VPE,
                                                     16 * et, CK, lane);
        else
          sacc[m] = Mma<T>::kc(sacc[m], sKbT, TP, 16 * ct, sVt, TP, 16 * et, CK, lane);
      }
    }
    if constexpr (LB) {  // publish U (sacc started from zero) and the chunk's decay factors
      if (wave >= SW0) {
        const long slot = (long)bh * p.nseg + seg;
        float* dst = p.lb_u + slot * dk * dv;
#pragma unroll
        for (int m = 0; m < STW; ++m) {
          const int u = wave - SW0 + NSW * m;
          if (u < NST) {
            const int ct = u / NDV, et = u - ct * NDV;
            const int e = et * 16 + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int c = ct * 16 + g4 * 4 + i;
              if ((FULLK || c < dk) && (FULLV || e < dv)) st_dev(dst + c * dv + e, sacc[m][i]);
            }
          }
        }
        for (int c = tid - 64 * SW0; c < dk; c += 64 * NSW) st_dev(p.seg_lg + slot * dk + c, sGam[c]);
      }
    }

    f32x4 oacc[NDV];
#pragma unroll
    for (int E = 0; E < NDV; ++E) oacc[E] = zero4();
    if (emit && wave < NT) {
      const int I = wave;  // this wave's 16 query rows
      // exact diagonal q_i.k_i (gate factor 1) from the unscaled inputs, so that a
      // cancelling dot product keeps its relative accuracy: 16 rows x 4 column groups
      float diag;
      {
        constexpr int DQ = 4 * NDK;  // four column groups over the 16-wide key tiles
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
        diag = (float)acc * p.q_scale;
      }
      // P^T tiles: pt[J][i] = P[16I + r16][16J + 4*g4 + i]
      f32x4 pt[NT];
      if (!slow) {
        if constexpr (kBf) {
          // split operands: where o_i cancels to a small vector its relative error is that of
          // these sums, and the RMSNorm gradient magnifies it by rstd_i
          const auto bq = split_b<QKC, QKP>(sQ, 16 * I, lane);  // once for every column tile
#pragma unroll
          for (int J = 0; J < NT; ++J)
            pt[J] = J <= I ? mm_split_pre<QKC, QKP, QKP>(zero4(), sK, 16 * J, bq, lane) : zero4();
        } else {
#pragma unroll
          for (int J = 0; J < NT; ++J)
            pt[J] = J <= I ? Mma<T>::kc(zero4(), sK, QKP, 16 * J, sQ, QKP, 16 * I, DKP, lane) : zero4();
        }
      } else {
        // strong decay: P_ij = sum_c q_ic k_jc 2^{b_ic - b_jc} elementwise (no overflow), each
        // lane its own elements (rare path, kept compact); j > i is masked below
        const int ir = 16 * I + r16;
#pragma unroll
        for (int J = 0; J < NT; ++J) pt[J] = zero4();
#pragma unroll 1
        for (int c = 0; c < dk; ++c) {
          const float qc = to_f(rawq[ir * kp + c]) * p.q_scale, bq = sB[ir * DK + c];
#pragma unroll
          for (int J = 0; J < NT; ++J) {
            if (J <= I) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int j = 16 * J + 4 * g4 + i;
                pt[J][i] += qc * to_f(rawk[j * kp + c]) * Fm<T>::exp2(bq - sB[j * DK + c]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int J = 0; J < NT; ++J) {  // diagonal tile: causal mask and the exact diagonal
        if (J == I) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (4 * g4 + i > r16) pt[J][i] = 0.f;
            if (4 * g4 + i == r16) pt[J][i] = diag;
          }
        }
      }

      // inter-chunk: O = (q e^{b}) S0 (the look-back adds it once S0 is known)
      if constexpr (!LB) q_s0(oacc, I);

      // intra-chunk: O += P V   (P straight from the accumulators above)
      if constexpr (kBf) {
#pragma unroll
        for (int pp = 0; pp < (NT + 1) / 2; ++pp) {
          if (2 * pp <= I) {
            const bool hi_on = 2 * pp + 1 <= I;
            bf16x8 a;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              a[i] = from_f<bf16>(pt[2 * pp][i]);
              a[4 + i] = from_f<bf16>(hi_on ? pt[min(2 * pp + 1, NT - 1)][i] : 0.f);
            }
#pragma unroll
            for (int E = 0; E < NDV; ++E) {
              bf16x4 lo, hi;
              if constexpr (VTR) {  // tokens 32pp + 4g4.. and +16 of value column 16E + r16
                lo = lds_tr4(rawv, VPE, 16 * E, 32 * pp + 4 * g4, r16);
                hi = lds_tr4(rawv, VPE, 16 * E, 32 * pp + 16 + 4 * g4, r16);
              } else {
                const T* vb = sVt + (E * 16 + r16) * TP + 32 * pp + 4 * g4;
                lo = *reinterpret_cast<const bf16x4*>(vb);
                hi = *reinterpret_cast<const bf16x4*>(vb + 16);
              }
              bf16x8 bv;
#pragma unroll
              for (int i = 0; i < 4; ++i) { bv[i] = lo[i]; bv[4 + i] = hi[i]; }
              oacc[E] = mfma_bf16(a, bv, oacc[E]);
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
              for (int E = 0; E < NDV; ++E) {
                const float bv = to_f(sVt[(E * 16 + r16) * TP + 16 * J + 4 * g4 + s4]);
                oacc[E] = mfma_f32(pt[J][s4], bv, oacc[E]);
              }
            }
          }
        }
      }

    }
    if constexpr (LB) {
      __builtin_amdgcn_s_waitcnt(0);  // U and the decay factors are out
      __syncthreads();
      const long slot0 = (long)bh * p.nseg;
      if (tid == 0)
        __hip_atomic_store(p.lb_flag + slot0 + seg, p.lb_tag, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      if (wave >= SW0) {
        // S0 = the earlier chunks' U, each decayed by the chunks between; the state tiles are
        // reused for it (U has been published)
#pragma unroll
        for (int m = 0; m < STW; ++m) sacc[m] = zero4();
        if (seg > 0) {
          const bool expired = lb_wait_all(p.lb_flag + slot0, seg, p.lb_wait_tag, lane, p.lb_spins);
          float fac[STW][4];
#pragma unroll
          for (int m = 0; m < STW; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) fac[m][i] = 1.f;
          constexpr int LBU = STW <= 2 ? 2 : 1;  // chunks whose loads are in flight together
          for (int m0 = seg - 1; m0 >= 0; m0 -= LBU) {
            float uv[LBU][STW][4], gv[LBU][STW][4];
#pragma unroll
            for (int a = 0; a < LBU; ++a) {
              const long sl = slot0 + max(m0 - a, 0);
#pragma unroll
              for (int m = 0; m < STW; ++m) {
                const int u = min(wave - SW0 + NSW * m, NST - 1);
                const int ct = u / NDV, et = u - ct * NDV;
                const int e = min(et * 16 + r16, dv - 1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int c = min(ct * 16 + g4 * 4 + i, dk - 1);
                  uv[a][m][i] = ld_dev(p.lb_u + sl * dk * dv + c * dv + e);
                  gv[a][m][i] = ld_dev(p.seg_lg + sl * dk + c);
                }
              }
            }
#pragma unroll
            for (int a = 0; a < LBU; ++a) {
              const bool on = m0 - a >= 0;
#pragma unroll
              for (int m = 0; m < STW; ++m) {
                const int u = wave - SW0 + NSW * m;
                const int ct = u / NDV, et = u - ct * NDV;
                const int e = et * 16 + r16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int c = ct * 16 + g4 * 4 + i;
                  const bool in = on && u < NST && (FULLK || c < dk) && (FULLV || e < dv);
                  sacc[m][i] += in ? fac[m][i] * uv[a][m][i] : 0.f;
                  fac[m][i] *= on ? gv[a][m][i] : 1.f;
                }
              }
            }
          }
          if (expired) {  // an earlier chunk's contribution never arrived: poison S0, record it
#pragma unroll
            for (int m = 0; m < STW; ++m) sacc[m] = f32x4{__builtin_nanf(""), __builtin_nanf(""),
                                                          __builtin_nanf(""), __builtin_nanf("")};
            if (lane == 0) lb_fail(p.lb_status);
          }
        }
        // S0: saved for the backward, bf16 copy for (q e^b) S0
        float* dst = p.states + (sbase + n) * dk * dv;
#pragma unroll
        for (int m = 0; m < STW; ++m) {
          const int u = wave - SW0 + NSW * m;
          if (u < NST) {
            const int ct = u / NDV, et = u - ct * NDV;
            const int e = et * 16 + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int c = ct * 16 + g4 * 4 + i;
              if (p.write_states && c < dk && e < dv) dst[c * dv + e] = sacc[m][i];
              sS[e * QP + c] = from_f<T>(sacc[m][i]);
            }
          }
        }
      }
      __syncthreads();
      if (tid == 0) lb_raise(p.lb_flag + (long)gridDim.x + slot0 + seg, p.lb_tag);  // done
    }
    if (emit && wave < NT) {
      const int I = wave;
      if constexpr (LB) q_s0(oacc, I);
      // output stage: head-wise RMSNorm x weight x Swish(r), stored from the accumulators
      T rr[NDV][4];  // all of this lane's r first (one LDS round trip)
      if constexpr (VTR) {  // the lane's four rows of each column tile in one transpose load
#pragma unroll
        for (int E = 0; E < NDV; ++E) {  // (the rows' padding columns read as zero)
          const bf16x4 r4 = lds_tr4(sR, VPE, 16 * E, 16 * I + 4 * g4, r16);
#pragma unroll
          for (int i = 0; i < 4; ++i) rr[E][i] = r4[i];
        }
      } else {
#pragma unroll
        for (int E = 0; E < NDV; ++E)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = E * 16 + r16;
            rr[E][i] = (FULLV || e < dv) ? sR[(16 * I + 4 * g4 + i) * vp + e] : from_f<T>(0.f);
          }
      }
      float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int E = 0; E < NDV; ++E)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss[i] += oacc[E][i] * oacc[E][i];
      float rstd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) rstd[i] = rsqrtf(row_sum16(ss[i]) / (float)dv + p.eps);
      // y, and for the backward (when saved) o rstd in fragment order and rstd per row
      Quad<float>* ob = p.obar ? static_cast<Quad<float>*>(p.obar) + ((sbase + n) * NT + I) * NDV * 64 + lane
                           : nullptr;
      // exact widths whose rows are whole 16-byte pieces: y goes through this wave's own 16
      // rows of the staged r (already read), then out as 16-byte row pieces
      constexpr bool VST = EXACT && (DV * (int)sizeof(T)) % 16 == 0 &&
                           (VPE * (int)sizeof(T)) % 16 == 0;
      const bool vst = VST && !gop;
      T* sY = const_cast<T*>(sR) + 16 * I * VPE;
#pragma unroll
      for (int E = 0; E < NDV; ++E) {
        const int e = E * 16 + r16;
        Quad<float> q4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * I + 4 * g4 + i;
          const float o = oacc[E][i];
          const float nv = o * rstd[i];
          q4.v[i] = nv;
          if (FULLV || e < dv) {
            const float rv = to_f(rr[E][i]);
            const T yv = from_f<T>(nv * gm[E] * rv * Fm<T>::sig(rv));
            if (vst) {
              sY[(4 * g4 + i) * VPE + e] = yv;
            } else if (row < valid) {
              const long off = (row0 + (long)row * H) * dv + e;
              if (gop) gop[off] = from_f<T>(o);
              gy[off] = yv;
            }
          }
        }
        if (ob) ob[E * 64] = q4;
      }
      if (vst) {
        // the wave's LDS writes above land before its reads below (in-order LDS per wave)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        constexpr int PPR = DV * (int)sizeof(T) / 16, NPC = 16 * PPR;  // pieces per row, tile
#pragma unroll
        for (int u = 0; u < (NPC + 63) / 64; ++u) {
          const int q = lane + 64 * u, rw = q / PPR, pc = q - rw * PPR;
          if (q < NPC && 16 * I + rw < valid) {
            const uint4 v4 = *reinterpret_cast<const uint4*>(sY + rw * VPE + pc * (16 / (int)sizeof(T)));
            *reinterpret_cast<uint4*>(gy + (row0 + (long)(16 * I + rw) * H) * dv +
                                      pc * (16 / (int)sizeof(T))) = v4;
          }
        }
      }
      if (ob && r16 == 0)
        *reinterpret_cast<float4*>(p.rstd + (sbase + n) * C + 16 * I + 4 * g4) =
            make_float4(rstd[0], rstd[1], rstd[2], rstd[3]);
    }
    __syncthreads();  // every read of the staging slot and of S^T is done
  }
  if constexpr (LB) {
    // the last workgroup: once every workgroup is done with its waits, clear the flags for
    // the next launch
    if (blockIdx.x == gridDim.x - 1) {
      const int n = (int)gridDim.x;
      if (lb_wait_each(p.lb_flag + n, n, p.lb_wait_tag, tid, NTH, p.lb_spins)) lb_fail(p.lb_status);
      __syncthreads();
      for (int i = tid; i < 2 * n; i += NTH) lb_raise(p.lb_flag + i, 0u);
    }
  }

  if (!OUT) {
    float* dst = p.states + (sbase + c_first) * dk * dv;
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave - SW0 + NSW * m;
      if (wave >= SW0 && u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
        const int e = et * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = ct * 16 + g4 * 4 + i;
          if (c < dk && e < dv) dst[c * dv + e] = sacc[m][i];
        }
      }
    }
    __syncthreads();
    for (int c = tid; c < dk; c += NTH)
      p.seg_lg[((long)bh * p.nseg + seg) * dk + c] = sLg[c];
  }
}

// Waves per workgroup: eight for the DiG-S head shape (the query-row waves and the state
// waves then run side by side), else four.
template <typename T, int DK, int DV, bool EXACT>
constexpr int fwd_waves() {
  return (EXACT && sizeof(T) == 2 && DK == 32 && DV == 64) ? DIG_FWD_WAVES8 : 4;
}

// LDS bytes and staging slots of one launch.  Exact shapes prefetch into registers (one
// slot); tile classes use two DMA slots when a workgroup walks more than one chunk and they fit.
template <typename T, int DK, int DV, bool EXACT, int C, bool OUT, bool LR>
static void fwd_lds(const GlaShape& s, int* bytes, int* nbuf) {
  using Lo = FwdLayout<T, DK, DV, C, OUT, fwd_waves<T, DK, DV, EXACT>(), EXACT, LR>;
  const int walk = (OUT && s.prefix) ? s.NC : s.sc;
  *nbuf = (!EXACT && walk > 1 && Lo::bytes(2) <= kFwdLdsBudget) ? 2 : 1;
  *bytes = Lo::bytes(*nbuf);
}

template <typename T, int DK, int DV, bool EXACT, int C, bool LR>
static hipError_t launch_fwd_c(const GlaShape& s, GlaFwdParams p, hipStream_t st, int* lds_out) {
  const long BH = (long)s.B * s.H;
  constexpr int NW = fwd_waves<T, DK, DV, EXACT>();
  int bytes_c, nbuf_c;
  fwd_lds<T, DK, DV, EXACT, C, true, LR>(s, &bytes_c, &nbuf_c);
  if (lds_out) {  // size query only
    *lds_out = bytes_c;
    return hipSuccess;
  }
  if constexpr (EXACT) {
    if (s.lookback) {
      if (!p.lb_u || !p.lb_flag) return hipErrorInvalidValue;
      hipLaunchKernelGGL((gla_fwd_kernel<T, DK, DV, EXACT, C, true, NW, true, LR>),
                         dim3((unsigned)(BH * s.nseg)), dim3(64 * NW), bytes_c, st, p, nbuf_c);
      return hipGetLastError();
    }
  }
  if (!s.prefix && s.nseg > 1) {
    int bytes_a, nbuf_a;
    fwd_lds<T, DK, DV, EXACT, C, false, LR>(s, &bytes_a, &nbuf_a);
    hipLaunchKernelGGL((gla_fwd_kernel<T, DK, DV, EXACT, C, false, NW, false, LR>),
                       dim3((unsigned)(BH * (s.nseg - 1))), dim3(64 * NW), bytes_a, st, p,
                       nbuf_a);
    const hipError_t e = launch_gla_state_scan(s, p.states, p.seg_lg, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((gla_fwd_kernel<T, DK, DV, EXACT, C, true, NW, false, LR>),
                     dim3((unsigned)(BH * s.nseg)), dim3(64 * NW), bytes_c, st, p, nbuf_c);
  return hipGetLastError();
}

template <typename T, int DK, int DV, bool EXACT, bool LR>
static hipError_t launch_fwd_dims(const GlaShape& s, GlaFwdParams p, hipStream_t st,
                                  int* lds_out) {
  switch (s.C) {
    case 16: return launch_fwd_c<T, DK, DV, EXACT, 16, LR>(s, p, st, lds_out);
    case 32: return launch_fwd_c<T, DK, DV, EXACT, 32, LR>(s, p, st, lds_out);
    case 64: return launch_fwd_c<T, DK, DV, EXACT, 64, LR>(s, p, st, lds_out);
    default: return hipErrorInvalidValue;
  }
}

// Exact DiG head shapes (S: 32/64, XL: 36/72, and 16/32), else the enclosing tile class.
// lds_out != nullptr: only report the LDS bytes of the output pass.
template <typename T, bool LR>
hipError_t launch_gla_fwd_t(const GlaShape& s, GlaFwdParams p, hipStream_t st, int* lds_out) {
  if (s.dk == 32 && s.dv == 64) return launch_fwd_dims<T, 32, 64, true, LR>(s, p, st, lds_out);
  if (s.dk == 36 && s.dv == 72) return launch_fwd_dims<T, 36, 72, true, LR>(s, p, st, lds_out);
  if (s.dk == 16 && s.dv == 32) return launch_fwd_dims<T, 16, 32, true, LR>(s, p, st, lds_out);
  switch (s.ndk * 16 + s.ndv) {
    case 1 * 16 + 2: return launch_fwd_dims<T, 16, 32, false, LR>(s, p, st, lds_out);
    case 2 * 16 + 4: return launch_fwd_dims<T, 32, 64, false, LR>(s, p, st, lds_out);
    case 3 * 16 + 5: return launch_fwd_dims<T, 48, 80, false, LR>(s, p, st, lds_out);
    case 4 * 16 + 8: return launch_fwd_dims<T, 64, 128, false, LR>(s, p, st, lds_out);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dig
