// gla_beta.hip -- the GLA mixer with the general gate of eq. (5), G_t = alpha_t^T beta_t
// (DiG study-group slides, slide "GLA の導入": a key-side gate alpha and a value-side gate
// beta), forward and backward, bf16 I/O and fp32 arithmetic.
//
// Per image and head: S_t = (alpha_t^T beta_t) (.) S_{t-1} + k_t^T v_t, o_t = (q_scale q_t) S_t,
// then the key-gate mixer's output stage y = RMSNorm(o) norm_w Swish(r).  log2 alpha =
// log2 sigmoid(z) / tau per key column, log2 beta = log2 sigmoid(w) / tau per value column;
// B and C are their inclusive running sums over a chunk's rows.
//
// Work layout.  Chunks of 64 tokens, one workgroup of four waves per chunk; wave w owns the
// 16-token tile w:
//   across chunks  each chunk's contribution U = sum_s (k_s 2^{B_end-B_s})^T (v_s 2^{C_end-C_s})
//                  and decays (pass 1); a scan over chunks (pass 2) gives the state entering
//                  every chunk, saved for the backward;
//   across tiles   the state entering tile w, S_w = 2^{B_w+C_w} (.) S_{w-1} + U_{w-1} (U of a
//                  tile formed like a chunk's), reaches tile w's rows as
//                  (q_t 2^{B_t-B_ref}) S_w 2^{C_t-C_ref}, ref = the row before the tile;
//   inside a tile  where both gates decay by at most 2^64 from ref to the tile's last row,
//                  the pair products are factored about ref, (q_t 2^{B_t-B_ref}) .
//                  (k_s 2^{B_ref-B_s}) and v_s 2^{C_ref-C_s}, 2^{C_t-C_ref}, on the matrix
//                  cores; elsewhere each of the 16 x 16 causal pairs takes its own factors
//                  2^{B_t[c]-B_s[c]} and 2^{C_t[e]-C_s[e]} on the vector ALU.
// Across chunks and tiles every factor 2^x has x <= 0; inside a tile |x| <= 64, so no gate
// strength overflows a factor or loses the small ones.
// The matrix products (chunk and tile contributions, the products with tile states) run on
// the fp32 matrix cores (16 x 16 x 4).  The backward mirrors this with gradient states G
// carried from later tiles and chunks (a reverse scan) and the boundary identity
//   dlog alpha_t = sum_{u >= t in chunk} (q_u dq_u - k_u dk_u) + sum_e (S_end (.) G_end)[:, e]
//   dlog beta_t  = sum_{u >= t in chunk} (do_u o_u - v_u dv_u) + sum_c (S_end (.) G_end)[c, :]
// (shifting every later running sum by eps scales S_end by 2^eps).
#include <type_traits>

#include "dig_device.h"
#include "dig_internal.h"

namespace dig {
namespace {

constexpr int kBC = 64;   // tokens per chunk
constexpr int kBT = 256;  // threads per workgroup (four waves, one 16-token tile each)

__device__ __forceinline__ float bf(bf16 x) { return static_cast<float>(x); }

template <int NDK, int NDV>
struct BetaLay {
  static constexpr int DKP = 16 * NDK, DVP = 16 * NDV;
  static constexpr int PQ = DKP + 8;    // bf16 row pitch of q and k
  static constexpr int PV = DVP + 8;    // bf16 row pitch of v
  static constexpr int PB = DKP + 4;    // fp32 row pitch of the key-gate sums
  static constexpr int PC = DVP + 4;    // fp32 row pitch of the value-gate sums, dO and states
  static constexpr int SZS = DKP * PC;  // floats of one state [DKP][PC]
  static constexpr int PA = 17;         // pitch of one wave's 16 x 16 pair table
  static constexpr int NQ = kBC * PQ * 2, NV = kBC * PV * 2;
  static constexpr int NB = kBC * PB * 4, NCB = kBC * PC * 4;
  // forward output pass: q, k, v, B, C, four states, four pair tables
  static constexpr int F_Q = 0, F_K = F_Q + NQ, F_V = F_K + NQ, F_B = F_V + NV, F_C = F_B + NB,
                       F_S = F_C + NCB, F_A = F_S + 4 * SZS * 4, F_END = F_A + 4 * 16 * PA * 4;
  // chunk-contribution passes: the two gate sums (then, in place, the scaled operands) and
  // the chunk's last row of each
  static constexpr int U_B = 0, U_C = U_B + NB, U_D = U_C + NCB, U_END = U_D + (DKP + DVP) * 4;
  // backward output pass: q, k, v, dO, B, C, four states, two sets of pair tables, boundary
  // sums and the norm-weight partials
  static constexpr int G_Q = 0, G_K = G_Q + NQ, G_V = G_K + NQ, G_D = G_V + NV, G_B = G_D + NCB,
                       G_C = G_B + NB, G_S = G_C + NCB, G_A = G_S + 4 * SZS * 4,
                       G_M = G_A + 4 * 16 * PA * 4, G_BA = G_M + 4 * 16 * PA * 4,
                       G_BB = G_BA + DKP * 4, G_GP = G_BB + DVP * 4, G_END = G_GP + 4 * DVP * 4;
};

struct BetaArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* z;   // key-gate logits [B, L, H, dk]
  const bf16* w;   // value-gate logits [B, L, H, dv]
  const bf16* r;
  const bf16* dy;
  const float* norm_w;
  bf16* y;
  bf16* o_pre;
  float* obuf;     // fp32 o [B*H][NC*64][dv] (saved), or null
  float* states;   // [B*H][NC][dk][dv] state entering each chunk (after the scan)
  float* dec;      // [B*H][NC][dk + dv] log2 decay of each chunk (key part, value part)
  float* gst;      // backward: [B*H][NC][dk][dv] gradient reaching each chunk's end
  float* dgp;      // backward: [B*H*NC][dv] norm-weight partials
  bf16* dq;
  bf16* dk_;
  bf16* dv_;
  bf16* dz;
  bf16* dw;
  bf16* dr;
  int B, L, H, dk, dv, NC;
  float inv_tau, q_scale, eps;
};

struct ChunkIx {
  int b, h, j, valid;
  long row0;  // element offset of (b, token 64 j, h, 0) divided by the row width
  long bh;
};
// Work items numbered chunk-major (heads fastest), XCD x (workgroup i runs on XCD i mod 8)
// taking the x-th contiguous eighth of them: the heads of a chunk, whose rows share 128-byte
// lines, meet in one L2.
__device__ __forceinline__ ChunkIx chunk_ix(const BetaArgs& p) {
  ChunkIx c;
  const int nbh = p.B * p.H;
  const int item = xcd_item((int)blockIdx.x, (int)gridDim.x);
  c.j = item / nbh;
  c.bh = item - (long)c.j * nbh;
  c.b = (int)(c.bh / p.H);
  c.h = (int)(c.bh - (long)c.b * p.H);
  c.valid = min(kBC, p.L - kBC * c.j);
  c.row0 = ((long)c.b * p.L + (long)kBC * c.j) * p.H + c.h;
  return c;
}

// Rows [0, valid) of a [B, L, H, n] bf16 tensor, for an LDS tile of 64 rows x NP columns
// (pitch P elements), zero elsewhere; row t starts at src + (row0 + t H) n.  load() issues
// every one of the thread's loads unconditionally (indices clamped into the tile's valid
// part; valid >= 1, n >= 1) so that a kernel can issue all its tiles' loads before it waits
// for any; store() selects the zeros and writes the tile.  VEC: pieces of four elements
// (8-byte loads; needs n % 4 == 0 and 8-byte aligned rows), else single elements.
template <int NP, bool VEC>
struct Rows {
  static constexpr int W = VEC ? 4 : 1;  // elements per piece
  static constexpr int NPP = NP / W;     // pieces per row
  static_assert((kBC * NPP) % kBT == 0, "tile must split evenly over the threads");
  static constexpr int N = kBC * NPP / kBT;
  using Piece = typename std::conditional<VEC, uint2, bf16>::type;
  Piece x[N];
  __device__ __forceinline__ void load(const bf16* src, long row0, int H, int n, int valid,
                                       int tid) {
    const int last = n / W - 1;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = tid + j * kBT, t = i / NPP, c = i - t * NPP;
      const bf16* q = src + (row0 + (long)min(t, valid - 1) * H) * n + W * min(c, last);
      x[j] = *reinterpret_cast<const Piece*>(q);
    }
  }
  template <int P, typename T>
  __device__ __forceinline__ void store(T* dst, int n, int valid, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = tid + j * kBT, t = i / NPP, c = i - t * NPP;
      const bool in = t < valid && W * c < n;
      if constexpr (VEC) {
        const bf16* e = reinterpret_cast<const bf16*>(&x[j]);
        if constexpr (sizeof(T) == 2) {
          uint2 z = in ? x[j] : make_uint2(0u, 0u);
          *reinterpret_cast<uint2*>(dst + t * P + W * c) = z;
        } else {
          float4 f;
          f.x = in ? bf(e[0]) : 0.f;
          f.y = in ? bf(e[1]) : 0.f;
          f.z = in ? bf(e[2]) : 0.f;
          f.w = in ? bf(e[3]) : 0.f;
          *reinterpret_cast<float4*>(dst + t * P + W * c) = f;
        }
      } else {
        dst[t * P + c] = from_f<T>(in ? bf(x[j]) : 0.f);
      }
    }
  }
  // In place over the same elements as store<P>(): G holds running sums G[t][c]; each becomes
  // xscale x 2^{dec[c] - G[t][c]} (dec given: the chunk's last row) or xscale x 2^{G[t][c]}
  // (dec null), zero outside the valid part.  A thread touches only its own elements.
  template <int P>
  __device__ __forceinline__ void scale_into(float* G, const float* dec, float xscale, int n,
                                             int valid, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = tid + j * kBT, t = i / NPP, c = i - t * NPP;
      const bool in = t < valid && W * c < n;
      const bf16* e = reinterpret_cast<const bf16*>(&x[j]);
#pragma unroll
      for (int k = 0; k < W; ++k) {
        const int col = W * c + k;
        const float gv = G[t * P + col];
        const float f = fexp2(dec ? dec[col] - gv : gv);
        G[t * P + col] = in ? xscale * bf(e[k]) * f : 0.f;
      }
    }
  }
};
// A [dk][dv] fp32 state for [DKP][P] LDS, zero padded, loaded and stored the same way (VEC:
// 16-byte pieces along a row, dv % 4 == 0; the last thread's surplus pieces repeat the last
// one, which writes the same values twice).
template <int DKP, int DVP, bool VEC>
struct StateRegs {
  static constexpr int W = VEC ? 4 : 1;
  static constexpr int NPP = DVP / W, TOT = DKP * NPP;
  static constexpr int N = (TOT + kBT - 1) / kBT;
  using Piece = typename std::conditional<VEC, float4, float>::type;
  Piece x[N];
  __device__ __forceinline__ void load(const float* src, int dk, int dv, int tid) {
    const int last = dv / W - 1;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = min(tid + j * kBT, TOT - 1), c = i / NPP, e = i - c * NPP;
      x[j] = *reinterpret_cast<const Piece*>(src + (long)min(c, dk - 1) * dv + W * min(e, last));
    }
  }
  template <int P>
  __device__ __forceinline__ void store(float* dst, int dk, int dv, int tid) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = min(tid + j * kBT, TOT - 1), c = i / NPP, e = i - c * NPP;
      const bool in = c < dk && W * e < dv;
      if constexpr (VEC) {
        float4 f = x[j];
        if (!in) f = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(dst + c * P + W * e) = f;
      } else {
        dst[c * P + e] = in ? x[j] : 0.f;
      }
    }
  }
  // elementwise product with another state of the same layout (the boundary sums)
  __device__ __forceinline__ void mul(const StateRegs& o, bool on) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if constexpr (VEC) {
        x[j].x = on ? x[j].x * o.x[j].x : 0.f;
        x[j].y = on ? x[j].y * o.x[j].y : 0.f;
        x[j].z = on ? x[j].z * o.x[j].z : 0.f;
        x[j].w = on ? x[j].w * o.x[j].w : 0.f;
      } else {
        x[j] = on ? x[j] * o.x[j] : 0.f;
      }
    }
  }
};

// In place: the raw logits of columns < n become the inclusive running sums over the chunk's
// rows of log2 sigmoid(.) / tau (rows >= valid add 0).  Lanes = rows; waves take columns.
template <int P>
__device__ __forceinline__ void gate_cumsum(float* s, int n, int valid, float inv_tau, int wave,
                                            int lane) {
  for (int c = wave; c < n; c += 4) {
    float x = lane < valid ? log2_sigmoid(s[lane * P + c]) * inv_tau : 0.f;
    x = scan_dpp<64>(x);
    s[lane * P + c] = x;
  }
}

// Running-sum value at row `ref` (0 for ref < 0: the chunk start).
__device__ __forceinline__ float at_ref(const float* s, int P, int ref, int c) {
  return ref >= 0 ? s[ref * P + c] : 0.f;
}

// acc[ct][et] (lane: rows c = 16 ct + 4 g + i, column e = 16 et + r) =
//   sum_{s in [s0, s0 + 16 NS)} (X[s][c] 2^{GX[end][c] - GX[s][c]}) (Y[s][e] 2^{GY[end][e] - GY[s][e]})
// X, Y given as bf16 (pitch PX/PY) or fp32 rows; GX, GY running sums (pitch PGX/PGY).
template <int NDK, int NDV, int NS, typename TX, int PX, int PGX, typename TY, int PY, int PGY>
__device__ __forceinline__ void outer_sum(f32x4 (&acc)[NDK][NDV], const TX* X, const float* GX,
                                          const TY* Y, const float* GY, int s0, int end,
                                          float xscale, int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ct = 0; ct < NDK; ++ct)
#pragma unroll
    for (int et = 0; et < NDV; ++et) acc[ct][et] = zero4();
#pragma unroll 2
  for (int ks = 0; ks < 4 * NS; ++ks) {
    const int s = s0 + 4 * ks + g;
    float a[NDK], b[NDV];
#pragma unroll
    for (int ct = 0; ct < NDK; ++ct) {
      const int c = 16 * ct + r;
      a[ct] = xscale * to_f(X[s * PX + c]) * fexp2(GX[end * PGX + c] - GX[s * PGX + c]);
    }
#pragma unroll
    for (int et = 0; et < NDV; ++et) {
      const int e = 16 * et + r;
      b[et] = to_f(Y[s * PY + e]) * fexp2(GY[end * PGY + e] - GY[s * PGY + e]);
    }
#pragma unroll
    for (int ct = 0; ct < NDK; ++ct)
#pragma unroll
      for (int et = 0; et < NDV; ++et) acc[ct][et] = mfma_f32(a[ct], b[et], acc[ct][et]);
  }
}

// Whether the products inside this wave's 16-token tile may be factored about the row before
// it: the largest log2 decay of either gate from that row to the tile's last row, over every
// column, is at most kFactorMax (so every factor 2^{B_ref - B_s}, 2^{C_ref - C_s} stays below
// 2^64 and its partner above 2^-64).  Wave-uniform.
constexpr float kFactorMax = 64.f;
template <int DKP, int DVP, int PB, int PC>
__device__ __forceinline__ bool tile_factorable(const float* sB, const float* sC, int t0,
                                                int lane) {
  const int ref = t0 - 1, end = t0 + 15;
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < (DKP + 63) / 64; ++j) {
    const int c = min(lane + 64 * j, DKP - 1);
    d = fmaxf(d, at_ref(sB, PB, ref, c) - sB[end * PB + c]);
  }
#pragma unroll
  for (int j = 0; j < (DVP + 63) / 64; ++j) {
    const int e = min(lane + 64 * j, DVP - 1);
    d = fmaxf(d, at_ref(sC, PC, ref, e) - sC[end * PC + e]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) d = fmaxf(d, __shfl_xor(d, off));
  return __builtin_amdgcn_readfirstlane((int)(d <= kFactorMax)) != 0;
}

template <int P, int NDK, int NDV>
__device__ __forceinline__ void store_tiles(float* dst, const f32x4 (&acc)[NDK][NDV], int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ct = 0; ct < NDK; ++ct)
#pragma unroll
    for (int et = 0; et < NDV; ++et)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * ct + 4 * g + i) * P + 16 * et + r] = acc[ct][et][i];
}

// Output-stage backward for the rows t = 16 w + 4 g + i of this lane, columns e = 16 E + r:
// dO = rstd (dn - n mean(dn n)), dn = dy norm_w Swish(r), n = o rstd, from the saved fp32 o.
// With EXTRA also dr (stored) and the per-column sums of dy n Swish(r) (gp) and do.o (od).
template <int NDV, bool EXTRA>
__device__ __forceinline__ void out_stage_bwd(const BetaArgs& p, const ChunkIx& ci, int w,
                                              int lane, float (&dO)[NDV][4], float (&od)[NDV][4],
                                              float (&gp)[NDV]) {
  const int r = lane & 15, g = lane >> 4;
  const float inv_dv = 1.f / (float)p.dv;
  float o[NDV][4], dn[NDV][4], sg[NDV][4], rr[NDV][4], dyv[NDV][4];
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
  const float* obase = p.obuf + ((ci.bh * p.NC + ci.j) * (long)kBC) * p.dv;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 16 * w + 4 * g + i;
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      const int e = 16 * E + r;
      const bool in = t < ci.valid && e < p.dv;
      const int tc = min(t, ci.valid - 1), ec = min(e, p.dv - 1);
      const long gi = (ci.row0 + (long)tc * p.H) * p.dv + ec;
      const float ov = obase[(long)tc * p.dv + ec], rv = bf(p.r[gi]), dv = bf(p.dy[gi]);
      o[E][i] = in ? ov : 0.f;
      rr[E][i] = in ? rv : 0.f;
      dyv[E][i] = in ? dv : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      ss[i] += o[E][i] * o[E][i];
    }
  }
  float nwv[NDV];
#pragma unroll
  for (int E = 0; E < NDV; ++E) nwv[E] = p.norm_w ? p.norm_w[min(16 * E + r, p.dv - 1)] : 1.f;
  float rstd[4], m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) rstd[i] = rsqrtf(row_sum16(ss[i]) * inv_dv + p.eps);
#pragma unroll
  for (int E = 0; E < NDV; ++E) {
    const int e = 16 * E + r;
    const float nw = (p.norm_w && e < p.dv) ? nwv[E] : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sg[E][i] = fast_sigmoid(rr[E][i]);
      const float s = rr[E][i] * sg[E][i];
      dn[E][i] = dyv[E][i] * nw * s;
      m[i] += dn[E][i] * o[E][i] * rstd[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = row_sum16(m[i]) * inv_dv;
#pragma unroll
  for (int E = 0; E < NDV; ++E) {
    const int e = 16 * E + r;
    const float nw = (p.norm_w && e < p.dv) ? nwv[E] : 1.f;
    float gsum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * g + i;
      const float n = o[E][i] * rstd[i];
      dO[E][i] = rstd[i] * (dn[E][i] - n * m[i]);
      if constexpr (EXTRA) {
        od[E][i] = dO[E][i] * o[E][i];
        const float s = rr[E][i] * sg[E][i];
        gsum += dyv[E][i] * n * s;
        if (t < ci.valid && e < p.dv) {
          const float d = dyv[E][i] * n * nw * sg[E][i] * (1.f + rr[E][i] * (1.f - sg[E][i]));
          p.dr[(ci.row0 + (long)t * p.H) * p.dv + e] = from_f<bf16>(d);
        }
      }
    }
    if constexpr (EXTRA) gp[E] = gsum;
  }
}

// ------------------------------------------------------------------------- pass 1 (forward)
// Each chunk's state contribution U (relative to its last row) and its log2 decays.
template <int NDK, int NDV, bool VEC>
__global__ __launch_bounds__(kBT) void beta_fwd_state(BetaArgs p) {
  using Lo = BetaLay<NDK, NDV>;
  constexpr int DKP = Lo::DKP, DVP = Lo::DVP, PB = Lo::PB, PC = Lo::PC;
  extern __shared__ __align__(16) unsigned char smem[];
  float* sB = reinterpret_cast<float*>(smem + Lo::U_B);  // key-gate sums, then k scaled
  float* sC = reinterpret_cast<float*>(smem + Lo::U_C);  // value-gate sums, then v scaled
  float* sD = reinterpret_cast<float*>(smem + Lo::U_D);  // the sums' last row (the decays)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const ChunkIx ci = chunk_ix(p);
  Rows<DKP, VEC> xk;
  Rows<DVP, VEC> xv;
  {
    Rows<DKP, VEC> xz;
    Rows<DVP, VEC> xw;
    xk.load(p.k, ci.row0, p.H, p.dk, ci.valid, tid);
    xv.load(p.v, ci.row0, p.H, p.dv, ci.valid, tid);
    xz.load(p.z, ci.row0, p.H, p.dk, ci.valid, tid);
    xw.load(p.w, ci.row0, p.H, p.dv, ci.valid, tid);
    xz.template store<PB>(sB, p.dk, ci.valid, tid);
    xw.template store<PC>(sC, p.dv, ci.valid, tid);
  }
  __syncthreads();
  gate_cumsum<PB>(sB, p.dk, ci.valid, p.inv_tau, wave, lane);
  gate_cumsum<PC>(sC, p.dv, ci.valid, p.inv_tau, wave, lane);
  __syncthreads();
  for (int i = tid; i < DKP + DVP; i += kBT)
    sD[i] = i < DKP ? sB[(kBC - 1) * PB + i] : sC[(kBC - 1) * PC + (i - DKP)];
  __syncthreads();
  const long slot = ci.bh * p.NC + ci.j;
  const int r = lane & 15, g = lane >> 4;
  // k_s 2^{B_end - B_s} over B and v_s 2^{C_end - C_s} over C, in place (the thread that staged
  // an element of z or w holds the same element of k or v)
  xk.template scale_into<PB>(sB, sD, 1.f, p.dk, ci.valid, tid);
  xv.template scale_into<PC>(sC, sD + DKP, 1.f, p.dv, ci.valid, tid);
  __syncthreads();
  const float* sX = sB;
  const float* sY = sC;
  for (int u = wave; u < NDK * NDV; u += 4) {
    const int ct = u / NDV, et = u - ct * NDV;
    const int c = 16 * ct + r, e = 16 * et + r;
    f32x4 acc = zero4();
#pragma unroll 8
    for (int ks = 0; ks < kBC / 4; ++ks) {
      const int s = 4 * ks + g;
      acc = mfma_f32(sX[s * PB + c], sY[s * PC + e], acc);
    }
    float* dst = p.states + slot * p.dk * p.dv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cc = 16 * ct + 4 * g + i;
      if (cc < p.dk && e < p.dv) dst[(long)cc * p.dv + e] = acc[i];
    }
  }
  for (int i = tid; i < p.dk + p.dv; i += kBT)
    p.dec[slot * (p.dk + p.dv) + i] = i < p.dk ? sD[i] : sD[DKP + (i - p.dk)];
}

// ----------------------------------------------------------------------- pass 2 (both ways)
// In place over chunks, per (image, head) and state element (c, e):
//   forward:  slot j <- S entering chunk j;  S <- 2^{dec_j[c] + dec_j[e]} S + U_j
//   reverse:  slot j <- G reaching chunk j's end;  G <- 2^{dec_j[c] + dec_j[e]} G + dU_j
constexpr int kScanBatch = 64;
__global__ __launch_bounds__(256) void beta_scan(float* st, const float* dec, int NC, int dk,
                                                 int dv, int reverse) {
  const long bh = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= dk * dv) return;
  const int c = idx / dv, e = idx - c * dv;
  const long sz = (long)dk * dv;
  float* base = st + bh * NC * sz + idx;
  const float* d = dec + bh * NC * (dk + dv);
  float S = 0.f;
  for (int j0 = 0; j0 < NC; j0 += kScanBatch) {
    float u[kScanBatch], f[kScanBatch];
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) {
      const int jj = min(j0 + i, NC - 1);
      const int j = reverse ? NC - 1 - jj : jj;
      u[i] = base[j * sz];
      f[i] = d[(long)j * (dk + dv) + c] + d[(long)j * (dk + dv) + dk + e];
    }
#pragma unroll
    for (int i = 0; i < kScanBatch; ++i) {
      if (j0 + i < NC) {
        const int j = reverse ? NC - 1 - (j0 + i) : j0 + i;
        base[j * sz] = S;
        S = fexp2(f[i]) * S + u[i];
      }
    }
  }
}

// --------------------------------------------------------------------- pass 3 (forward)
template <int NDK, int NDV, bool VEC>
__global__ __launch_bounds__(kBT) void beta_fwd_out(BetaArgs p) {
  using Lo = BetaLay<NDK, NDV>;
  constexpr int DKP = Lo::DKP, DVP = Lo::DVP, PQ = Lo::PQ, PV = Lo::PV, PB = Lo::PB,
                PC = Lo::PC, PA = Lo::PA, SZS = Lo::SZS;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* sQ = reinterpret_cast<bf16*>(smem + Lo::F_Q);
  bf16* sK = reinterpret_cast<bf16*>(smem + Lo::F_K);
  bf16* sV = reinterpret_cast<bf16*>(smem + Lo::F_V);
  float* sB = reinterpret_cast<float*>(smem + Lo::F_B);
  float* sC = reinterpret_cast<float*>(smem + Lo::F_C);
  float* sS = reinterpret_cast<float*>(smem + Lo::F_S);  // S_0..S_3
  float* sA = reinterpret_cast<float*>(smem + Lo::F_A);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const ChunkIx ci = chunk_ix(p);
  const long slot = ci.bh * p.NC + ci.j;
  bf16 rpre[NDV][4];
  float nwv[NDV];
  {
    Rows<DKP, VEC> xq, xk, xz;
    Rows<DVP, VEC> xv, xw;
    StateRegs<DKP, DVP, VEC> xs;
    xq.load(p.q, ci.row0, p.H, p.dk, ci.valid, tid);
    xk.load(p.k, ci.row0, p.H, p.dk, ci.valid, tid);
    xv.load(p.v, ci.row0, p.H, p.dv, ci.valid, tid);
    xz.load(p.z, ci.row0, p.H, p.dk, ci.valid, tid);
    xw.load(p.w, ci.row0, p.H, p.dv, ci.valid, tid);
    xs.load(p.states + slot * p.dk * p.dv, p.dk, p.dv, tid);
    // r and the norm weight for the output stage (this lane's rows and columns)
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      const int ec = min(16 * E + r, p.dv - 1);
      nwv[E] = p.norm_w ? p.norm_w[ec] : 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tc = min(16 * wave + 4 * g + i, ci.valid - 1);
        rpre[E][i] = p.r[(ci.row0 + (long)tc * p.H) * p.dv + ec];
      }
    }
    xq.template store<PQ>(sQ, p.dk, ci.valid, tid);
    xk.template store<PQ>(sK, p.dk, ci.valid, tid);
    xv.template store<PV>(sV, p.dv, ci.valid, tid);
    xz.template store<PB>(sB, p.dk, ci.valid, tid);
    xw.template store<PC>(sC, p.dv, ci.valid, tid);
    xs.template store<PC>(sS, p.dk, p.dv, tid);
  }
  __syncthreads();
  gate_cumsum<PB>(sB, p.dk, ci.valid, p.inv_tau, wave, lane);
  gate_cumsum<PC>(sC, p.dv, ci.valid, p.inv_tau, wave, lane);
  __syncthreads();
  // tile contributions U_0..U_2 (relative to each tile's last row) into S_1..S_3
  if (wave < 3) {
    f32x4 acc[NDK][NDV];
    outer_sum<NDK, NDV, 1, bf16, PQ, PB, bf16, PV, PC>(acc, sK, sB, sV, sC, 16 * wave,
                                                         16 * wave + 15, 1.f, lane);
    store_tiles<PC>(sS + (wave + 1) * SZS, acc, lane);
  }
  __syncthreads();
  // S_{w+1} = 2^{B_w + C_w} S_w + U_w, elementwise, each thread the same elements throughout
  for (int i = tid; i < DKP * DVP; i += kBT) {
    const int c = i / DVP, e = i - c * DVP;
    float S = sS[c * PC + e];
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      const float d = (sB[(16 * w + 15) * PB + c] - at_ref(sB, PB, 16 * w - 1, c)) +
                      (sC[(16 * w + 15) * PC + e] - at_ref(sC, PC, 16 * w - 1, e));
      S = fexp2(d) * S + sS[(w + 1) * SZS + c * PC + e];
      sS[(w + 1) * SZS + c * PC + e] = S;
    }
  }
  __syncthreads();
  const int w = wave, t0 = 16 * w, ref = t0 - 1;
  const bool fast = tile_factorable<DKP, DVP, PB, PC>(sB, sC, t0, lane);
  // across tiles: (q_t 2^{B_t - B_ref}) S_w
  f32x4 acc[NDV];
  float a[DKP / 4];  // A operand: q_scale q_t 2^{B_t - B_ref}, t = t0 + r, c = 4 ks + g
#pragma unroll
  for (int ks = 0; ks < DKP / 4; ++ks) {
    const int c = 4 * ks + g, t = t0 + r;
    a[ks] = p.q_scale * bf(sQ[t * PQ + c]) * fexp2(sB[t * PB + c] - at_ref(sB, PB, ref, c));
  }
  {
    const float* S = sS + w * SZS;
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      acc[E] = zero4();
#pragma unroll
      for (int ks = 0; ks < DKP / 4; ++ks)
        acc[E] = mfma_f32(a[ks], S[(4 * ks + g) * PC + 16 * E + r], acc[E]);
    }
  }
  if (fast) {
    // inside the tile, factored about the row before it (every factor within 2^64):
    // A^T = Khat Qhat^T with Khat_s = k_s 2^{B_ref - B_s}; this lane holds A[t0 + r][t0 + 4 g + i]
    f32x4 at = zero4();
#pragma unroll
    for (int ks = 0; ks < DKP / 4; ++ks) {
      const int c = 4 * ks + g, s = t0 + r;
      const float kh = bf(sK[s * PQ + c]) * fexp2(at_ref(sB, PB, ref, c) - sB[s * PB + c]);
      at = mfma_f32(kh, a[ks], at);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) at[i] = (4 * g + i <= r) ? at[i] : 0.f;
    // o_t += sum_s A[t][s] Vhat_s, Vhat_s = v_s 2^{C_ref - C_s} (k step i: s = t0 + 4 g + i)
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      const int e = 16 * E + r;
      const float cr = at_ref(sC, PC, ref, e);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = t0 + 4 * g + i;
        acc[E] = mfma_f32(at[i], bf(sV[s * PV + e]) * fexp2(cr - sC[s * PC + e]), acc[E]);
      }
    }
  }
  // then 2^{C_t - C_ref}
#pragma unroll
  for (int E = 0; E < NDV; ++E)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i, e = 16 * E + r;
      acc[E][i] *= fexp2(sC[t * PC + e] - at_ref(sC, PC, ref, e));
    }
  // inside a tile with stronger decay: pair weights A[t][s] = q_scale sum_c q_t k_s 2^{B_t - B_s},
  // s <= t, each with its own factor
  float* myA = sA + w * 16 * PA;
  if (!fast) {
    const int tl = r, sg = 4 * g;
    float pa[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = 0; c < DKP; ++c) {
      const float qv = bf(sQ[(t0 + tl) * PQ + c]), bt = sB[(t0 + tl) * PB + c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = t0 + sg + i;
        pa[i] += qv * bf(sK[s * PQ + c]) * fexp2(fminf(bt - sB[s * PB + c], 0.f));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) myA[tl * PA + sg + i] = (sg + i <= tl) ? p.q_scale * pa[i] : 0.f;
  }
  __syncthreads();
  // o_t += sum_{s <= t in tile} A[t][s] v_s 2^{C_t - C_s}
  if (!fast) {
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      const int e = 16 * E + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = 4 * g + i, t = t0 + tl;
        const float ct = sC[t * PC + e];
        float sum = 0.f;
        for (int sl = 0; sl <= 12 + i; ++sl) {
          const int s = t0 + sl;
          const float term = myA[tl * PA + sl] * bf(sV[s * PV + e]) *
                             fexp2(fminf(ct - sC[s * PC + e], 0.f));
          sum += sl <= tl ? term : 0.f;
        }
        acc[E][i] += sum;
      }
    }
  }
  // output stage
  const float inv_dv = 1.f / (float)p.dv;
  float rstd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int E = 0; E < NDV; ++E) ss += acc[E][i] * acc[E][i];
    rstd[i] = rsqrtf(row_sum16(ss) * inv_dv + p.eps);
  }
  float* obase = p.obuf ? p.obuf + (slot * (long)kBC) * p.dv : nullptr;
#pragma unroll
  for (int E = 0; E < NDV; ++E) {
    const int e = 16 * E + r;
    if (e >= p.dv) continue;
    const float nw = nwv[E];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      if (t >= ci.valid) continue;
      const long gi = (ci.row0 + (long)t * p.H) * p.dv + e;
      const float o = acc[E][i];
      if (obase) obase[(long)t * p.dv + e] = o;
      if (p.o_pre) p.o_pre[gi] = from_f<bf16>(o);
      const float rv = bf(rpre[E][i]);
      p.y[gi] = from_f<bf16>(o * rstd[i] * nw * rv * fast_sigmoid(rv));
    }
  }
}

// ------------------------------------------------------------------------ pass 1 (backward)
// Each chunk's gradient-state contribution dU = sum_t (q_scale q_t 2^{B_t})^T (dO_t 2^{C_t})
// (relative to the chunk start) and its log2 decays.
template <int NDK, int NDV, bool VEC>
__global__ __launch_bounds__(kBT) __attribute__((amdgpu_waves_per_eu(VEC ? 4 : 1))) void beta_bwd_state(
    BetaArgs p) {
  using Lo = BetaLay<NDK, NDV>;
  constexpr int DKP = Lo::DKP, DVP = Lo::DVP, PB = Lo::PB, PC = Lo::PC;
  extern __shared__ __align__(16) unsigned char smem[];
  float* sB = reinterpret_cast<float*>(smem + Lo::U_B);  // key-gate sums, then q scaled
  float* sC = reinterpret_cast<float*>(smem + Lo::U_C);  // value-gate sums, then dO scaled
  float* sD = reinterpret_cast<float*>(smem + Lo::U_D);  // the sums' last row (the decays)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const ChunkIx ci = chunk_ix(p);
  Rows<DKP, VEC> xq;
  {
    Rows<DKP, VEC> xz;
    Rows<DVP, VEC> xw;
    xq.load(p.q, ci.row0, p.H, p.dk, ci.valid, tid);
    xz.load(p.z, ci.row0, p.H, p.dk, ci.valid, tid);
    xw.load(p.w, ci.row0, p.H, p.dv, ci.valid, tid);
    xz.template store<PB>(sB, p.dk, ci.valid, tid);
    xw.template store<PC>(sC, p.dv, ci.valid, tid);
  }
  float dO[NDV][4];
  {
    float od[NDV][4], gp[NDV];
    out_stage_bwd<NDV, false>(p, ci, wave, lane, dO, od, gp);
  }
  __syncthreads();
  gate_cumsum<PB>(sB, p.dk, ci.valid, p.inv_tau, wave, lane);
  gate_cumsum<PC>(sC, p.dv, ci.valid, p.inv_tau, wave, lane);
  __syncthreads();
  for (int i = tid; i < DKP + DVP; i += kBT)
    sD[i] = i < DKP ? sB[(kBC - 1) * PB + i] : sC[(kBC - 1) * PC + (i - DKP)];
  __syncthreads();
  const long slot = ci.bh * p.NC + ci.j;
  // q_scale q_t 2^{B_t} over B and dO_t 2^{C_t} over C, in place (each thread its own elements:
  // q as staged, dO as the output-stage backward left it in this lane)
  xq.template scale_into<PB>(sB, nullptr, p.q_scale, p.dk, ci.valid, tid);
#pragma unroll
  for (int E = 0; E < NDV; ++E)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* cp = sC + (16 * wave + 4 * g + i) * PC + 16 * E + r;
      *cp = dO[E][i] * fexp2(*cp);
    }
  __syncthreads();
  const float* sX = sB;
  const float* sY = sC;
  for (int u = wave; u < NDK * NDV; u += 4) {
    const int ct = u / NDV, et = u - ct * NDV;
    f32x4 acc = zero4();
    {
      const int c = 16 * ct + r, e = 16 * et + r;
#pragma unroll 8
      for (int ks = 0; ks < kBC / 4; ++ks) {
        const int s = 4 * ks + g;
        acc = mfma_f32(sX[s * PB + c], sY[s * PC + e], acc);
      }
    }
    float* dst = p.gst + slot * p.dk * p.dv;
    const int e = 16 * et + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * ct + 4 * g + i;
      if (c < p.dk && e < p.dv) dst[(long)c * p.dv + e] = acc[i];
    }
  }
  for (int i = tid; i < p.dk + p.dv; i += kBT)
    p.dec[slot * (p.dk + p.dv) + i] = i < p.dk ? sD[i] : sD[DKP + (i - p.dk)];
}

// ------------------------------------------------------------------------ pass 3 (backward)
template <int NDK, int NDV, bool VEC>
__global__ __launch_bounds__(kBT) void beta_bwd_out(BetaArgs p) {
  using Lo = BetaLay<NDK, NDV>;
  constexpr int DKP = Lo::DKP, DVP = Lo::DVP, PQ = Lo::PQ, PV = Lo::PV, PB = Lo::PB,
                PC = Lo::PC, PA = Lo::PA, SZS = Lo::SZS;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* sQ = reinterpret_cast<bf16*>(smem + Lo::G_Q);
  bf16* sK = reinterpret_cast<bf16*>(smem + Lo::G_K);
  bf16* sV = reinterpret_cast<bf16*>(smem + Lo::G_V);
  float* sD = reinterpret_cast<float*>(smem + Lo::G_D);  // dO
  float* sB = reinterpret_cast<float*>(smem + Lo::G_B);
  float* sC = reinterpret_cast<float*>(smem + Lo::G_C);
  float* sS = reinterpret_cast<float*>(smem + Lo::G_S);  // S_0..S_3, then G_0..G_3
  float* sA = reinterpret_cast<float*>(smem + Lo::G_A);
  float* sM = reinterpret_cast<float*>(smem + Lo::G_M);
  float* sBa = reinterpret_cast<float*>(smem + Lo::G_BA);
  float* sBb = reinterpret_cast<float*>(smem + Lo::G_BB);
  float* sGp = reinterpret_cast<float*>(smem + Lo::G_GP);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const ChunkIx ci = chunk_ix(p);
  const long slot = ci.bh * p.NC + ci.j;
  const long sz = (long)p.dk * p.dv;
  const int w = wave, t0 = 16 * w, ref = t0 - 1, end = t0 + 15;
  const bool has_end = ci.j + 1 < p.NC;
  {
    Rows<DKP, VEC> xq, xk, xz;
    Rows<DVP, VEC> xv, xw;
    StateRegs<DKP, DVP, VEC> xs;
    xq.load(p.q, ci.row0, p.H, p.dk, ci.valid, tid);
    xk.load(p.k, ci.row0, p.H, p.dk, ci.valid, tid);
    xv.load(p.v, ci.row0, p.H, p.dv, ci.valid, tid);
    xz.load(p.z, ci.row0, p.H, p.dk, ci.valid, tid);
    xw.load(p.w, ci.row0, p.H, p.dv, ci.valid, tid);
    xs.load(p.states + slot * sz, p.dk, p.dv, tid);
    // the state leaving the chunk (the next chunk's entering state) and the gradient reaching
    // the chunk's end, for the boundary sums; the last chunk has none (zero products)
    StateRegs<DKP, DVP, VEC> xe, xg;
    xe.load(p.states + (has_end ? slot + 1 : slot) * sz, p.dk, p.dv, tid);
    xg.load(p.gst + slot * sz, p.dk, p.dv, tid);
    xe.mul(xg, has_end);
    xe.template store<PC>(sS + 3 * SZS, p.dk, p.dv, tid);
    xq.template store<PQ>(sQ, p.dk, ci.valid, tid);
    xk.template store<PQ>(sK, p.dk, ci.valid, tid);
    xv.template store<PV>(sV, p.dv, ci.valid, tid);
    xz.template store<PB>(sB, p.dk, ci.valid, tid);
    xw.template store<PC>(sC, p.dv, ci.valid, tid);
    xs.template store<PC>(sS, p.dk, p.dv, tid);
  }
  float od[NDV][4];
  {
    float dO[NDV][4], gp[NDV];
    out_stage_bwd<NDV, true>(p, ci, w, lane, dO, od, gp);
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sD[(t0 + 4 * g + i) * PC + 16 * E + r] = dO[E][i];
      // norm-weight partial: this wave's 16 rows, summed over the lane groups below
      float x = gp[E];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      if (g == 0) sGp[w * DVP + 16 * E + r] = x;
    }
  }
  // boundary sums of S_end (.) G_end (staged in slot 3, zero padded) over value columns (per
  // key column) and over key columns (per value column)
  __syncthreads();
  if (tid < DKP) {
    const float* row = sS + 3 * SZS + tid * PC;
    float x = 0.f;
#pragma unroll 8
    for (int e = 0; e < DVP; ++e) x += row[e];
    sBa[tid] = x;
  } else if (tid < DKP + DVP) {
    const int e = tid - DKP;
    const float* col = sS + 3 * SZS + e;
    float x = 0.f;
#pragma unroll 8
    for (int c = 0; c < DKP; ++c) x += col[c * PC];
    sBb[e] = x;
  }
  __syncthreads();
  if (tid < DVP && p.dgp && tid < p.dv)
    p.dgp[slot * p.dv + tid] = (sGp[tid] + sGp[DVP + tid]) + (sGp[2 * DVP + tid] + sGp[3 * DVP + tid]);
  gate_cumsum<PB>(sB, p.dk, ci.valid, p.inv_tau, wave, lane);
  gate_cumsum<PC>(sC, p.dv, ci.valid, p.inv_tau, wave, lane);
  __syncthreads();

  // ---- forward tile states S_1..S_3 (as in the forward output pass)
  if (w < 3) {
    f32x4 acc[NDK][NDV];
    outer_sum<NDK, NDV, 1, bf16, PQ, PB, bf16, PV, PC>(acc, sK, sB, sV, sC, t0, end, 1.f, lane);
    store_tiles<PC>(sS + (w + 1) * SZS, acc, lane);
  }
  __syncthreads();
  for (int i = tid; i < DKP * DVP; i += kBT) {
    const int c = i / DVP, e = i - c * DVP;
    float S = sS[c * PC + e];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const float d = (sB[(16 * u + 15) * PB + c] - at_ref(sB, PB, 16 * u - 1, c)) +
                      (sC[(16 * u + 15) * PC + e] - at_ref(sC, PC, 16 * u - 1, e));
      S = fexp2(d) * S + sS[(u + 1) * SZS + c * PC + e];
      sS[(u + 1) * SZS + c * PC + e] = S;
    }
  }
  __syncthreads();
  // dq across tiles: q_scale 2^{B_t - B_ref} sum_e (dO_t 2^{C_t - C_ref})[e] S_w[c][e]
  f32x4 dqa[NDK];
  {
    float a[DVP / 4];
#pragma unroll
    for (int ks = 0; ks < DVP / 4; ++ks) {
      const int e = 4 * ks + g, t = t0 + r;
      a[ks] = sD[t * PC + e] * fexp2(sC[t * PC + e] - at_ref(sC, PC, ref, e));
    }
    const float* S = sS + w * SZS;
#pragma unroll
    for (int ct = 0; ct < NDK; ++ct) {
      dqa[ct] = zero4();
#pragma unroll
      for (int ks = 0; ks < DVP / 4; ++ks)
        dqa[ct] = mfma_f32(a[ks], S[(16 * ct + r) * PC + 4 * ks + g], dqa[ct]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * g + i, c = 16 * ct + r;
        dqa[ct][i] *= p.q_scale * fexp2(sB[t * PB + c] - at_ref(sB, PB, ref, c));
      }
    }
  }
  __syncthreads();  // every read of S_w done
  // ---- gradient tile states: G_3 = gradient reaching the chunk's end; tile contributions
  // dU_1..dU_3 (relative to each tile's start) into slots 0..2; then
  // G_{u-1} = 2^{B_u + C_u} G_u + dU_u
  {
    StateRegs<DKP, DVP, VEC> xg;
    xg.load(p.gst + slot * sz, p.dk, p.dv, tid);
    xg.template store<PC>(sS + 3 * SZS, p.dk, p.dv, tid);
  }
  if (w >= 1) {
    const int s0 = t0, rf = t0 - 1;
    const int r_ = lane & 15, g_ = lane >> 4;
    f32x4 acc[NDK][NDV];
#pragma unroll
    for (int ct = 0; ct < NDK; ++ct)
#pragma unroll
      for (int et = 0; et < NDV; ++et) acc[ct][et] = zero4();
#pragma unroll 2
    for (int ks = 0; ks < 4; ++ks) {
      const int t = s0 + 4 * ks + g_;
      float a[NDK], b[NDV];
#pragma unroll
      for (int ct = 0; ct < NDK; ++ct) {
        const int c = 16 * ct + r_;
        a[ct] = p.q_scale * bf(sQ[t * PQ + c]) * fexp2(sB[t * PB + c] - sB[rf * PB + c]);
      }
#pragma unroll
      for (int et = 0; et < NDV; ++et) {
        const int e = 16 * et + r_;
        b[et] = sD[t * PC + e] * fexp2(sC[t * PC + e] - sC[rf * PC + e]);
      }
#pragma unroll
      for (int ct = 0; ct < NDK; ++ct)
#pragma unroll
        for (int et = 0; et < NDV; ++et) acc[ct][et] = mfma_f32(a[ct], b[et], acc[ct][et]);
    }
    store_tiles<PC>(sS + (w - 1) * SZS, acc, lane);
  }
  __syncthreads();
  for (int i = tid; i < DKP * DVP; i += kBT) {
    const int c = i / DVP, e = i - c * DVP;
    float G = sS[3 * SZS + c * PC + e];
#pragma unroll
    for (int u = 3; u >= 1; --u) {
      const float d = (sB[(16 * u + 15) * PB + c] - sB[(16 * u - 1) * PB + c]) +
                      (sC[(16 * u + 15) * PC + e] - sC[(16 * u - 1) * PC + e]);
      G = fexp2(d) * G + sS[(u - 1) * SZS + c * PC + e];
      sS[(u - 1) * SZS + c * PC + e] = G;
    }
  }
  __syncthreads();
  // dk, dv across tiles from G_w (gradient reaching the tile's last row):
  //   dk_s[c] = 2^{B_end - B_s} sum_e (v_s 2^{C_end - C_s})[e] G_w[c][e]
  //   dv_s[e] = 2^{C_end - C_s} sum_c (k_s 2^{B_end - B_s})[c] G_w[c][e]
  f32x4 dka[NDK], dva[NDV];
  {
    const float* G = sS + w * SZS;
    float a[DVP / 4];
#pragma unroll
    for (int ks = 0; ks < DVP / 4; ++ks) {
      const int e = 4 * ks + g, s = t0 + r;
      a[ks] = bf(sV[s * PV + e]) * fexp2(sC[end * PC + e] - sC[s * PC + e]);
    }
#pragma unroll
    for (int ct = 0; ct < NDK; ++ct) {
      dka[ct] = zero4();
#pragma unroll
      for (int ks = 0; ks < DVP / 4; ++ks)
        dka[ct] = mfma_f32(a[ks], G[(16 * ct + r) * PC + 4 * ks + g], dka[ct]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = t0 + 4 * g + i, c = 16 * ct + r;
        dka[ct][i] *= fexp2(sB[end * PB + c] - sB[s * PB + c]);
      }
    }
    float b[DKP / 4];
#pragma unroll
    for (int ks = 0; ks < DKP / 4; ++ks) {
      const int c = 4 * ks + g, s = t0 + r;
      b[ks] = bf(sK[s * PQ + c]) * fexp2(sB[end * PB + c] - sB[s * PB + c]);
    }
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      dva[E] = zero4();
#pragma unroll
      for (int ks = 0; ks < DKP / 4; ++ks)
        dva[E] = mfma_f32(b[ks], G[(4 * ks + g) * PC + 16 * E + r], dva[E]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = t0 + 4 * g + i, e = 16 * E + r;
        dva[E][i] *= fexp2(sC[end * PC + e] - sC[s * PC + e]);
      }
    }
  }
  // ---- inside the tile.  Where both gates' decay across the tile stays within 2^64 the
  // products are factored about the row before the tile (ref) and run on the matrix cores:
  //   Qhat_t = q_scale q_t 2^{B_t - B_ref}, Khat_s = k_s 2^{B_ref - B_s},
  //   dOhat_t = dO_t 2^{C_t - C_ref},       Vhat_s = v_s 2^{C_ref - C_s},
  //   A = Qhat Khat^T, M = dOhat Vhat^T (causal), dq += q_scale 2^{B_t - B_ref} (M Khat),
  //   dk += 2^{B_ref - B_s} (M^T Qhat), dv += 2^{C_ref - C_s} (A^T dOhat);
  // otherwise every pair takes its own factors (pair tables below).
  const bool fast = tile_factorable<DKP, DVP, PB, PC>(sB, sC, t0, lane);
  if (fast) {
    // A and M in this lane's accumulator order ([t0 + 4 g + i][t0 + r]) and M transposed
    // ([t0 + r][t0 + 4 g + i]); operands of row t0 + r, column 4 ks + g
    f32x4 an = zero4(), mn = zero4(), mt = zero4();
    {
      const int t = t0 + r;
#pragma unroll 2
      for (int ks = 0; ks < DKP / 4; ++ks) {
        const int c = 4 * ks + g;
        const float br = at_ref(sB, PB, ref, c), bt = sB[t * PB + c];
        const float qh = p.q_scale * bf(sQ[t * PQ + c]) * fexp2(bt - br);
        const float kh = bf(sK[t * PQ + c]) * fexp2(br - bt);
        an = mfma_f32(qh, kh, an);
      }
#pragma unroll 2
      for (int ks = 0; ks < DVP / 4; ++ks) {
        const int e = 4 * ks + g;
        const float cr = at_ref(sC, PC, ref, e), cv = sC[t * PC + e];
        const float dh = sD[t * PC + e] * fexp2(cv - cr);
        const float vh = bf(sV[t * PV + e]) * fexp2(cr - cv);
        mn = mfma_f32(dh, vh, mn);
        mt = mfma_f32(vh, dh, mt);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool nat = r <= 4 * g + i;  // s = t0 + r <= t = t0 + 4 g + i
      an[i] = nat ? an[i] : 0.f;
      mn[i] = nat ? mn[i] : 0.f;
      mt[i] = (4 * g + i <= r) ? mt[i] : 0.f;
    }
    // k step i: the contracted row is t0 + 4 g + i
#pragma unroll
    for (int ct = 0; ct < NDK; ++ct) {
      const int c = 16 * ct + r;
      const float br = at_ref(sB, PB, ref, c);
      f32x4 xq = zero4(), xk = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int u = t0 + 4 * g + i;
        const float bu = sB[u * PB + c];
        xq = mfma_f32(mt[i], bf(sK[u * PQ + c]) * fexp2(br - bu), xq);              // M Khat
        xk = mfma_f32(mn[i], p.q_scale * bf(sQ[u * PQ + c]) * fexp2(bu - br), xk);  // M^T Qhat
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bx = sB[(t0 + 4 * g + i) * PB + c];
        dqa[ct][i] += p.q_scale * fexp2(bx - br) * xq[i];
        dka[ct][i] += fexp2(br - bx) * xk[i];
      }
    }
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      const int e = 16 * E + r;
      const float cr = at_ref(sC, PC, ref, e);
      f32x4 xv = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int u = t0 + 4 * g + i;
        xv = mfma_f32(an[i], sD[u * PC + e] * fexp2(sC[u * PC + e] - cr), xv);      // A^T dOhat
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float cx = sC[(t0 + 4 * g + i) * PC + e];
        dva[E][i] += fexp2(cr - cx) * xv[i];
      }
    }
  } else {
    // pair tables A[t][s] (q_scale included) and M[t][s] = sum_e dO_t v_s 2^{C_t - C_s}, s <= t
    float* myA = sA + w * 16 * PA;
    float* myM = sM + w * 16 * PA;
    const int tl = r, sg = 4 * g, t = t0 + tl;
    float pa[4] = {0.f, 0.f, 0.f, 0.f}, pm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = 0; c < DKP; ++c) {
      const float qv = bf(sQ[t * PQ + c]), bt = sB[t * PB + c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = t0 + sg + i;
        pa[i] += qv * bf(sK[s * PQ + c]) * fexp2(fminf(bt - sB[s * PB + c], 0.f));
      }
    }
#pragma unroll 4
    for (int e = 0; e < DVP; ++e) {
      const float dov = sD[t * PC + e], ctv = sC[t * PC + e];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = t0 + sg + i;
        pm[i] += dov * bf(sV[s * PV + e]) * fexp2(fminf(ctv - sC[s * PC + e], 0.f));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool on = sg + i <= tl;
      myA[tl * PA + sg + i] = on ? p.q_scale * pa[i] : 0.f;
      myM[tl * PA + sg + i] = on ? pm[i] : 0.f;
    }
    // the tables are this wave's own: its LDS accesses complete in order
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // dq_t[c] += q_scale sum_{s <= t} M[t][s] k_s[c] 2^{B_t - B_s}
    // dk_s[c] += q_scale sum_{t >= s} M[t][s] q_t[c] 2^{B_t - B_s}
#pragma unroll
    for (int ct = 0; ct < NDK; ++ct) {
      const int c = 16 * ct + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int xl = 4 * g + i, x = t0 + xl;
        const float bx = sB[x * PB + c];
        float sq = 0.f, sk = 0.f;
        for (int ul = 0; ul < 16; ++ul) {
          const int u = t0 + ul;
          // u as the key (u <= x) for dq, as the query (u >= x) for dk: one factor
          // 2^{-|B_x - B_u|} serves both
          const float f = fexp2(-fabsf(bx - sB[u * PB + c]));
          const float tq = myM[xl * PA + ul] * bf(sK[u * PQ + c]) * f;
          const float tk = myM[ul * PA + xl] * bf(sQ[u * PQ + c]) * f;
          sq += ul <= xl ? tq : 0.f;
          sk += ul >= xl ? tk : 0.f;
        }
        dqa[ct][i] += p.q_scale * sq;
        dka[ct][i] += p.q_scale * sk;
      }
    }
    // dv_s[e] += sum_{t >= s} A[t][s] dO_t[e] 2^{C_t - C_s}
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      const int e = 16 * E + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sl = 4 * g + i, s = t0 + sl;
        const float cs = sC[s * PC + e];
        float sum = 0.f;
        for (int ul = i; ul < 16; ++ul) {
          const int u = t0 + ul;
          const float term = myA[ul * PA + sl] * sD[u * PC + e] * fexp2(fminf(sC[u * PC + e] - cs, 0.f));
          sum += ul >= sl ? term : 0.f;
        }
        dva[E][i] += sum;
      }
    }
  }
  // ---- gate gradients: per-row terms, suffix sums over the chunk, boundary sums
  __syncthreads();  // every read of B, C done: their regions take the per-row terms
#pragma unroll
  for (int ct = 0; ct < NDK; ++ct) {
    const int c = 16 * ct + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      sB[t * PB + c] = bf(sQ[t * PQ + c]) * dqa[ct][i] - bf(sK[t * PQ + c]) * dka[ct][i];
    }
  }
#pragma unroll
  for (int E = 0; E < NDV; ++E) {
    const int e = 16 * E + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      sC[t * PC + e] = od[E][i] - bf(sV[t * PV + e]) * dva[E][i];
    }
  }
  __syncthreads();
  {
    const int t = kBC - 1 - lane;  // lanes walk the rows backwards: a prefix is a suffix
    const long rowt = ci.row0 + (long)min(t, ci.valid - 1) * p.H;
    constexpr int NZ = DKP / 4, NW = DVP / 4;
    bf16 zr[NZ], wr[NW];  // the raw logits, loaded together (clamped columns)
#pragma unroll
    for (int k = 0; k < NZ; ++k) zr[k] = p.z[rowt * p.dk + min(wave + 4 * k, p.dk - 1)];
#pragma unroll
    for (int k = 0; k < NW; ++k) wr[k] = p.w[rowt * p.dv + min(wave + 4 * k, p.dv - 1)];
#pragma unroll
    for (int k = 0; k < NZ; ++k) {
      const int c = wave + 4 * k;
      const float x = scan_dpp<64>(sB[t * PB + c]) + sBa[c];
      if (t < ci.valid && c < p.dk)
        p.dz[rowt * p.dk + c] = from_f<bf16>(x * fast_sigmoid(-bf(zr[k])) * p.inv_tau);
    }
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int e = wave + 4 * k;
      const float x = scan_dpp<64>(sC[t * PC + e]) + sBb[e];
      if (t < ci.valid && e < p.dv)
        p.dw[rowt * p.dv + e] = from_f<bf16>(x * fast_sigmoid(-bf(wr[k])) * p.inv_tau);
    }
  }
  // ---- dq, dk, dv
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * g + i;
    if (t >= ci.valid) continue;
#pragma unroll
    for (int ct = 0; ct < NDK; ++ct) {
      const int c = 16 * ct + r;
      if (c < p.dk) {
        const long gi = (ci.row0 + (long)t * p.H) * p.dk + c;
        p.dq[gi] = from_f<bf16>(dqa[ct][i]);
        p.dk_[gi] = from_f<bf16>(dka[ct][i]);
      }
    }
#pragma unroll
    for (int E = 0; E < NDV; ++E) {
      const int e = 16 * E + r;
      if (e < p.dv) p.dv_[(ci.row0 + (long)t * p.H) * p.dv + e] = from_f<bf16>(dva[E][i]);
    }
  }
}

// d_norm_w[e] = sum over chunks of the partials, in a fixed order.
__global__ __launch_bounds__(256) void beta_dgamma_reduce(const float* part, long nparts, int dv,
                                                          float* out) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float x = 0.f;
  for (long i = threadIdx.x; i < nparts; i += 256) x += part[i * dv + e];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[e] = red[0];
}

template <int NDK, int NDV, bool VEC>
hipError_t launch_beta_v(const GlaShape& s, const BetaArgs& a, bool bwd, hipStream_t st) {
  using Lo = BetaLay<NDK, NDV>;
  const unsigned grid = (unsigned)((long)s.B * s.H * s.NC);
  const dim3 sgrid((unsigned)((s.dk * s.dv + 255) / 256), (unsigned)(s.B * s.H));
  if (!bwd) {
    hipLaunchKernelGGL((beta_fwd_state<NDK, NDV, VEC>), dim3(grid), dim3(kBT), Lo::U_END, st, a);
    hipLaunchKernelGGL(beta_scan, sgrid, dim3(256), 0, st, a.states, a.dec, s.NC, s.dk, s.dv, 0);
    hipLaunchKernelGGL((beta_fwd_out<NDK, NDV, VEC>), dim3(grid), dim3(kBT), Lo::F_END, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((beta_bwd_state<NDK, NDV, VEC>), dim3(grid), dim3(kBT), Lo::U_END, st, a);
  hipLaunchKernelGGL(beta_scan, sgrid, dim3(256), 0, st, a.gst, a.dec, s.NC, s.dk, s.dv, 1);
  hipLaunchKernelGGL((beta_bwd_out<NDK, NDV, VEC>), dim3(grid), dim3(kBT), Lo::G_END, st, a);
  return hipGetLastError();
}

// Four-element staging where every staged row is whole 8-byte pieces.
template <int NDK, int NDV>
hipError_t launch_beta(const GlaShape& s, const BetaArgs& a, bool bwd, hipStream_t st) {
  auto al8 = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 7) == 0; };
  const bool vec = s.dk % 4 == 0 && s.dv % 4 == 0 && al8(a.q) && al8(a.k) && al8(a.v) &&
                   al8(a.z) && al8(a.w);
  return vec ? launch_beta_v<NDK, NDV, true>(s, a, bwd, st)
             : launch_beta_v<NDK, NDV, false>(s, a, bwd, st);
}

}  // namespace

int gla_beta_lds_bytes(const GlaShape& s, bool bwd) {
  switch (s.ndk * 16 + s.ndv) {
    case 1 * 16 + 2: return bwd ? BetaLay<1, 2>::G_END : BetaLay<1, 2>::F_END;
    case 2 * 16 + 4: return bwd ? BetaLay<2, 4>::G_END : BetaLay<2, 4>::F_END;
    case 3 * 16 + 5: return bwd ? BetaLay<3, 5>::G_END : BetaLay<3, 5>::F_END;
    default: return 1 << 30;  // no kernel for this class
  }
}

static size_t al256b(size_t x) { return (x + 255) / 256 * 256; }

size_t gla_beta_states_bytes(const GlaShape& s) {
  return (size_t)s.B * s.H * s.NC * s.dk * s.dv * sizeof(float);
}
size_t gla_beta_obuf_bytes(const GlaShape& s) {
  return (size_t)s.B * s.H * s.NC * kBC * s.dv * sizeof(float);
}
size_t gla_beta_saved_bytes(const GlaShape& s) {
  return al256b(gla_beta_states_bytes(s)) + al256b(gla_beta_obuf_bytes(s));
}
size_t gla_beta_dec_bytes(const GlaShape& s) {
  return (size_t)s.B * s.H * s.NC * (s.dk + s.dv) * sizeof(float);
}
size_t gla_beta_fwd_workspace(const GlaShape& s) {
  return al256b(gla_beta_states_bytes(s)) + al256b(gla_beta_dec_bytes(s));
}
size_t gla_beta_bwd_workspace(const GlaShape& s) {
  return al256b(gla_beta_states_bytes(s)) + al256b(gla_beta_dec_bytes(s)) +
         al256b((size_t)s.B * s.H * s.NC * s.dv * sizeof(float));
}

hipError_t launch_gla_beta_fwd(const GlaShape& s, const GlaBetaFwd& f, hipStream_t st) {
  BetaArgs a{};
  a.q = static_cast<const bf16*>(f.q); a.k = static_cast<const bf16*>(f.k);
  a.v = static_cast<const bf16*>(f.v); a.z = static_cast<const bf16*>(f.z);
  a.w = static_cast<const bf16*>(f.w); a.r = static_cast<const bf16*>(f.r);
  a.norm_w = f.norm_w;
  a.y = static_cast<bf16*>(f.y); a.o_pre = static_cast<bf16*>(f.o_pre);
  char* ws = static_cast<char*>(f.workspace);
  if (f.saved) {
    a.states = static_cast<float*>(f.saved);
    a.obuf = reinterpret_cast<float*>(static_cast<char*>(f.saved) +
                                      al256b(gla_beta_states_bytes(s)));
  } else {
    a.states = reinterpret_cast<float*>(ws);
  }
  a.dec = reinterpret_cast<float*>(ws + al256b(gla_beta_states_bytes(s)));
  a.B = s.B; a.L = s.L; a.H = s.H; a.dk = s.dk; a.dv = s.dv; a.NC = s.NC;
  a.inv_tau = f.inv_tau; a.q_scale = f.q_scale; a.eps = f.eps;
  switch (s.ndk * 16 + s.ndv) {
    case 1 * 16 + 2: return launch_beta<1, 2>(s, a, false, st);
    case 2 * 16 + 4: return launch_beta<2, 4>(s, a, false, st);
    case 3 * 16 + 5: return launch_beta<3, 5>(s, a, false, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gla_beta_bwd(const GlaShape& s, const GlaBetaBwd& f, hipStream_t st) {
  BetaArgs a{};
  a.q = static_cast<const bf16*>(f.q); a.k = static_cast<const bf16*>(f.k);
  a.v = static_cast<const bf16*>(f.v); a.z = static_cast<const bf16*>(f.z);
  a.w = static_cast<const bf16*>(f.w); a.r = static_cast<const bf16*>(f.r);
  a.dy = static_cast<const bf16*>(f.dy);
  a.norm_w = f.norm_w;
  a.states = const_cast<float*>(static_cast<const float*>(f.saved));
  a.obuf = reinterpret_cast<float*>(const_cast<char*>(static_cast<const char*>(f.saved)) +
                                    al256b(gla_beta_states_bytes(s)));
  char* ws = static_cast<char*>(f.workspace);
  a.gst = reinterpret_cast<float*>(ws);
  a.dec = reinterpret_cast<float*>(ws + al256b(gla_beta_states_bytes(s)));
  a.dgp = reinterpret_cast<float*>(ws + al256b(gla_beta_states_bytes(s)) +
                                   al256b(gla_beta_dec_bytes(s)));
  a.dq = static_cast<bf16*>(f.dq); a.dk_ = static_cast<bf16*>(f.dk);
  a.dv_ = static_cast<bf16*>(f.dv); a.dz = static_cast<bf16*>(f.dz);
  a.dw = static_cast<bf16*>(f.dw); a.dr = static_cast<bf16*>(f.dr);
  a.B = s.B; a.L = s.L; a.H = s.H; a.dk = s.dk; a.dv = s.dv; a.NC = s.NC;
  a.inv_tau = f.inv_tau; a.q_scale = f.q_scale; a.eps = f.eps;
  hipError_t e;
  switch (s.ndk * 16 + s.ndv) {
    case 1 * 16 + 2: e = launch_beta<1, 2>(s, a, true, st); break;
    case 2 * 16 + 4: e = launch_beta<2, 4>(s, a, true, st); break;
    case 3 * 16 + 5: e = launch_beta<3, 5>(s, a, true, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || !f.d_norm_w) return e;
  hipLaunchKernelGGL(beta_dgamma_reduce, dim3((unsigned)s.dv), dim3(256), 0, st, a.dgp,
                     (long)s.B * s.H * s.NC, s.dv, f.d_norm_w);
  return hipGetLastError();
}

}  // namespace dig
