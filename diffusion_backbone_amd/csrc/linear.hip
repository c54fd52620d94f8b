// linear.hip -- the dense projections of a DiG block on gfx950 bf16 matrix cores:
//   C_o = epilogue_o(A W_o^T + bias_o)   for up to kLinearMaxOut outputs o sharing the input A
// (DiG study-group slides, slide introducing GLA, eqs. (5) and (9)-(10): Q = X W_Q,
// K = X W_K, V = X W_V, the gate logits X W_alpha (here the rank-16 factor X W_a1, then
// (X W_a1) W_a2 + b_alpha), R = X W_r + b_r, and Y = (Swish(R) * Norm(O)) W_O; slides
// Figure 4 and the write-up's section 3 "DiG Block": the feedforward, and the residual adds
// scaled by the regressed alpha_1, alpha_2).  Epilogues: none, GELU, and the gated residual
// C = R + g[row / rows_per_gate] * (A W^T + bias), R possibly C itself.
//
// One launch covers every output: the grid runs over (row tile, column tile of the
// concatenated outputs), and a tile never straddles two outputs.  Each wave owns 64 x 64
// outputs as 2 x 2 MFMA tiles of 32 x 32 (K step 16: on gfx950 the 32x32x16 bf16 instruction
// sustains about 1.7 times the rate of 16x16x32); K blocks of 32 or 64 staged in LDS (A rows
// and W rows, both K-contiguous, pitch 16 bytes past a multiple of 64: conflict-free 16-byte
// reads) with the next block loaded into registers while the current one is multiplied (two
// LDS buffers).  Tiles of 128 x 128 (four waves, two or three workgroups per compute unit) or
// 256 x 256 (sixteen waves, one per unit).  fp32 accumulation; bias and GELU in fp32; bf16
// output stored from LDS in 16-byte row pieces, where the gated residual is applied.  Products
// whose grid would not fill the GPU can split K over a workspace (fp32 partial sums, then a
// reducing launch with the epilogue).
#include "dig_device.h"
#include "dig_internal.h"

namespace dig {
namespace {


struct LinOut {
  bf16* c;
  const bf16* w;
  const float* bias;
  const bf16* res;   // gated residual R (may be c), or null
  const bf16* gate;  // its gate rows g, [M / rows_per_gate][gate_ld]
  long gate_ld;
  int rows_per_gate;
  int act;           // kActNone | kActGelu
  int n;             // columns of this output (rows of W)
  int tile0;         // first column tile of this output in the grid
};

// GELU in its exact form, x Phi(x) = x (1 + erf(x / sqrt 2)) / 2.
__device__ __forceinline__ float gelu_exact(float x) {
  return 0.5f * x * (1.f + erff(x * 0.70710678118654752f));
}
struct LinParams {
  const bf16* a;
  int M, K, nout;
  int ntot;  // packed launches: the outputs' columns side by side (tile0 = first column)
  LinOut out[kLinearMaxOut];
};

// Square tiles of BM x BM outputs, (BM / 64)^2 waves of 64 x 64.
template <int BM>
struct Tile {
  static constexpr int BN = BM, NTHR = (BM / 64) * (BM / 64) * 64, CPITCH = BN + 8;
};

// BM rows x BK bf16 (one K block of a tile) of a K-contiguous source into registers: the
// tile's BM * BK / 8 16-byte pieces, NP per thread (thread t: pieces t + NTHR u, piece q at
// row q / (BK / 8), K piece q % (BK / 8)).  Rows past `rows` and columns past K read as zero.
template <int BM, int BK>
struct BlockRegs {
  static constexpr int NTHR = Tile<BM>::NTHR, PPR = BK / 8, NP = BM * PPR / NTHR;
  static_assert(BM * PPR % NTHR == 0, "pieces per thread");
  uint4 v[NP];
};
template <int BM, int BK>
__device__ __forceinline__ void load_block(BlockRegs<BM, BK>& r, const bf16* src, int rows, int K,
                                           int r0, int k0, int tid) {
  constexpr int PPR = BlockRegs<BM, BK>::PPR, NTHR = Tile<BM>::NTHR;
#pragma unroll
  for (int u = 0; u < BlockRegs<BM, BK>::NP; ++u) {
    const int q = tid + NTHR * u, row = q / PPR, piece = q % PPR;
    const int gr = r0 + row, gk = k0 + piece * 8;
    const bool in = gr < rows && gk < K;
    const uint4 x = *reinterpret_cast<const uint4*>(src + (long)(in ? gr : 0) * K + (in ? gk : 0));
    r.v[u] = in ? x : make_uint4(0, 0, 0, 0);
  }
}
// The same for W rows gathered from several outputs: piece u of this thread reads the row at
// wrow[u] (nullptr: a row past the last output, read as zero; the load then goes to `safe`,
// any readable 16 bytes, so that no load sits under a branch).
template <int BM, int BK>
__device__ __forceinline__ void load_rows(BlockRegs<BM, BK>& r,
                                          const bf16* const (&wrow)[BlockRegs<BM, BK>::NP],
                                          const bf16* safe, int K, int k0, int tid) {
  constexpr int PPR = BlockRegs<BM, BK>::PPR, NTHR = Tile<BM>::NTHR;
#pragma unroll
  for (int u = 0; u < BlockRegs<BM, BK>::NP; ++u) {
    const int q = tid + NTHR * u, piece = q % PPR;
    const int gk = k0 + piece * 8;
    const bool in = wrow[u] != nullptr && gk < K;
    const uint4 x = *reinterpret_cast<const uint4*>(in ? wrow[u] + gk : safe);
    r.v[u] = in ? x : make_uint4(0, 0, 0, 0);
  }
}
template <int BM, int BK>
__device__ __forceinline__ void store_block(const BlockRegs<BM, BK>& r, bf16* lds, int tid) {
  constexpr int PPR = BlockRegs<BM, BK>::PPR, LPITCH = BK + 8, NTHR = Tile<BM>::NTHR;
#pragma unroll
  for (int u = 0; u < BlockRegs<BM, BK>::NP; ++u) {
    const int q = tid + NTHR * u, row = q / PPR, piece = q % PPR;
    *reinterpret_cast<uint4*>(lds + row * LPITCH + piece * 8) = r.v[u];
  }
}

// EPI: which epilogues this instantiation can apply (bit 0: GELU, bit 1: gated residual); the
// choice per output is uniform over a workgroup.  EPI == kPartial: split K -- workgroup z of
// the grid's third dimension multiplies K blocks [z kbs, (z + 1) kbs) and stores its fp32 sums
// to part[z][M][n] (one output), for linear_splitk_reduce to finish.  EPI & kPacked: the
// outputs' columns side by side (p.ntot of them, output o from column p.out[o].tile0), column
// tiles straddling outputs: W rows are gathered per row, bias and stores per column (outputs
// sharing one activation, no residual).
constexpr int kPartial = 4, kPacked = 8;
template <int BM, int BK, int EPI>
__global__ __launch_bounds__(Tile<BM>::NTHR) void linear_kernel(LinParams p, float* part, int kbs) {
  constexpr int BN = Tile<BM>::BN, NTHR = Tile<BM>::NTHR, CPITCH = Tile<BM>::CPITCH;
  constexpr int WPR = BM / 64;    // waves per tile row
  constexpr int LPITCH = BK + 8;  // elements (16-byte aligned rows, conflict-free reads)
  // the epilogue stages the 128 x 128 bf16 tile over the operand buffers
  constexpr int SA = 2 * BM * LPITCH, SB = 2 * BN * LPITCH;
  constexpr int SLDS = SA + SB > 128 * CPITCH ? SA + SB : 128 * CPITCH;
  __shared__ __align__(16) bf16 lds[SLDS];
  auto sA = [&](int b) { return lds + b * (BM * LPITCH); };
  auto sB = [&](int b) { return lds + SA + b * (BN * LPITCH); };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm = wave / WPR, wn = wave % WPR;  // waves of 64 x 64
  constexpr bool PK = (EPI & kPacked) != 0;
  // which output this column tile belongs to (uniform; packed: output 0 for K and the shared
  // activation, the columns mapped one by one below)
  const int nt = blockIdx.x;
  int o = 0;
  if constexpr (!PK) {
#pragma unroll
    for (int i = 1; i < kLinearMaxOut; ++i)
      if (i < p.nout && nt >= p.out[i].tile0) o = i;
  }
  const LinOut out = p.out[o];
  const int m0 = blockIdx.y * BM, n0 = PK ? nt * BN : (nt - out.tile0) * BN;
  auto owner = [&](int col) {  // packed: the output holding global column col
    int oo = 0;
#pragma unroll
    for (int i = 1; i < kLinearMaxOut; ++i)
      if (i < p.nout && col >= p.out[i].tile0) oo = i;
    return oo;
  };
  const int K = p.K;
  const int nkb_all = (K + BK - 1) / BK;
  const int kb0 = EPI == kPartial ? (int)blockIdx.z * kbs : 0;
  const int nkb = EPI == kPartial ? min(kbs, nkb_all - kb0) : nkb_all;  // >= 1 by the launch

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  BlockRegs<BM, BK> ra, rb;  // the next K block of the A tile and of the W tile
  // packed: this thread's W rows (fixed over K)
  const bf16* wrow[BlockRegs<BM, BK>::NP];
  if constexpr (PK) {
#pragma unroll
    for (int u = 0; u < BlockRegs<BM, BK>::NP; ++u) {
      const int gcol = n0 + (tid + NTHR * u) / BlockRegs<BM, BK>::PPR;
      const int oo = owner(gcol);
      wrow[u] = gcol < p.ntot ? p.out[oo].w + (long)(gcol - p.out[oo].tile0) * K : nullptr;
    }
  }
  auto load = [&](int kb) {
    load_block(ra, p.a, p.M, K, m0, (kb0 + kb) * BK, tid);
    if constexpr (PK) load_rows(rb, wrow, p.out[0].w, K, (kb0 + kb) * BK, tid);
    else load_block(rb, out.w, out.n, K, n0, (kb0 + kb) * BK, tid);
  };
  auto put = [&](int buf) {
    store_block(ra, sA(buf), tid);
    store_block(rb, sB(buf), tid);
  };
  // 32x32x16 operands: lane l holds row (l % 32) of its 32-row tile, K slice 8 (l / 32)..+7
  const int r32 = lane & 31, h32 = lane >> 5;
  load(0);
  put(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load(kb + 1);  // in flight while this block is multiplied
    const bf16* A = sA(buf) + (wm * 64 + r32) * LPITCH + 8 * h32;
    const bf16* B = sB(buf) + (wn * 64 + r32) * LPITCH + 8 * h32;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(A + 32 * i * LPITCH + 16 * ks);
        bfr[i] = *reinterpret_cast<const bf16x8*>(B + 32 * i * LPITCH + 16 * ks);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32_bf16(af[i], bfr[j], acc[i][j]);
    }
    if (kb + 1 < nkb) {
      put(buf ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
    }
  }
  if constexpr (EPI == kPartial) {  // fp32 sums straight from the accumulators (32 lanes store
                                    // 128 consecutive bytes of one row)
    float* dst = part + (long)blockIdx.z * p.M * out.n;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + 32 * j + r32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * 64 + 32 * i + 8 * (v >> 2) + 4 * h32 + (v & 3);
          if (row < p.M && col < out.n) dst[(long)row * out.n + col] = acc[i][j][v];
        }
      }
    return;
  }
  __syncthreads();  // every wave is done with the operand tiles: reuse them for the output

  // epilogue, in BM / 128 parts of 128 rows (the staging tile fits the operand buffers):
  // acc[i][j][v] = C[m0 + wm*64 + 32i + 8(v/4) + 4(l/32) + v%4][n0 + wn*64 + 32j + l%32]
  bf16* sC = lds;  // [BM / 2][CPITCH] bf16
#pragma unroll
  for (int half = 0; half < BM / 128; ++half) {
    if (half) __syncthreads();  // the previous part's rows have been read
    if ((wm >> 1) == half) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + 32 * j + r32;
        float bias;
        if constexpr (PK) {
          const int gcol = n0 + col, oo = owner(gcol);
          const float* bp = p.out[oo].bias;
          bias = (bp && gcol < p.ntot) ? bp[gcol - p.out[oo].tile0] : 0.f;
        } else {
          bias = (out.bias && n0 + col < out.n) ? out.bias[n0 + col] : 0.f;
        }
        const bool gelu = (EPI & 1) && out.act == kActGelu;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float t = acc[i][j][v] + bias;
            if constexpr (EPI & 1) t = gelu ? gelu_exact(t) : t;
            sC[((wm & 1) * 64 + 32 * i + 8 * (v >> 2) + 4 * h32 + (v & 3)) * CPITCH + col] =
                from_f<bf16>(t);
          }
      }
    }
    __syncthreads();
    // 128 rows of BN columns = 128 * BN / 8 pieces of 8 bf16 over the threads
    constexpr int PPRC = BN / 8, NPC = 128 * PPRC / NTHR;
#pragma unroll
    for (int u = 0; u < NPC; ++u) {
      const int piece = tid + NTHR * u;
      const int row = piece / PPRC, cp = (piece % PPRC) * 8;
      const int gr = m0 + 128 * half + row, gc = n0 + cp;
      if constexpr (PK) {  // every output's width is a multiple of 8: pieces never straddle
        if (gr >= p.M || gc >= p.ntot) continue;
        const int oo = owner(gc);
        *reinterpret_cast<bf16x8*>(p.out[oo].c + (long)gr * p.out[oo].n + (gc - p.out[oo].tile0)) =
            *reinterpret_cast<const bf16x8*>(sC + row * CPITCH + cp);
        continue;
      }
      if (gr >= p.M || gc >= out.n) continue;  // n is a multiple of 8: whole pieces only
      bf16x8 val = *reinterpret_cast<const bf16x8*>(sC + row * CPITCH + cp);
      if ((EPI & 2) && out.res) {  // C = R + g * val, each element read and written here only
        const bf16x8 rv = *reinterpret_cast<const bf16x8*>(out.res + (long)gr * out.n + gc);
        const bf16x8 gv = *reinterpret_cast<const bf16x8*>(
            out.gate + (long)(gr / out.rows_per_gate) * out.gate_ld + gc);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          val[e] = from_f<bf16>(fmaf(to_f(gv[e]), to_f(val[e]), to_f(rv[e])));
      }
      *reinterpret_cast<bf16x8*>(out.c + (long)gr * out.n + gc) = val;
    }
  }
}

// Finishes a split-K product: sums the S fp32 partial tiles in a fixed order, adds the bias,
// applies the output's epilogue and stores bf16, eight elements per thread.
template <int EPI>
__global__ __launch_bounds__(256) void linear_splitk_reduce(LinOut out, const float* part, int M,
                                                            int S) {
  const long npc = (long)M * out.n / 8;
  for (long q = (long)blockIdx.x * 256 + threadIdx.x; q < npc; q += (long)gridDim.x * 256) {
    const long e0 = q * 8;
    const int gr = (int)(e0 / out.n), gc = (int)(e0 - (long)gr * out.n);
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = out.bias ? out.bias[gc + e] : 0.f;
    for (int z = 0; z < S; ++z) {
      const float4* src = reinterpret_cast<const float4*>(part + (long)z * M * out.n + e0);
      const float4 a = src[0], b = src[1];
      t[0] += a.x; t[1] += a.y; t[2] += a.z; t[3] += a.w;
      t[4] += b.x; t[5] += b.y; t[6] += b.z; t[7] += b.w;
    }
    bf16x8 val;
    const bool gelu = (EPI & 1) && out.act == kActGelu;
#pragma unroll
    for (int e = 0; e < 8; ++e) val[e] = from_f<bf16>(gelu ? gelu_exact(t[e]) : t[e]);
    if ((EPI & 2) && out.res) {
      const bf16x8 rv = *reinterpret_cast<const bf16x8*>(out.res + e0);
      const bf16x8 gv = *reinterpret_cast<const bf16x8*>(
          out.gate + (long)(gr / out.rows_per_gate) * out.gate_ld + gc);
#pragma unroll
      for (int e = 0; e < 8; ++e) val[e] = from_f<bf16>(fmaf(to_f(gv[e]), to_f(val[e]), to_f(rv[e])));
    }
    *reinterpret_cast<bf16x8*>(out.c + e0) = val;
  }
}

// Launch with BM x BM tiles (tile0 of each output counted in BM-wide column tiles).
template <int BM, int BK = 32>
static hipError_t launch_linear_bm(int M, int K, const void* a, int nout, const LinearOut* outs,
                                   hipStream_t st) {
  LinParams p{};
  p.a = static_cast<const bf16*>(a);
  p.M = M;
  p.K = K;
  p.nout = nout;
  int tiles = 0;
  for (int i = 0; i < nout; ++i) {
    p.out[i].c = static_cast<bf16*>(outs[i].c);
    p.out[i].w = static_cast<const bf16*>(outs[i].w);
    p.out[i].bias = outs[i].bias;
    p.out[i].res = static_cast<const bf16*>(outs[i].res);
    p.out[i].gate = static_cast<const bf16*>(outs[i].gate);
    p.out[i].gate_ld = outs[i].gate_ld;
    p.out[i].rows_per_gate = outs[i].rows_per_gate;
    p.out[i].act = outs[i].act;
    p.out[i].n = outs[i].n;
    p.out[i].tile0 = tiles;
    tiles += (outs[i].n + BM - 1) / BM;
  }
  const long mt = ((long)M + BM - 1) / BM;
  if (mt > 65535) return hipErrorInvalidValue;
  int epi = 0;
  for (int i = 0; i < nout; ++i) epi |= (outs[i].act == kActGelu ? 1 : 0) | (outs[i].res ? 2 : 0);
  // several outputs sharing one activation and no residual: pack their columns (no tile
  // padded out per output) when K is long enough for the per-column gathers to pay (at
  // K = 384 the per-output tiles measured faster)
  bool pack = nout > 1 && !(epi & 2) && K >= 1024;
  for (int i = 1; i < nout; ++i) pack = pack && outs[i].act == outs[0].act;
  if (pack) {
    int col = 0;
    for (int i = 0; i < nout; ++i) {
      p.out[i].tile0 = col;
      col += outs[i].n;
    }
    p.ntot = col;
    if ((col + BM - 1) / BM < tiles) {
      const dim3 grid((unsigned)((col + BM - 1) / BM), (unsigned)mt), block(Tile<BM>::NTHR);
      if (epi & 1) hipLaunchKernelGGL((linear_kernel<BM, BK, kPacked | 1>), grid, block, 0, st, p, nullptr, 0);
      else hipLaunchKernelGGL((linear_kernel<BM, BK, kPacked>), grid, block, 0, st, p, nullptr, 0);
      return hipGetLastError();
    }
    for (int i = 0, t = 0; i < nout; ++i) {  // no column saved: per-output tiles after all
      p.out[i].tile0 = t;
      t += (outs[i].n + BM - 1) / BM;
    }
  }
  const dim3 grid((unsigned)tiles, (unsigned)mt), block(Tile<BM>::NTHR);
  switch (epi) {
    case 0: hipLaunchKernelGGL((linear_kernel<BM, BK, 0>), grid, block, 0, st, p, nullptr, 0); break;
    case 1: hipLaunchKernelGGL((linear_kernel<BM, BK, 1>), grid, block, 0, st, p, nullptr, 0); break;
    case 2: hipLaunchKernelGGL((linear_kernel<BM, BK, 2>), grid, block, 0, st, p, nullptr, 0); break;
    default: hipLaunchKernelGGL((linear_kernel<BM, BK, 3>), grid, block, 0, st, p, nullptr, 0); break;
  }
  return hipGetLastError();
}

// Split-K plan of a one-output product on 128 x 128 tiles: the number of K splits that brings
// the grid to about 384 workgroups (1.5 rounds of the 256 compute units at three per unit),
// with at least eight K blocks of 32 per split (shorter splits lose more to the second launch
// and the partial sums' traffic than they gain); 1 = no split.
static int splitk_count(int M, int K, int n) {
  const long tiles = ((long)M + 127) / 128 * ((n + 127) / 128);
  if (tiles >= 192) return 1;
  int s = (int)((384 + tiles - 1) / tiles);
  const int kbmax = ((K + 31) / 32) / 8;
  if (s > kbmax) s = kbmax;
  if (s > 8) s = 8;
  return s < 2 ? 1 : s;
}

static hipError_t launch_linear_splitk(int M, int K, const void* a, const LinearOut& o, int S,
                                       float* part, hipStream_t st) {
  LinParams p{};
  p.a = static_cast<const bf16*>(a);
  p.M = M;
  p.K = K;
  p.nout = 1;
  LinOut& lo = p.out[0];
  lo.c = static_cast<bf16*>(o.c);
  lo.w = static_cast<const bf16*>(o.w);
  lo.bias = o.bias;
  lo.res = static_cast<const bf16*>(o.res);
  lo.gate = static_cast<const bf16*>(o.gate);
  lo.gate_ld = o.gate_ld;
  lo.rows_per_gate = o.rows_per_gate;
  lo.act = o.act;
  lo.n = o.n;
  lo.tile0 = 0;
  const int nkb = (K + 31) / 32, kbs = (nkb + S - 1) / S;
  S = (nkb + kbs - 1) / kbs;  // every split holds at least one K block
  const dim3 grid((unsigned)((o.n + 127) / 128), (unsigned)((M + 127) / 128), (unsigned)S);
  hipLaunchKernelGGL((linear_kernel<128, 32, kPartial>), grid, dim3(Tile<128>::NTHR), 0, st, p,
                     part, kbs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long npc = (long)M * o.n / 8;
  long g = (npc + 255) / 256;
  if (g > 2048) g = 2048;
  const int epi = (o.act == kActGelu ? 1 : 0) | (o.res ? 2 : 0);
  switch (epi) {
    case 0: hipLaunchKernelGGL(linear_splitk_reduce<0>, dim3((unsigned)g), dim3(256), 0, st, lo, part, M, S); break;
    case 1: hipLaunchKernelGGL(linear_splitk_reduce<1>, dim3((unsigned)g), dim3(256), 0, st, lo, part, M, S); break;
    case 2: hipLaunchKernelGGL(linear_splitk_reduce<2>, dim3((unsigned)g), dim3(256), 0, st, lo, part, M, S); break;
    default: hipLaunchKernelGGL(linear_splitk_reduce<3>, dim3((unsigned)g), dim3(256), 0, st, lo, part, M, S); break;
  }
  return hipGetLastError();
}

}  // namespace

// 256 x 256 tiles (sixteen waves, one workgroup per compute unit, twice the flops per byte
// loaded) when they give at least four rounds of workgroups over the 256 compute units; else
// 128 x 128 tiles (four waves, three workgroups per unit), which fill smaller problems.
size_t linear_splitk_bytes(int M, int K, int n) {
  const int s = splitk_count(M, K, n);
  return s > 1 ? (size_t)s * M * n * sizeof(float) : 0;
}

hipError_t launch_linear(int M, int K, const void* a, int nout, const LinearOut* outs,
                         hipStream_t st, void* ws, size_t ws_bytes) {
  if (nout < 1 || nout > kLinearMaxOut) return hipErrorInvalidValue;
  if (nout == 1 && ws) {  // small grids: split K into partial sums in the workspace
    const int s = splitk_count(M, K, outs[0].n);
    if (s > 1 && ws_bytes >= (size_t)s * M * outs[0].n * sizeof(float))
      return launch_linear_splitk(M, K, a, outs[0], s, static_cast<float*>(ws), st);
  }
  long t256 = 0;
  for (int i = 0; i < nout; ++i) t256 += (outs[i].n + 255) / 256;
  t256 *= ((long)M + 255) / 256;
  // K stages of 64 (half the barriers and load round trips per flop) pay off once K is long
  // and the grid holds at least three rounds of 128 x 128 tiles; smaller problems keep 32
  long t128 = 0;
  for (int i = 0; i < nout; ++i) t128 += (outs[i].n + 127) / 128;
  t128 *= ((long)M + 127) / 128;
  const bool k64 = K >= 1024 && t128 >= 3 * 256;
  if (t256 >= 4 * 256)
    return k64 ? launch_linear_bm<256, 64>(M, K, a, nout, outs, st)
               : launch_linear_bm<256>(M, K, a, nout, outs, st);
  return k64 ? launch_linear_bm<128, 64>(M, K, a, nout, outs, st)
             : launch_linear_bm<128>(M, K, a, nout, outs, st);
}

}  // namespace dig
