// linear.hip -- the projections around the GLA token mixer on gfx950 bf16 matrix cores:
//   C_o = A W_o^T (+ bias_o)   for up to kLinearMaxOut outputs o sharing the input A
// (DiG study-group slides, slide introducing GLA, eqs. (5) and (9)-(10): Q = X W_Q,
// K = X W_K, V = X W_V, the gate logits X W_alpha (here the rank-16 factor X W_a1, then
// (X W_a1) W_a2 + b_alpha), R = X W_r + b_r, and Y = (Swish(R) * Norm(O)) W_O).
//
// One launch covers every output: the grid runs over (row tile, column tile of the
// concatenated outputs), and a tile never straddles two outputs.  Tiles of 128 x 128 outputs,
// four waves of 64 x 64 (4 x 4 MFMA tiles of 16 x 16, K step 32), K blocks of 64 staged in
// LDS (A rows and W rows, both K-contiguous, 144-byte pitch) with the next block loaded into
// registers while the current one is multiplied (two LDS buffers).  fp32 accumulation; bias
// added in fp32; bf16 output stored from LDS in 16-byte row pieces.
#include "dig_device.h"
#include "dig_internal.h"

namespace dig {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, LPITCH = BK + 8;  // elements
constexpr int NTHR = 256;
constexpr int CPITCH = BN + 8;                                 // epilogue staging pitch

struct LinOut {
  bf16* c;
  const bf16* w;
  const float* bias;
  int n;       // columns of this output (rows of W)
  int tile0;   // first column tile of this output in the grid
};
struct LinParams {
  const bf16* a;
  int M, K, nout;
  LinOut out[kLinearMaxOut];
};

// 128 rows x 64 bf16 (one K block of a tile) of a K-contiguous source into registers: thread
// t takes rows t / 4 and t / 4 + 64, 16-byte pieces (t % 4) * 2 and (t % 4) * 2 + 1 of each.
// Rows past `rows` and columns past K read as zero.
struct BlockRegs {
  uint4 v[4];
};
__device__ __forceinline__ void load_block(BlockRegs& r, const bf16* src, int rows, int K, int r0,
                                           int k0, int tid) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = (tid >> 2) + 64 * (u >> 1), piece = (tid & 3) * 2 + (u & 1);
    const int gr = r0 + row, gk = k0 + piece * 8;
    const bool in = gr < rows && gk < K;
    const uint4 x = *reinterpret_cast<const uint4*>(src + (long)(in ? gr : 0) * K + (in ? gk : 0));
    r.v[u] = in ? x : make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ void store_block(const BlockRegs& r, bf16* lds, int tid) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = (tid >> 2) + 64 * (u >> 1), piece = (tid & 3) * 2 + (u & 1);
    *reinterpret_cast<uint4*>(lds + row * LPITCH + piece * 8) = r.v[u];
  }
}

__global__ __launch_bounds__(NTHR) void linear_kernel(LinParams p) {
  __shared__ __align__(16) bf16 sA[2][BM * LPITCH];
  __shared__ __align__(16) bf16 sB[2][BN * LPITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  // which output this column tile belongs to (uniform)
  const int nt = blockIdx.x;
  int o = 0;
#pragma unroll
  for (int i = 1; i < kLinearMaxOut; ++i)
    if (i < p.nout && nt >= p.out[i].tile0) o = i;
  const LinOut out = p.out[o];
  const int m0 = blockIdx.y * BM, n0 = (nt - out.tile0) * BN;
  const int K = p.K;
  const int nkb = (K + BK - 1) / BK;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

  BlockRegs ra, rb;  // the next K block of the A tile and of the W tile
  auto load = [&](int kb) {
    load_block(ra, p.a, p.M, K, m0, kb * BK, tid);
    load_block(rb, out.w, out.n, K, n0, kb * BK, tid);
  };
  auto put = [&](int buf) {
    store_block(ra, sA[buf], tid);
    store_block(rb, sB[buf], tid);
  };
  load(0);
  put(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < nkb) load(kb + 1);  // in flight while this block is multiplied
    const bf16* A = sA[buf] + (wm * 64 + r16) * LPITCH + 8 * g4;
    const bf16* B = sB[buf] + (wn * 64 + r16) * LPITCH + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(A + 16 * i * LPITCH + 32 * ks);
        bfr[i] = *reinterpret_cast<const bf16x8*>(B + 16 * i * LPITCH + 32 * ks);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(af[i], bfr[j], acc[i][j]);
    }
    if (kb + 1 < nkb) {
      put(buf ^ 1);  // the other buffer was last read before the previous barrier
      __syncthreads();
    }
  }
  __syncthreads();  // every wave is done with the operand tiles: reuse them for the output

  // epilogue: acc[i][j][v] = C[m0 + wm*64 + 16i + 4g4 + v][n0 + wn*64 + 16j + r16]
  bf16* sC = sA[0];  // [BM][CPITCH] bf16 (34 816 bytes, within sA)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = wn * 64 + 16 * j + r16;
    const float bias = (out.bias && n0 + col < out.n) ? out.bias[n0 + col] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        sC[(wm * 64 + 16 * i + 4 * g4 + v) * CPITCH + col] = from_f<bf16>(acc[i][j][v] + bias);
  }
  __syncthreads();
  // rows of 128 columns = 16 pieces of 8 bf16; 2048 pieces over 256 threads
  const bool full_n = n0 + BN <= out.n && out.n % 8 == 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int piece = tid + NTHR * u;
    const int row = piece >> 4, cp = (piece & 15) * 8;
    const int gr = m0 + row, gc = n0 + cp;
    if (gr >= p.M) continue;
    const uint4 x = *reinterpret_cast<const uint4*>(sC + row * CPITCH + cp);
    bf16* dst = out.c + (long)gr * out.n + gc;
    if (full_n || gc + 8 <= out.n) {
      *reinterpret_cast<uint4*>(dst) = x;
    } else if (gc < out.n) {
      const bf16* e = reinterpret_cast<const bf16*>(&x);
      for (int q = 0; q < out.n - gc; ++q) dst[q] = e[q];
    }
  }
}

}  // namespace

hipError_t launch_linear(int M, int K, const void* a, int nout, const LinearOut* outs,
                         hipStream_t st) {
  if (nout < 1 || nout > kLinearMaxOut) return hipErrorInvalidValue;
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
    p.out[i].n = outs[i].n;
    p.out[i].tile0 = tiles;
    tiles += (outs[i].n + BN - 1) / BN;
  }
  const long mt = ((long)M + BM - 1) / BM;
  if (mt > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(linear_kernel, dim3((unsigned)tiles, (unsigned)mt), dim3(NTHR), 0, st, p);
  return hipGetLastError();
}

}  // namespace dig
