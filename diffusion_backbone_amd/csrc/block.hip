// block.hip -- the elementwise steps of a DiG block around its GLA layer and feedforward on
// gfx950 (DiG study-group slides, Figure 4; DiG write-up, section 3 "DiG Block"): the
// RMSNorm whose output is scaled and shifted by the parameters regressed from the
// conditioning (adaptive normalisation), and the SiLU applied to the conditioning vector
// before that regression.
//
// Both are bound by HBM: one read of each input row, one write of each output row.  One wave
// per token row; a lane holds up to four 16-byte pieces of the row (D <= 2048 bf16), all loads
// issued before any arithmetic.
#include "dig_device.h"
#include "dig_internal.h"

namespace dig {
namespace {

constexpr int kMaxPieces = 4;  // 16-byte pieces per lane: D <= 64 * 8 * 4

__device__ __forceinline__ float wave_sum_dpp(float x) {
  x = row_sum16(x);
  return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}

// Rows are D contiguous bf16; the image of row r is r / rows_per_group; its scale and shift
// rows are D contiguous bf16 at mod_ld element strides.
template <int NP>
__global__ __launch_bounds__(256) void rmsnorm_modulate_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ scale, const bf16* __restrict__ shift,
    long mod_ld, long rows, int D, long rows_per_group, float eps, bf16* __restrict__ h) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int npieces = D / 8;
  const bf16* xr = x + row * D;
  bf16x8 xv[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int pc = lane + 64 * u;
    const int pcl = pc < npieces ? pc : 0;  // clamped: every load stays inside the row
    xv[u] = *reinterpret_cast<const bf16x8*>(xr + 8 * pcl);
  }
  const long g = row / rows_per_group;
  const bf16* sc = scale + g * mod_ld;
  const bf16* sh = shift + g * mod_ld;
  bf16x8 sv[NP], tv[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int pc = lane + 64 * u;
    const int pcl = pc < npieces ? pc : 0;
    sv[u] = *reinterpret_cast<const bf16x8*>(sc + 8 * pcl);
    tv[u] = *reinterpret_cast<const bf16x8*>(sh + 8 * pcl);
  }
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    if (lane + 64 * u < npieces) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = to_f(xv[u][e]);
        ss = fmaf(f, f, ss);
      }
    }
  }
  const float rstd = rsqrtf(wave_sum_dpp(ss) / (float)D + eps);
  bf16* hr = h + row * D;
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int pc = lane + 64 * u;
    if (pc < npieces) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = from_f<bf16>(fmaf(to_f(xv[u][e]) * rstd, to_f(sv[u][e]), to_f(tv[u][e])));
      *reinterpret_cast<bf16x8*>(hr + 8 * pc) = o;
    }
  }
}

__global__ __launch_bounds__(256) void silu_kernel(const bf16* __restrict__ x, long n,
                                                   bf16* __restrict__ y) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const float f = to_f(x[i]);
    y[i] = from_f<bf16>(f / (1.f + expf(-f)));
  }
}

}  // namespace

hipError_t launch_rmsnorm_modulate(long rows, int D, long rows_per_group, float eps,
                                   const void* x, const void* scale, const void* shift,
                                   long mod_ld, void* h, hipStream_t st) {
  if (D % 8 || D < 8 || D > 64 * 8 * kMaxPieces || rows_per_group < 1)
    return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  const long blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  const int np = (D / 8 + 63) / 64;
  auto* xp = static_cast<const bf16*>(x);
  auto* sp = static_cast<const bf16*>(scale);
  auto* tp = static_cast<const bf16*>(shift);
  auto* hp = static_cast<bf16*>(h);
  const dim3 grid((unsigned)blocks), block(256);
  switch (np) {
    case 1: hipLaunchKernelGGL(rmsnorm_modulate_kernel<1>, grid, block, 0, st, xp, sp, tp, mod_ld, rows, D, rows_per_group, eps, hp); break;
    case 2: hipLaunchKernelGGL(rmsnorm_modulate_kernel<2>, grid, block, 0, st, xp, sp, tp, mod_ld, rows, D, rows_per_group, eps, hp); break;
    case 3: hipLaunchKernelGGL(rmsnorm_modulate_kernel<3>, grid, block, 0, st, xp, sp, tp, mod_ld, rows, D, rows_per_group, eps, hp); break;
    default: hipLaunchKernelGGL(rmsnorm_modulate_kernel<4>, grid, block, 0, st, xp, sp, tp, mod_ld, rows, D, rows_per_group, eps, hp); break;
  }
  return hipGetLastError();
}

hipError_t launch_silu(long n, const void* x, void* y, hipStream_t st) {
  if (n == 0) return hipSuccess;
  long g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(silu_kernel, dim3((unsigned)g), dim3(256), 0, st,
                     static_cast<const bf16*>(x), n, static_cast<bf16*>(y));
  return hipGetLastError();
}

}  // namespace dig
