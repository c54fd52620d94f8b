// srem.hip -- DiG's Spatial Reorient & Enhancement Module on gfx950: scan-direction
// reorient (exact row gather) and the 3x3 depthwise conv on the current-order token grid,
// optionally writing its output directly in the next block's scan order.
//
// Pages: DiG study-group slides, slide "SREM の導入"; DiG write-up, section 3 "DiG Block":
// the sequence is reshaped to 2-D, a lightweight 3x3 depthwise conv adds local perception,
// and the token matrix is transposed / the flattened sequence flipped to change the scan
// direction of the next block.
//
// Tensors are [B, L, D] with D channels contiguous per token, so one token row is one
// contiguous run: every access below is a vector load/store of a channel group, with
// consecutive threads on consecutive channel groups of the same token (coalesced).
#include "dig_device.h"
#include "dig_internal.h"

namespace dig {

enum { kRow = 0, kRowRev = 1, kCol = 2, kColRev = 3 };

// pi_d(p): canonical id (i*gw + j) of the token at position p of scan order d.
__device__ __forceinline__ long scan_pi(int d, long p, int gh, int gw, long L) {
  switch (d) {
    case kRow: return p;
    case kRowRev: return L - 1 - p;
    case kCol: return (p % gh) * gw + p / gh;
    default: { const long s = L - 1 - p; return (s % gh) * gw + s / gh; }
  }
}
// inverse of pi_d: position in scan order d of canonical id c.
__device__ __forceinline__ long scan_inv(int d, long c, int gh, int gw, long L) {
  switch (d) {
    case kRow: return c;
    case kRowRev: return L - 1 - c;
    case kCol: return (c % gw) * gh + c / gw;
    default: return L - 1 - ((c % gw) * gh + c / gw);
  }
}

template <typename T, int VW>
struct __attribute__((aligned(VW * sizeof(T)))) Vec {
  T v[VW];
};

// ------------------------------------------------------------------ reorient
template <typename V>
__global__ __launch_bounds__(256) void reorient_kernel(const V* __restrict__ x, V* __restrict__ y,
                                                       long rows, long L, int nv, int gh, int gw,
                                                       int from, int to) {
  const long total = rows * nv;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    const long row = i / nv;
    const int v = (int)(i - row * nv);
    const long b = row / L, p = row - b * L;
    const long src = scan_inv(from, scan_pi(to, p, gh, gw, L), gh, gw, L);
    y[i] = x[(b * L + src) * nv + v];
  }
}

hipError_t launch_reorient(int B, int gh, int gw, int D, int elt, int from, int to,
                           const void* x, void* y, hipStream_t st) {
  const long L = (long)gh * gw, rows = (long)B * L;
  const long rowbytes = (long)D * elt;
  const long total_bytes = rows * rowbytes;
  long blocks_cap = 256L * 16;
  auto grid = [&](long items) {
    long g = (items + 255) / 256;
    return (unsigned)(g < blocks_cap ? g : blocks_cap);
  };
  if (rowbytes % 16 == 0) {
    const int nv = (int)(rowbytes / 16);
    hipLaunchKernelGGL(reorient_kernel<uint4>, dim3(grid(total_bytes / 16)), dim3(256), 0, st,
                       static_cast<const uint4*>(x), static_cast<uint4*>(y), rows, L, nv, gh, gw,
                       from, to);
  } else if (rowbytes % 8 == 0) {
    const int nv = (int)(rowbytes / 8);
    hipLaunchKernelGGL(reorient_kernel<uint2>, dim3(grid(total_bytes / 8)), dim3(256), 0, st,
                       static_cast<const uint2*>(x), static_cast<uint2*>(y), rows, L, nv, gh, gw,
                       from, to);
  } else if (rowbytes % 4 == 0) {
    const int nv = (int)(rowbytes / 4);
    hipLaunchKernelGGL(reorient_kernel<uint32_t>, dim3(grid(total_bytes / 4)), dim3(256), 0, st,
                       static_cast<const uint32_t*>(x), static_cast<uint32_t*>(y), rows, L, nv,
                       gh, gw, from, to);
  } else {
    const int nv = (int)(rowbytes / 2);
    hipLaunchKernelGGL(reorient_kernel<uint16_t>, dim3(grid(total_bytes / 2)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), rows, L, nv,
                       gh, gw, from, to);
  }
  return hipGetLastError();
}

// -------------------------------------------------------------- depthwise conv
// One thread owns VW channels of one current-grid column j and walks a strip of rows,
// keeping a 3x3 window of input vectors in registers (3 new loads per output).
//   forward:  input row of grid position p is p; output row is the position of p's token in
//             scan order out_layout; taps w[c][a+1][s+1] at offset (a, s).
//   backward (dx): input is dy gathered back to the current order (row of p is the position
//             of p's token in out_layout); output row is p; taps rotated by 180 degrees.
template <typename T, int VW, bool BWD>
__global__ __launch_bounds__(256) void dwconv_kernel(const T* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ bias,
                                                     T* __restrict__ y, int gh, int gw, int D,
                                                     int layout, int out_layout, int rows,
                                                     int cols, int SR, int ncolb, int nstrip,
                                                     int nchb) {
  const int cg = threadIdx.x, jj = threadIdx.y;
  int blk = blockIdx.x;
  const int chb = blk % nchb; blk /= nchb;
  const int cb = blk % ncolb; blk /= ncolb;
  const int strip = blk % nstrip;
  const int b = blk / nstrip;
  const int j = cb * blockDim.y + jj;
  const int c0 = (chb * blockDim.x + cg) * VW;
  if (j >= cols || c0 >= D) return;
  const long L = (long)gh * gw;

  float wr[3][3][VW];
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int v = 0; v < VW; ++v)
        wr[a][s][v] = BWD ? w[(c0 + v) * 9 + (2 - a) * 3 + (2 - s)] : w[(c0 + v) * 9 + a * 3 + s];
  float bs[VW];
#pragma unroll
  for (int v = 0; v < VW; ++v) bs[v] = (!BWD && bias) ? bias[c0 + v] : 0.f;

  auto load = [&](int ii, int jc, float* out) {
    if (ii < 0 || ii >= rows || jc < 0 || jc >= cols) {
#pragma unroll
      for (int v = 0; v < VW; ++v) out[v] = 0.f;
      return;
    }
    const long p = (long)ii * cols + jc;
    const long row = BWD ? scan_inv(out_layout, scan_pi(layout, p, gh, gw, L), gh, gw, L) : p;
    const Vec<T, VW> vv = *reinterpret_cast<const Vec<T, VW>*>(x + ((long)b * L + row) * D + c0);
#pragma unroll
    for (int v = 0; v < VW; ++v) out[v] = to_f(vv.v[v]);
  };

  const int i0 = strip * SR, i1 = min(rows, i0 + SR);
  float win[3][3][VW];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    load(i0 - 1, j + s - 1, win[0][s]);
    load(i0, j + s - 1, win[1][s]);
  }
  for (int i = i0; i < i1; ++i) {
#pragma unroll
    for (int s = 0; s < 3; ++s) load(i + 1, j + s - 1, win[2][s]);
    Vec<T, VW> o;
#pragma unroll
    for (int v = 0; v < VW; ++v) {
      float acc = bs[v];
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int s = 0; s < 3; ++s) acc = fmaf(wr[a][s][v], win[a][s][v], acc);
      o.v[v] = from_f<T>(acc);
    }
    const long p = (long)i * cols + j;
    const long orow = BWD ? p : scan_inv(out_layout, scan_pi(layout, p, gh, gw, L), gh, gw, L);
    *reinterpret_cast<Vec<T, VW>*>(y + ((long)b * L + orow) * D + c0) = o;
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int v = 0; v < VW; ++v) {
        win[0][s][v] = win[1][s][v];
        win[1][s][v] = win[2][s][v];
      }
  }
}

// Weight/bias gradient partials: per block, sum over its grid positions of
// dy_conv[i][j] * x[i+a][j+s] (taps 0..8) and dy_conv (tap 9, the bias), reduced over the
// block's columns in a fixed order; part[blk][tap][D].
template <typename T, int VW>
__global__ __launch_bounds__(256) void dwconv_dw_kernel(const T* __restrict__ x,
                                                        const T* __restrict__ dy,
                                                        float* __restrict__ part, int gh, int gw,
                                                        int D, int layout, int out_layout,
                                                        int rows, int cols, int SR, int ncolb,
                                                        int nstrip, int nchb) {
  extern __shared__ float red[];  // [blockDim.y][blockDim.x * VW]
  const int cg = threadIdx.x, jj = threadIdx.y;
  int blk = blockIdx.x;
  const int chb = blk % nchb; blk /= nchb;
  const int cb = blk % ncolb; blk /= ncolb;
  const int strip = blk % nstrip;
  const int b = blk / nstrip;
  const int j = cb * blockDim.y + jj;
  const int cl = cg * VW;  // channel offset inside this block's slab
  const int c0 = chb * blockDim.x * VW + cl;
  const bool active = j < cols && c0 < D;
  const long L = (long)gh * gw;

  float acc[10][VW];
#pragma unroll
  for (int t = 0; t < 10; ++t)
#pragma unroll
    for (int v = 0; v < VW; ++v) acc[t][v] = 0.f;

  if (active) {
    auto loadx = [&](int ii, int jc, float* out) {
      if (ii < 0 || ii >= rows || jc < 0 || jc >= cols) {
#pragma unroll
        for (int v = 0; v < VW; ++v) out[v] = 0.f;
        return;
      }
      const long p = (long)ii * cols + jc;
      const Vec<T, VW> vv = *reinterpret_cast<const Vec<T, VW>*>(x + ((long)b * L + p) * D + c0);
#pragma unroll
      for (int v = 0; v < VW; ++v) out[v] = to_f(vv.v[v]);
    };
    const int i0 = strip * SR, i1 = min(rows, i0 + SR);
    float win[3][3][VW];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      loadx(i0 - 1, j + s - 1, win[0][s]);
      loadx(i0, j + s - 1, win[1][s]);
    }
    for (int i = i0; i < i1; ++i) {
#pragma unroll
      for (int s = 0; s < 3; ++s) loadx(i + 1, j + s - 1, win[2][s]);
      const long p = (long)i * cols + j;
      const long grow = scan_inv(out_layout, scan_pi(layout, p, gh, gw, L), gh, gw, L);
      const Vec<T, VW> gv = *reinterpret_cast<const Vec<T, VW>*>(dy + ((long)b * L + grow) * D + c0);
#pragma unroll
      for (int v = 0; v < VW; ++v) {
        const float g = to_f(gv.v[v]);
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
          for (int s = 0; s < 3; ++s) acc[a * 3 + s][v] = fmaf(g, win[a][s][v], acc[a * 3 + s][v]);
        acc[9][v] += g;
      }
#pragma unroll
      for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int v = 0; v < VW; ++v) {
          win[0][s][v] = win[1][s][v];
          win[1][s][v] = win[2][s][v];
        }
    }
  }

  const int slab = blockDim.x * VW;
  for (int t = 0; t < 10; ++t) {
#pragma unroll
    for (int v = 0; v < VW; ++v) red[jj * slab + cl + v] = acc[t][v];
    __syncthreads();
    if (jj == 0 && c0 < D) {
#pragma unroll
      for (int v = 0; v < VW; ++v) {
        float s = 0.f;
        for (int q = 0; q < (int)blockDim.y; ++q) s += red[q * slab + cl + v];
        part[((long)(blockIdx.x / nchb) * 10 + t) * D + c0 + v] = s;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void dwconv_dw_reduce(const float* __restrict__ part, int nblk,
                                                        int D, float* __restrict__ dw,
                                                        float* __restrict__ dbias) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= 10L * D) return;
  const int t = (int)(idx / D), c = (int)(idx - (long)t * D);
  float s = 0.f;
  for (int i = 0; i < nblk; ++i) s += part[((long)i * 10 + t) * D + c];
  if (t < 9)
    dw[c * 9 + t] = s;
  else if (dbias)
    dbias[c] = s;
}

// ------------------------------------------------------------------ planning
struct ConvPlan {
  int VW, cgs, nchb, nj, rows, cols, SR, ncolb, nstrip, nblocks;
};

static ConvPlan conv_plan(int B, int gh, int gw, int D, int elt, int layout, int SR, int max_vw) {
  ConvPlan c;
  const bool col = layout == kCol || layout == kColRev;
  c.rows = col ? gw : gh;
  c.cols = col ? gh : gw;
  int vw = 16 / elt;
  if (vw > max_vw) vw = max_vw;
  while (vw > 1 && D % vw) vw >>= 1;
  c.VW = vw;
  const int groups = D / vw;  // vw divides D
  c.cgs = groups < 256 ? groups : 256;
  c.nchb = (groups + c.cgs - 1) / c.cgs;
  c.nj = 256 / c.cgs;
  if (c.nj < 1) c.nj = 1;
  if (c.nj > c.cols) c.nj = c.cols;
  c.SR = SR < c.rows ? SR : c.rows;
  if (c.SR < 1) c.SR = 1;
  c.ncolb = (c.cols + c.nj - 1) / c.nj;
  c.nstrip = (c.rows + c.SR - 1) / c.SR;
  c.nblocks = B * c.ncolb * c.nstrip * c.nchb;
  return c;
}

constexpr int kConvSR = 16;
constexpr int kDwSR = 64;

template <typename T, bool BWD>
static hipError_t launch_conv_t(int B, int gh, int gw, int D, int layout, int out_layout,
                                const void* x, const float* w, const float* bias, void* y,
                                hipStream_t st) {
  const ConvPlan c = conv_plan(B, gh, gw, D, sizeof(T), layout, kConvSR, 16 / sizeof(T));
  dim3 blk(c.cgs, c.nj), grd(c.nblocks);
#define DIG_CONV_CASE(V)                                                                       \
  case V:                                                                                      \
    hipLaunchKernelGGL((dwconv_kernel<T, V, BWD>), grd, blk, 0, st, static_cast<const T*>(x),  \
                       w, bias, static_cast<T*>(y), gh, gw, D, layout, out_layout, c.rows,     \
                       c.cols, c.SR, c.ncolb, c.nstrip, c.nchb);                              \
    break;
  switch (c.VW) {
    DIG_CONV_CASE(1)
    DIG_CONV_CASE(2)
    DIG_CONV_CASE(4)
    DIG_CONV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef DIG_CONV_CASE
  return hipGetLastError();
}

hipError_t launch_dwconv(int B, int gh, int gw, int D, int bf16v, int layout, int out_layout,
                         const void* x, const float* w, const float* bias, void* y,
                         hipStream_t st) {
  if (bf16v) return launch_conv_t<bf16, false>(B, gh, gw, D, layout, out_layout, x, w, bias, y, st);
  return launch_conv_t<float, false>(B, gh, gw, D, layout, out_layout, x, w, bias, y, st);
}

static ConvPlan dw_plan(int B, int gh, int gw, int D, int elt, int layout) {
  return conv_plan(B, gh, gw, D, elt, layout, kDwSR, 16 / elt);
}

size_t dwconv_bwd_workspace(int B, int gh, int gw, int D) {
  size_t best = 0;
  for (int elt = 2; elt <= 4; elt += 2)
    for (int lay = 0; lay < 4; lay += 2) {
      const ConvPlan c = dw_plan(B, gh, gw, D, elt, lay);
      const size_t b = (size_t)(c.nblocks / c.nchb) * 10 * D * sizeof(float);
      if (b > best) best = b;
    }
  return best;
}

template <typename T>
static hipError_t launch_dw_t(int B, int gh, int gw, int D, int layout, int out_layout,
                              const void* x, const void* dy, float* dw, float* dbias,
                              float* part, hipStream_t st) {
  const ConvPlan c = dw_plan(B, gh, gw, D, sizeof(T), layout);
  dim3 blk(c.cgs, c.nj), grd(c.nblocks);
  const size_t shm = (size_t)c.nj * c.cgs * c.VW * sizeof(float);
#define DIG_DW_CASE(V)                                                                        \
  case V:                                                                                     \
    hipLaunchKernelGGL((dwconv_dw_kernel<T, V>), grd, blk, shm, st, static_cast<const T*>(x), \
                       static_cast<const T*>(dy), part, gh, gw, D, layout, out_layout, c.rows, \
                       c.cols, c.SR, c.ncolb, c.nstrip, c.nchb);                             \
    break;
  switch (c.VW) {
    DIG_DW_CASE(1)
    DIG_DW_CASE(2)
    DIG_DW_CASE(4)
    DIG_DW_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef DIG_DW_CASE
  const long n = 10L * D;
  hipLaunchKernelGGL(dwconv_dw_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part,
                     c.nblocks / c.nchb, D, dw, dbias);
  return hipGetLastError();
}

hipError_t launch_dwconv_bwd(int B, int gh, int gw, int D, int bf16v, int layout, int out_layout,
                             const void* x, const float* w, const void* dy, void* dx, float* dw,
                             float* dbias, void* workspace, hipStream_t st) {
  hipError_t e;
  if (bf16v) {
    e = launch_conv_t<bf16, true>(B, gh, gw, D, layout, out_layout, dy, w, nullptr, dx, st);
    if (e != hipSuccess) return e;
    return launch_dw_t<bf16>(B, gh, gw, D, layout, out_layout, x, dy, dw, dbias,
                             static_cast<float*>(workspace), st);
  }
  e = launch_conv_t<float, true>(B, gh, gw, D, layout, out_layout, dy, w, nullptr, dx, st);
  if (e != hipSuccess) return e;
  return launch_dw_t<float>(B, gh, gw, D, layout, out_layout, x, dy, dw, dbias,
                            static_cast<float*>(workspace), st);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t g = (n + 255) / 256;
  if (g > 1024) g = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)g), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace dig
