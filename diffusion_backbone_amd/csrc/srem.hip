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
#include <mutex>

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

// Buffer-resource access: a per-image resource (base, byte size) in scalar registers, the
// lane's byte offset in one vector register and a uniform byte offset (a row) in a scalar
// register, so stepping to the next row costs no vector instruction.  Every access here lies
// inside the resource.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t image_rsrc(const void* base, long bytes) {
  constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 raw buffer: no format conversion
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRawBufferWord3);
}
template <typename V>
__device__ __forceinline__ V buf_ld(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
  static_assert(sizeof(V) == 4 || sizeof(V) == 8, "4- or 8-byte lanes");
  V v;
  if constexpr (sizeof(V) == 4) {
    const unsigned u = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    __builtin_memcpy(&v, &u, 4);
  } else {
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    __builtin_memcpy(&v, &u, 8);
  }
  return v;
}
template <typename V>
__device__ __forceinline__ void buf_st(const V& v, __amdgpu_buffer_rsrc_t r, unsigned voff,
                                       unsigned soff) {
  static_assert(sizeof(V) == 4 || sizeof(V) == 8, "4- or 8-byte lanes");
  if constexpr (sizeof(V) == 4) {
    unsigned u;
    __builtin_memcpy(&u, &v, 4);
    __builtin_amdgcn_raw_buffer_store_b32(u, r, voff, soff, 0);
  } else {
    unsigned __attribute__((ext_vector_type(2))) u;
    __builtin_memcpy(&u, &v, 8);
    __builtin_amdgcn_raw_buffer_store_b64(u, r, voff, soff, 0);
  }
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
  // eight running sums combined in a fixed order; 32 partials are loaded before any is added,
  // so up to 32 partials cost one memory round trip
  float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* pc = part + (long)t * D + c;
  const long step = 10L * D;
  int i = 0;
  for (; i + 32 <= nblk; i += 32) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = pc[(long)(i + u) * step];
#pragma unroll
    for (int u = 0; u < 32; ++u) s8[u & 7] += v[u];
  }
  for (; i + 8 <= nblk; i += 8)
#pragma unroll
    for (int u = 0; u < 8; ++u) s8[u] += pc[(long)(i + u) * step];
  for (; i < nblk; ++i) s8[0] += pc[(long)i * step];
  float s = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
  if (t < 9)
    dw[c * 9 + t] = s;
  else if (dbias)
    dbias[c] = s;
}

// ---------------------------------------------------- scan-order map of the grid
// Position of the token at current-grid (i, j) in another scan order: an affine function
// A + Bi i + Bj j of the grid indices (each scan order is a flip and/or transpose of the
// canonical row-major grid), so the fused reorient costs no division in the kernel.
struct GridMap {
  long A, Bi, Bj;
};
static GridMap grid_map(int gh, int gw, int layout, int out_layout) {
  const long L = (long)gh * gw;
  // canonical (ci, cj) of current-grid (i, j): ci = c0 + cii i + cij j, cj = d0 + dji i + djj j
  long c0 = 0, cii = 0, cij = 0, d0 = 0, dji = 0, djj = 0;
  switch (layout) {
    case kRow: cii = 1; djj = 1; break;
    case kRowRev: c0 = gh - 1; cii = -1; d0 = gw - 1; djj = -1; break;
    case kCol: cij = 1; dji = 1; break;
    default: c0 = gh - 1; cij = -1; d0 = gw - 1; dji = -1; break;
  }
  // position in out_layout of canonical (ci, cj): o0 + oi ci + oj cj
  long o0 = 0, oi = 0, oj = 0;
  switch (out_layout) {
    case kRow: oi = gw; oj = 1; break;
    case kRowRev: o0 = L - 1; oi = -gw; oj = -1; break;
    case kCol: oi = 1; oj = gh; break;
    default: o0 = L - 1; oi = -1; oj = -gh; break;
  }
  return GridMap{o0 + oi * c0 + oj * d0, oi * cii + oj * dji, oi * cij + oj * djj};
}

// ------------------------------------------------------------------ reorient
// Whole token rows move: the row of current position s goes to its position in the target
// order, the affine map A + Bi i + Bj j of its grid indices (i, j) = (s / cols, s mod cols).
// One wave per row at a time, the row index and its destination wave-uniform (scalar
// arithmetic); each lane moves CPR 16-byte pieces of U rows, all loads before the stores.
// Pieces past the row end and rows past the end repeat the last ones (identical values
// written twice), so no branch surrounds a load or store.
template <int CPR>
__global__ __launch_bounds__(256) void reorient_rows_kernel(const uint4* __restrict__ x,
                                                            uint4* __restrict__ y, int nrows,
                                                            int L, int cols, int nv, GridMap m) {
  constexpr int U = 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nw = (int)gridDim.x * 4;
  for (int r0 = (int)blockIdx.x * 4 + wave; r0 < nrows; r0 += nw * U) {
    uint4 buf[U][CPR];
    long dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(r0 + u * nw, nrows - 1);
      const int b = r / L, s = r - b * L;
      const int i = s / cols, j = s - i * cols;
      dst[u] = ((long)b * L + m.A + m.Bi * i + m.Bj * j) * nv;
      const uint4* src = x + (long)r * nv;
#pragma unroll
      for (int c = 0; c < CPR; ++c) buf[u][c] = src[min(lane + 64 * c, nv - 1)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int c = 0; c < CPR; ++c) y[dst[u] + min(lane + 64 * c, nv - 1)] = buf[u][c];
  }
}

// Fallback for rows that are not whole 16-byte pieces or longer than 8 KiB: a grid-stride
// loop over elements.
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
  // (the row loop's indices reach rows + 3 * 4 * blocks_cap in int: kept below 2^31)
  if (rowbytes % 16 == 0 && rowbytes <= 16 * 64 * 8 && rows < (1L << 31) - (1L << 17)) {
    const int nv = (int)(rowbytes / 16), cpr = (nv + 63) / 64;
    const bool col = from == kCol || from == kColRev;
    const GridMap m = grid_map(gh, gw, from, to);
    long g = (rows + 7) / 8;  // 4 waves x 2 rows per block step
    if (g > blocks_cap) g = blocks_cap;
#define DIG_REO_CASE(N)                                                                       \
  case N:                                                                                     \
    hipLaunchKernelGGL(reorient_rows_kernel<N>, dim3((unsigned)g), dim3(256), 0, st,           \
                       static_cast<const uint4*>(x), static_cast<uint4*>(y), (int)rows, (int)L, \
                       col ? gh : gw, nv, m);                                                  \
    break;
    switch (cpr) {
      DIG_REO_CASE(1)
      DIG_REO_CASE(2)
      DIG_REO_CASE(3)
      DIG_REO_CASE(4)
      DIG_REO_CASE(5)
      DIG_REO_CASE(6)
      DIG_REO_CASE(7)
      DIG_REO_CASE(8)
      default: return hipErrorInvalidValue;
    }
#undef DIG_REO_CASE
  } else if (rowbytes % 16 == 0) {
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

// ------------------------------------------------------------ LDS-tiled conv
// One block: an 8 x 8 tile of current-grid positions x one 128-byte channel slab.  The
// 10 x 10 halo tile arrives through global->LDS DMA (one round trip); positions outside the
// grid are zero-filled.  Used when the slab divides the channel count.
constexpr int kTile = 8, kHalo = kTile + 2, kSlabBytes = 128;

template <typename T, bool GATHER>
__device__ __forceinline__ void load_halo(T* tile, const T* x, long bL, int D, int c0, int i0,
                                          int j0, int rows, int cols, GridMap m, int wave,
                                          int lane) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NG = kSlabBytes / 16;  // 16-byte pieces per position
  constexpr int NP = kHalo * kHalo * NG;
  unsigned char* tb = reinterpret_cast<unsigned char*>(tile);
  for (int base = wave * 64; base < NP; base += 4 * 64) {
    const int e = base + lane;
    if (e < NP) {
      const int pos = e / NG, k = e - pos * NG;
      const int hi = pos / kHalo, hj = pos - hi * kHalo;
      const int ii = i0 - 1 + hi, jj = j0 - 1 + hj;
      if (ii >= 0 && ii < rows && jj >= 0 && jj < cols) {
        const long row = GATHER ? m.A + m.Bi * ii + m.Bj * jj : (long)ii * cols + jj;
        const T* g = x + (bL + row) * D + c0 + k * VEC;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)(tb + base * 16), 16, 0, 0);
      } else {
        *reinterpret_cast<uint4*>(tb + (long)e * 16) = make_uint4(0, 0, 0, 0);
      }
    }
  }
}

// The slab's taps, w[c0 .. c0+CS)[9] (contiguous), staged into LDS tap-major, wl[tap][CS],
// with coalesced loads; read back after the block's barrier as 16-byte runs of channels.
template <int CS>
__device__ __forceinline__ void stage_taps(float* wl, const float* w, int c0, int tid) {
  for (int e = tid; e < 9 * CS; e += 256) {
    const int ch = e / 9, t = e - ch * 9;
    wl[t * CS + ch] = w[(long)c0 * 9 + e];
  }
}
template <int CS, int VEC>
__device__ __forceinline__ void read_taps(float (&wr)[9][VEC], const float* wl, int cl, bool rot) {
#pragma unroll
  for (int t = 0; t < 9; ++t) {
    const float4* src = reinterpret_cast<const float4*>(wl + (rot ? 8 - t : t) * CS + cl);
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      const float4 f = src[q];
      wr[t][4 * q] = f.x; wr[t][4 * q + 1] = f.y; wr[t][4 * q + 2] = f.z; wr[t][4 * q + 3] = f.w;
    }
  }
}

// Forward: out[p'] = sum_taps w x + b, written at the position of p's token in out_layout.
template <typename T>
__global__ __launch_bounds__(256) void dwconv_tiled_kernel(const T* __restrict__ x,
                                                           const float* __restrict__ w,
                                                           const float* __restrict__ bias,
                                                           T* __restrict__ y, int D, long L,
                                                           GridMap m, int rows, int cols,
                                                           int ntr, int ntc, int nslab) {
  constexpr int CS = kSlabBytes / sizeof(T);  // channels per slab
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NG = CS / VEC;                // = 8 pieces per position
  __shared__ __align__(16) T tile[kHalo * kHalo * CS];
  __shared__ __align__(16) float wl[9 * CS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int slab = blk % nslab; blk /= nslab;
  const int tc = blk % ntc; blk /= ntc;
  const int tr = blk % ntr;
  const int b = blk / ntr;
  const int i0 = tr * kTile, j0 = tc * kTile, c0 = slab * CS;
  const long bL = (long)b * L;

  load_halo<T, false>(tile, x, bL, D, c0, i0, j0, rows, cols, m, wave, lane);

  const int g = tid % NG, pl = tid / NG;  // channel group, first output position
  stage_taps<CS>(wl, w, c0, tid);
  float bs[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) bs[v] = bias ? bias[c0 + g * VEC + v] : 0.f;
  dma_wait();
  __syncthreads();
  float wr[9][VEC];
  read_taps<CS, VEC>(wr, wl, g * VEC, false);

#pragma unroll
  for (int task = 0; task < 2; ++task) {
    const int q = pl + 32 * task, oi = q / kTile, oj = q - oi * kTile;
    const int i = i0 + oi, j = j0 + oj;
    if (i < rows && j < cols) {
      float acc[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = bs[v];
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int s2 = 0; s2 < 3; ++s2) {
          const Vec<T, VEC> xv =
              *reinterpret_cast<const Vec<T, VEC>*>(tile + ((oi + a) * kHalo + oj + s2) * CS + g * VEC);
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] = fmaf(wr[a * 3 + s2][v], to_f(xv.v[v]), acc[v]);
        }
      Vec<T, VEC> o;
#pragma unroll
      for (int v = 0; v < VEC; ++v) o.v[v] = from_f<T>(acc[v]);
      const long orow = m.A + m.Bi * i + m.Bj * j;
      *reinterpret_cast<Vec<T, VEC>*>(y + (bL + orow) * D + c0 + g * VEC) = o;
    }
  }
}

// Backward of one 8 x 8 tile x 128-byte slab in one pass: the dy halo tile (gathered back to
// the current order) and the x halo tile arrive by LDS DMA; each thread forms dx at its two
// positions (taps rotated by 180 degrees) and accumulates dy(i, j) * x(i+a-1, j+s-1) (taps
// 0..8) and dy(i, j) (tap 9, the bias).  The 32 position lanes of a channel group are then
// summed in a fixed order: lane pairs of a 16-lane row by DPP, the 16 row partials through
// LDS (reusing the tile space), all taps behind one barrier, into part[tile][tap][D], tile
// over (b, tile row, tile column).
template <typename T>
__global__ __launch_bounds__(256) void dwconv_bwd_tiled_kernel(const T* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               const T* __restrict__ dy,
                                                               T* __restrict__ dx,
                                                               float* __restrict__ part, int D,
                                                               long L, GridMap m, int rows,
                                                               int cols, int ntr, int ntc,
                                                               int nslab) {
  constexpr int CS = kSlabBytes / sizeof(T);
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NG = CS / VEC;
  static_assert(NG == 8, "a 16-lane row holds two positions of one channel group");
  constexpr int NRP = 16, RP = NRP + 1;  // row partials per channel, odd pitch
  constexpr int TILE_BYTES = 2 * kHalo * kHalo * CS * (int)sizeof(T) + 9 * CS * (int)sizeof(float);
  constexpr int RED_BYTES = 10 * CS * RP * (int)sizeof(float);
  __shared__ __align__(16) unsigned char sm[TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES];
  T* dyt = reinterpret_cast<T*>(sm);
  T* xt = dyt + kHalo * kHalo * CS;
  float* wl = reinterpret_cast<float*>(xt + kHalo * kHalo * CS);
  float* red = reinterpret_cast<float*>(sm);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int blk = blockIdx.x;
  const int slab = blk % nslab; blk /= nslab;
  const int tc = blk % ntc; blk /= ntc;
  const int tr = blk % ntr;
  const int b = blk / ntr;
  const int i0 = tr * kTile, j0 = tc * kTile, c0 = slab * CS;
  const long bL = (long)b * L;

  load_halo<T, true>(dyt, dy, bL, D, c0, i0, j0, rows, cols, m, wave, lane);
  load_halo<T, false>(xt, x, bL, D, c0, i0, j0, rows, cols, m, wave, lane);
  const int g = tid % NG, pl = tid / NG;  // channel group, first position
  stage_taps<CS>(wl, w, c0, tid);
  float acc[10][VEC];
#pragma unroll
  for (int t = 0; t < 10; ++t)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[t][v] = 0.f;
  dma_wait();
  __syncthreads();
  float wr[9][VEC];
  read_taps<CS, VEC>(wr, wl, g * VEC, true);

#pragma unroll
  for (int task = 0; task < 2; ++task) {
    const int q = pl + 32 * task, oi = q / kTile, oj = q - oi * kTile;
    const int i = i0 + oi, j = j0 + oj;
    if (i < rows && j < cols) {
      const Vec<T, VEC> gc =
          *reinterpret_cast<const Vec<T, VEC>*>(dyt + ((oi + 1) * kHalo + oj + 1) * CS + g * VEC);
      float o[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[v] = 0.f;
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int s2 = 0; s2 < 3; ++s2) {
          const int h = ((oi + a) * kHalo + oj + s2) * CS + g * VEC;
          const Vec<T, VEC> dv = *reinterpret_cast<const Vec<T, VEC>*>(dyt + h);
          const Vec<T, VEC> xv = *reinterpret_cast<const Vec<T, VEC>*>(xt + h);
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            o[v] = fmaf(wr[a * 3 + s2][v], to_f(dv.v[v]), o[v]);
            acc[a * 3 + s2][v] = fmaf(to_f(gc.v[v]), to_f(xv.v[v]), acc[a * 3 + s2][v]);
          }
        }
      Vec<T, VEC> ov;
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        acc[9][v] += to_f(gc.v[v]);
        ov.v[v] = from_f<T>(o[v]);
      }
      *reinterpret_cast<Vec<T, VEC>*>(dx + (bL + (long)i * cols + j) * D + c0 + g * VEC) = ov;
    }
  }

  // lanes l and l ^ 8 of a row hold positions pl and pl ^ 1 of the same channel group
#pragma unroll
  for (int t = 0; t < 10; ++t)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[t][v] += dpp_f<0x128>(acc[t][v]);
  __syncthreads();  // tiles and taps are dead: their space becomes red[tap][channel][row partial]
  if ((tid & 8) == 0) {
    const int rp = tid >> 4;
#pragma unroll
    for (int t = 0; t < 10; ++t)
#pragma unroll
      for (int v = 0; v < VEC; ++v) red[(t * CS + g * VEC + v) * RP + rp] = acc[t][v];
  }
  __syncthreads();
  const long pblk = ((long)b * ntr + tr) * ntc + tc;
  for (int o = tid; o < 10 * CS; o += 256) {
    const float* r = red + o * RP;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NRP; ++q) s4[q & 3] += r[q];
    const int t = o / CS, ch = o - t * CS;
    part[(pblk * 10 + t) * D + c0 + ch] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  }
}

// ------------------------------------------------------------ column-strip conv
// One block: a strip of W current-grid columns x rh rows x one 128-byte channel slab of G
// groups of kStripVec channels (4 bytes per lane in bf16, 8 in fp32; G W = 256).  Thread
// (group g, column j) streams down its column: input rows arrive in groups of kStripK, two
// groups in flight while the previous ones are consumed, and each row's three vectors
// (columns j-1, j, j+1; the side columns are the adjacent lanes' centre loads and come from
// L1) enter a rolling 3-row window of floats.  No branch surrounds a load or store (the
// compiler would then wait for every outstanding access): rows and columns outside the grid
// are loaded clamped and scaled by zero (rows) or get zero taps (columns); columns past the
// grid repeat the last one and the last row group overlaps its neighbour, both writing
// identical values.  rh is a multiple of 2 kStripK and at most the row count.  Row bases are
// uniform and lane offsets 32-bit (one image is below 2^31 bytes).
constexpr int kStripVec = 2, kStripSlabBytes = 128, kStripK = 4;

// Byte offset from a uniform row base of the token at map position Bj jj: with Bj < 0 the
// lane term is taken over the reflected column so that it stays non-negative, the constant
// Bj (cols - 1) moving into the base (see map_base).
__device__ __forceinline__ unsigned map_lane_off(const GridMap& m, int jj, int cols, int D, int c,
                                                 int elt) {
  const bool rev = m.Bj < 0;
  return (unsigned)(((rev ? cols - 1 - jj : jj) * (rev ? -m.Bj : m.Bj) * D + c) * (long)elt);
}
__device__ __forceinline__ long map_base(const GridMap& m, int cols) {
  return m.A + (m.Bj < 0 ? m.Bj * (cols - 1) : 0);
}

// Workgroups are handed to the 8 XCDs (each with its own L2) in turn, workgroup i to XCD
// i mod 8.  Tiles are ordered slab fastest, then strip, and XCD x takes the x-th contiguous
// eighth of them: the slabs of a strip run together (whole token rows are read and written
// at about the same time) and the halo columns a block reads from its neighbour strips are
// mostly in its own XCD's L2.
__device__ __forceinline__ int xcd_tile(int blk, int nblk) {
  constexpr int kXcds = 8;
  const int x = blk % kXcds, local = blk / kXcds;
  const int n8 = nblk / kXcds, rem = nblk % kXcds;
  return x * n8 + min(x, rem) + local;
}

// Lane geometry shared by the strip kernels.
template <typename T>
struct StripLane {
  static constexpr int VEC = kStripVec;
  static constexpr int G = kStripSlabBytes / (VEC * (int)sizeof(T));  // groups per slab
  static constexpr int W = 256 / G;                                   // columns per strip
  static constexpr int CS = G * VEC;                                  // channels per slab
  int g, jc, slab, strip, rg, b, c0, c, i0, jr, j, jm, jp;
  long bL;
  float ml, mr;  // 0 where the left / right neighbour column is outside the grid
  __device__ StripLane(int rows, int cols, long L, int nslab, int nstrip, int nrg, int rh) {
    const int tid = threadIdx.x;
    g = tid % G; jc = tid / G;
    int blk = xcd_tile(blockIdx.x, gridDim.x);
    slab = blk % nslab; blk /= nslab;
    strip = blk % nstrip; blk /= nstrip;
    rg = blk % nrg;
    b = blk / nrg;
    c0 = slab * CS; c = c0 + g * VEC;
    i0 = min(rg * rh, rows - rh);
    jr = strip * W + jc; j = min(jr, cols - 1);
    jm = max(j - 1, 0); jp = min(j + 1, cols - 1);
    bL = (long)b * L;
    ml = j > 0 ? 1.f : 0.f; mr = j < cols - 1 ? 1.f : 0.f;
  }
};

// The lane's taps w[c .. c+VEC)[9]: 9 VEC contiguous floats, 8-byte aligned (VEC even).
template <int VEC>
__device__ __forceinline__ void lane_taps(float (&wv)[9 * VEC], const float* w, int c) {
  const float2* wp = reinterpret_cast<const float2*>(w + (long)c * 9);
#pragma unroll
  for (int q = 0; q < 9 * VEC / 2; ++q) {
    const float2 f = wp[q];
    wv[2 * q] = f.x;
    wv[2 * q + 1] = f.y;
  }
}

// A channel pair as floats.  bf16 pairs are widened with byte permutes of the loaded dword
// (a shift or mask of it lets the compiler re-load the upper half as a separate 16-bit load).
template <typename T>
__device__ __forceinline__ void pair_f(const Vec<T, 2>& p, float& lo, float& hi) {
  if constexpr (sizeof(T) == 2) {
    const unsigned u = *reinterpret_cast<const unsigned*>(&p);
    lo = __uint_as_float(__builtin_amdgcn_perm(0u, u, 0x01000c0cu));
    hi = __uint_as_float(__builtin_amdgcn_perm(0u, u, 0x03020c0cu));
  } else {
    lo = to_f(p.v[0]);
    hi = to_f(p.v[1]);
  }
}
template <typename T, int VEC>
__device__ __forceinline__ void vec_f(const Vec<T, VEC>& p, float (&f)[VEC]) {
  static_assert(VEC % 2 == 0, "channel pairs");
#pragma unroll
  for (int q = 0; q < VEC / 2; ++q)
    pair_f<T>(reinterpret_cast<const Vec<T, 2>*>(&p)[q], f[2 * q], f[2 * q + 1]);
}
template <typename T, int VEC>
__device__ __forceinline__ void cvt3(float (&dst)[3][VEC], const Vec<T, VEC> (&src)[3], float sc) {
#pragma unroll
  for (int s2 = 0; s2 < 3; ++s2) {
    float f[VEC];
    vec_f<T, VEC>(src[s2], f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) dst[s2][e] = sc * f[e];
  }
}
template <int VEC>
__device__ __forceinline__ void copy3(float (&dst)[3][VEC], const float (&src)[3][VEC]) {
#pragma unroll
  for (int s2 = 0; s2 < 3; ++s2)
#pragma unroll
    for (int e = 0; e < VEC; ++e) dst[s2][e] = src[s2][e];
}

// Forward: y at the position of (i, j) in out_layout (map m) = sum_{a,s} w[a][s] x(i+a-1,
// j+s-1) + b, x read in the current order.  `bscale` is 0 when there is no bias (then `bias`
// points at any readable D floats).
template <typename T>
__global__ __launch_bounds__(256) void dwconv_strip_kernel(const T* __restrict__ x,
                                                           const float* __restrict__ w,
                                                           const float* __restrict__ bias,
                                                           T* __restrict__ y, int rows, int cols,
                                                           int D, long L, GridMap m,
                                                           float bscale, int nslab, int nstrip,
                                                           int nrg, int rh) {
  using Ln = StripLane<T>;
  constexpr int VEC = Ln::VEC, K = kStripK;
  using V = Vec<T, VEC>;
  const Ln ln(rows, cols, L, nslab, nstrip, nrg, rh);
  const int i0 = ln.i0;

  const long ibytes = L * D * (long)sizeof(T), rowb = (long)cols * D * (long)sizeof(T);
  const __amdgpu_buffer_rsrc_t rx = image_rsrc(x + ln.bL * D, ibytes);
  const unsigned oM = (unsigned)(((long)ln.jm * D + ln.c) * (long)sizeof(T));
  const unsigned oC = (unsigned)(((long)ln.j * D + ln.c) * (long)sizeof(T));
  const unsigned oP = (unsigned)(((long)ln.jp * D + ln.c) * (long)sizeof(T));
  auto load_row = [&](V (&dst)[3], int ii) {
    const unsigned ro = (unsigned)(min(max(ii, 0), rows - 1) * rowb);
    dst[0] = buf_ld<V>(rx, oM, ro);
    dst[1] = buf_ld<V>(rx, oC, ro);
    dst[2] = buf_ld<V>(rx, oP, ro);
  };
  // group q holds input rows i0 + qK + 1 .. i0 + qK + K (the row below each output row)
  V bufA[K][3], bufB[K][3];
  auto load_group = [&](V (&buf)[K][3], int q) {
#pragma unroll
    for (int k = 0; k < K; ++k) load_row(buf[k], i0 + q * K + 1 + k);
  };
  V top[2][3];
  load_row(top[0], i0 - 1);
  load_row(top[1], i0);
  load_group(bufA, 0);
  load_group(bufB, 1);

  float wv[9 * VEC];
  lane_taps<VEC>(wv, w, ln.c);
  float wr[3][3][VEC];
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int s2 = 0; s2 < 3; ++s2)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        wr[a][s2][e] = wv[e * 9 + a * 3 + s2] * (s2 == 0 ? ln.ml : (s2 == 2 ? ln.mr : 1.f));
  float bs[VEC];
#pragma unroll
  for (int q = 0; q < VEC / 2; ++q) {
    const float2 bb = reinterpret_cast<const float2*>(bias + ln.c)[q];
    bs[2 * q] = bscale * bb.x;
    bs[2 * q + 1] = bscale * bb.y;
  }
  // y's position of (i, j) is A + Bi i + Bj j: a uniform row offset (a valid position, so
  // non-negative) plus a lane offset
  const __amdgpu_buffer_rsrc_t ry = image_rsrc(y + ln.bL * D, ibytes);
  const long ybase = map_base(m, cols);
  const unsigned oY = map_lane_off(m, ln.j, cols, D, ln.c, (int)sizeof(T));

  float fa[3][VEC], fb[3][VEC];  // window rows i-1 and i
  cvt3<T, VEC>(fa, top[0], i0 > 0 ? 1.f : 0.f);
  cvt3<T, VEC>(fb, top[1], 1.f);
  // only the block's last row can have its lower neighbour outside the grid
  const float m_bot = i0 + rh < rows ? 1.f : 0.f;
  auto process = [&](const V (&buf)[K][3], int q, auto last) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = i0 + q * K + k;
      float fc[3][VEC];
      cvt3<T, VEC>(fc, buf[k], decltype(last)::value && k == K - 1 ? m_bot : 1.f);
      V o;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float acc = bs[e];
#pragma unroll
        for (int s2 = 0; s2 < 3; ++s2) {
          acc = fmaf(wr[0][s2][e], fa[s2][e], acc);
          acc = fmaf(wr[1][s2][e], fb[s2][e], acc);
          acc = fmaf(wr[2][s2][e], fc[s2][e], acc);
        }
        o.v[e] = from_f<T>(acc);
      }
      buf_st<V>(o, ry, oY, (unsigned)((ybase + m.Bi * i) * D * (long)sizeof(T)));
      copy3<VEC>(fa, fb);
      copy3<VEC>(fb, fc);
    }
  };
  const int ng = rh / K;  // even, >= 2
  for (int q = 0; q < ng - 2; q += 2) {
    process(bufA, q, std::false_type{});
    load_group(bufA, q + 2);
    process(bufB, q + 1, std::false_type{});
    load_group(bufB, q + 3);
  }
  process(bufA, ng - 2, std::false_type{});
  process(bufB, ng - 1, std::true_type{});
}

// Backward of the conv in one pass over column strips: dx and the dW/dbias partials.  Thread
// (group g, column j) owns VEC channels of one current-grid column and streams its rh rows as
// the forward does.  With the dy window win[u][v] = dy(i-1+u, j-1+v) around the input
// position (i, j), dy being zero outside the grid, the adjoint of y(i, j) = sum_{a,s} w[a][s]
// x(i+a-1, j+s-1) + b is
//   dx(i, j) = sum_{u,v} w[2-u][2-v] win[u][v],   dw[2-u][2-v] += x(i, j) win[u][v],
//   dbias += win[1][1]
// so one window serves both, and dy is read once per position (x and dx once each).
// Out-of-grid dy rows are loaded clamped and scaled by zero; out-of-grid dy columns get zero
// dx taps and have their dW sums cleared at the end (a lane's column is fixed).  Positions a
// thread does not own (columns past the grid repeating the last one, rows of an overlapping
// last row group that the previous group owns) add nothing to dW and rewrite identical dx.
// The block's W columns are summed in a fixed order through LDS into part[blk][tap][D], blk
// over (b, strip, row group).
template <typename T>
__global__ __launch_bounds__(256) void dwconv_bwd_strip_kernel(
    const T* __restrict__ x, const float* __restrict__ w, const T* __restrict__ dy,
    T* __restrict__ dx, float* __restrict__ part, int rows, int cols, int D, long L, GridMap m,
    int nslab, int nstrip, int nrg, int rh) {
  using Ln = StripLane<T>;
  constexpr int VEC = Ln::VEC, K = kStripK, W = Ln::W, CS = Ln::CS;
  using V = Vec<T, VEC>;
  __shared__ float red[W * 10 * CS];
  const Ln ln(rows, cols, L, nslab, nstrip, nrg, rh);
  const int i0 = ln.i0, first_own = ln.rg * rh;
  const float mj = ln.jr < cols ? 1.f : 0.f;

  // dy's position of (ii, jj) is A + Bi ii + Bj jj: a uniform row offset (a valid position,
  // so non-negative) plus a lane offset
  const long ibytes = L * D * (long)sizeof(T), rowb = (long)cols * D * (long)sizeof(T);
  const __amdgpu_buffer_rsrc_t rdy = image_rsrc(dy + ln.bL * D, ibytes);
  const __amdgpu_buffer_rsrc_t rx = image_rsrc(x + ln.bL * D, ibytes);
  const __amdgpu_buffer_rsrc_t rdx = image_rsrc(dx + ln.bL * D, ibytes);
  const long dybase = map_base(m, cols);
  const unsigned oM = map_lane_off(m, ln.jm, cols, D, ln.c, (int)sizeof(T));
  const unsigned oC = map_lane_off(m, ln.j, cols, D, ln.c, (int)sizeof(T));
  const unsigned oP = map_lane_off(m, ln.jp, cols, D, ln.c, (int)sizeof(T));
  const unsigned oX = (unsigned)(((long)ln.j * D + ln.c) * (long)sizeof(T));
  auto load_dy = [&](V (&dst)[3], int ii) {
    const unsigned ro =
        (unsigned)((dybase + m.Bi * min(max(ii, 0), rows - 1)) * D * (long)sizeof(T));
    dst[0] = buf_ld<V>(rdy, oM, ro);
    dst[1] = buf_ld<V>(rdy, oC, ro);
    dst[2] = buf_ld<V>(rdy, oP, ro);
  };
  // group q: dy rows i0 + qK + 1 .. i0 + qK + K (slots 0..2) and x rows i0 + qK .. (slot 3)
  V bufA[K][4], bufB[K][4];
  auto load_group = [&](V (&buf)[K][4], int q) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = i0 + q * K + k;
      V t[3];
      load_dy(t, i + 1);
      buf[k][0] = t[0]; buf[k][1] = t[1]; buf[k][2] = t[2];
      buf[k][3] = buf_ld<V>(rx, oX, (unsigned)(i * rowb));
    }
  };
  V top[2][3];
  load_dy(top[0], i0 - 1);
  load_dy(top[1], i0);
  load_group(bufA, 0);
  load_group(bufB, 1);

  float wv[9 * VEC];
  lane_taps<VEC>(wv, w, ln.c);
  // dx taps, rotated by 180 degrees; out-of-grid side columns get zero taps
  float wr[3][3][VEC];
#pragma unroll
  for (int u = 0; u < 3; ++u)
#pragma unroll
    for (int v = 0; v < 3; ++v)
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        wr[u][v][e] = wv[e * 9 + (2 - u) * 3 + (2 - v)] * (v == 0 ? ln.ml : (v == 2 ? ln.mr : 1.f));
  float acc[10][VEC];
#pragma unroll
  for (int t = 0; t < 10; ++t)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[t][e] = 0.f;

  float fa[3][VEC], fb[3][VEC];  // dy window rows i-1 and i
  cvt3<T, VEC>(fa, top[0], i0 > 0 ? 1.f : 0.f);
  cvt3<T, VEC>(fb, top[1], 1.f);
  // only the block's last row can have its lower neighbour outside the grid
  const float m_bot = i0 + rh < rows ? 1.f : 0.f;
  auto process = [&](const V (&buf)[K][4], int q, auto last) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i = i0 + q * K + k;
      float fc[3][VEC];
      const V dr[3] = {buf[k][0], buf[k][1], buf[k][2]};
      cvt3<T, VEC>(fc, dr, decltype(last)::value && k == K - 1 ? m_bot : 1.f);
      const float md = i >= first_own ? mj : 0.f;
      float xm[VEC], o[VEC];
      vec_f<T, VEC>(buf[k][3], xm);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        xm[e] *= md;
        o[e] = 0.f;
      }
#pragma unroll
      for (int v = 0; v < 3; ++v)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          o[e] = fmaf(wr[0][v][e], fa[v][e], o[e]);
          o[e] = fmaf(wr[1][v][e], fb[v][e], o[e]);
          o[e] = fmaf(wr[2][v][e], fc[v][e], o[e]);
          acc[v][e] = fmaf(xm[e], fa[v][e], acc[v][e]);
          acc[3 + v][e] = fmaf(xm[e], fb[v][e], acc[3 + v][e]);
          acc[6 + v][e] = fmaf(xm[e], fc[v][e], acc[6 + v][e]);
        }
      V ov;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        acc[9][e] = fmaf(md, fb[1][e], acc[9][e]);
        ov.v[e] = from_f<T>(o[e]);
      }
      buf_st<V>(ov, rdx, oX, (unsigned)(i * rowb));
      copy3<VEC>(fa, fb);
      copy3<VEC>(fb, fc);
    }
  };
  const int ng = rh / K;  // even, >= 2
  for (int q = 0; q < ng - 2; q += 2) {
    process(bufA, q, std::false_type{});
    load_group(bufA, q + 2);
    process(bufB, q + 1, std::false_type{});
    load_group(bufB, q + 3);
  }
  process(bufA, ng - 2, std::false_type{});
  process(bufB, ng - 1, std::true_type{});

  // tap t = a*3 + s of dw is window slot 8 - t; clear the sums of out-of-grid side columns
  const int jc = ln.jc, g = ln.g;
#pragma unroll
  for (int t = 0; t < 10; ++t) {
    const int k = t < 9 ? 8 - t : 9;
    const float mk = k % 3 == 0 && k < 9 ? ln.ml : (k % 3 == 2 ? ln.mr : 1.f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[(jc * 10 + t) * CS + g * VEC + e] = mk * acc[k][e];
  }
  __syncthreads();
  const long pblk = ((long)ln.b * nstrip + ln.strip) * nrg + ln.rg;
  for (int o = threadIdx.x; o < 10 * CS; o += 256) {
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < W; ++q) s4[q & 3] += red[q * 10 * CS + o];
    const int t = o / CS, ch = o - t * CS;
    part[(pblk * 10 + t) * D + ln.c0 + ch] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  }
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
constexpr long kStripTargetBlocks = 1024;

// Column-strip plan (forward and backward): W-column strips x rh-row groups x 128-byte
// channel slabs, rh a multiple of 2 kStripK chosen for about kStripTargetBlocks blocks (longer
// row runs when the strips and slabs alone give many).  Used when the slab divides the
// channels, the grid has at least 2 kStripK rows and one image is below 2^31 bytes; grids
// with fewer rows go to the 8 x 8 tiles.  (On the 16 x 16 grid of DiG-S/2 at 256 px, B = 8,
// the strips take 4.0 / 4.9 us forward / backward against 5.1 / 9.1 us on the tiles.)
struct StripPlan {
  bool ok;
  int rows, cols, nslab, nstrip, nrg, rh;
  long blocks;
};
static StripPlan strip_plan(int B, int gh, int gw, int D, int elt, int layout) {
  constexpr int unit = 2 * kStripK;
  const int width = 256 / (kStripSlabBytes / (kStripVec * elt));
  StripPlan p{};
  const bool col = layout == kCol || layout == kColRev;
  p.rows = col ? gw : gh;
  p.cols = col ? gh : gw;
  const int slabc = kStripSlabBytes / elt;
  p.nslab = D / slabc;
  p.nstrip = (p.cols + width - 1) / width;
  if (p.rows < unit || D % slabc != 0 || B < 1) return p;
  const long base = (long)B * p.nstrip * p.nslab;
  long want = (kStripTargetBlocks + base - 1) / base;  // row groups wanted
  if (want < 1) want = 1;
  long rh = ((p.rows + want - 1) / want + unit - 1) / unit * unit;
  const int rmax = p.rows / unit * unit;
  if (rh > rmax) rh = rmax;
  p.rh = (int)rh;
  p.nrg = (p.rows + p.rh - 1) / p.rh;
  p.blocks = base * p.nrg;
  p.ok = (long)p.rows * p.cols * D * elt < (1L << 31);
  return p;
}
constexpr int kDwSR = 64;

// Plan of the LDS-tiled path: 8 x 8 position tiles x 128-byte channel slabs.
struct TilePlan {
  bool ok;
  int rows, cols, ntr, ntc, nslab;
  long conv_blocks;
};

static TilePlan tile_plan(int B, int gh, int gw, int D, int elt, int layout) {
  TilePlan t{};
  const bool col = layout == kCol || layout == kColRev;
  t.rows = col ? gw : gh;
  t.cols = col ? gh : gw;
  t.ok = ((long)D * elt) % kSlabBytes == 0;
  if (!t.ok) return t;
  t.nslab = (int)((long)D * elt / kSlabBytes);
  t.ntr = (t.rows + kTile - 1) / kTile;
  t.ntc = (t.cols + kTile - 1) / kTile;
  t.conv_blocks = (long)B * t.ntr * t.ntc * t.nslab;
  return t;
}

// Forward (column strips on large grids, 8 x 8 tiles on small ones, the generic kernel for
// channel counts no slab divides); the backward's dx uses the generic kernel only (its strip
// and tile paths are fused with the weight gradient).
template <typename T, bool BWD>
static hipError_t launch_conv_t(int B, int gh, int gw, int D, int layout, int out_layout,
                                const void* x, const float* w, const float* bias, void* y,
                                hipStream_t st) {
  if constexpr (!BWD) {
    const StripPlan sp = strip_plan(B, gh, gw, D, sizeof(T), layout);
    if (sp.ok) {
      hipLaunchKernelGGL((dwconv_strip_kernel<T>), dim3((unsigned)sp.blocks), dim3(256), 0, st,
                         static_cast<const T*>(x), w, bias ? bias : w, static_cast<T*>(y),
                         sp.rows, sp.cols, D, (long)gh * gw, grid_map(gh, gw, layout, out_layout),
                         bias ? 1.f : 0.f, sp.nslab, sp.nstrip, sp.nrg, sp.rh);
      return hipGetLastError();
    }
    const TilePlan tp = tile_plan(B, gh, gw, D, sizeof(T), layout);
    if (tp.ok) {
      hipLaunchKernelGGL((dwconv_tiled_kernel<T>), dim3((unsigned)tp.conv_blocks), dim3(256), 0,
                         st, static_cast<const T*>(x), w, bias, static_cast<T*>(y), D,
                         (long)gh * gw, grid_map(gh, gw, layout, out_layout), tp.rows, tp.cols,
                         tp.ntr, tp.ntc, tp.nslab);
      return hipGetLastError();
    }
  }
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

// Number of [10][D] partial-sum slices the dw pass writes for one dtype and layout.
static long dw_partials(int B, int gh, int gw, int D, int elt, int layout) {
  const StripPlan sp = strip_plan(B, gh, gw, D, elt, layout);
  if (sp.ok) return (long)B * sp.nstrip * sp.nrg;
  const TilePlan tp = tile_plan(B, gh, gw, D, elt, layout);
  if (tp.ok) return (long)B * tp.ntr * tp.ntc;
  const ConvPlan c = dw_plan(B, gh, gw, D, elt, layout);
  return c.nblocks / c.nchb;
}

size_t dwconv_bwd_workspace(int B, int gh, int gw, int D) {
  size_t best = 0;
  for (int elt = 2; elt <= 4; elt += 2)
    for (int lay = 0; lay < 4; lay += 2) {
      const size_t b = (size_t)dw_partials(B, gh, gw, D, elt, lay) * 10 * D * sizeof(float);
      if (b > best) best = b;
    }
  return best;
}

template <typename T>
static hipError_t launch_dw_t(int B, int gh, int gw, int D, int layout, int out_layout,
                              const void* x, const void* dy, float* dw, float* dbias,
                              float* part, hipStream_t st) {
  const long n = 10L * D;
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
  hipLaunchKernelGGL(dwconv_dw_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part,
                     c.nblocks / c.nchb, D, dw, dbias);
  return hipGetLastError();
}

// dx and the dW/dbias partials in one pass (column strips on large grids, 8 x 8 tiles on
// small ones; two generic kernels for channel counts no slab divides), then the per-channel
// sums of the partials.
template <typename T>
static hipError_t launch_dwconv_bwd_t(int B, int gh, int gw, int D, int layout, int out_layout,
                                      const void* x, const float* w, const void* dy, void* dx,
                                      float* dw, float* dbias, float* part, hipStream_t st) {
  const long n = 10L * D;
  const StripPlan sp = strip_plan(B, gh, gw, D, sizeof(T), layout);
  if (sp.ok) {
    hipLaunchKernelGGL((dwconv_bwd_strip_kernel<T>), dim3((unsigned)sp.blocks), dim3(256), 0,
                       st, static_cast<const T*>(x), w, static_cast<const T*>(dy),
                       static_cast<T*>(dx), part, sp.rows, sp.cols, D, (long)gh * gw,
                       grid_map(gh, gw, layout, out_layout), sp.nslab, sp.nstrip, sp.nrg, sp.rh);
    hipLaunchKernelGGL(dwconv_dw_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       part, (int)((long)B * sp.nstrip * sp.nrg), D, dw, dbias);
    return hipGetLastError();
  }
  const TilePlan tp = tile_plan(B, gh, gw, D, sizeof(T), layout);
  if (tp.ok) {
    hipLaunchKernelGGL((dwconv_bwd_tiled_kernel<T>), dim3((unsigned)tp.conv_blocks), dim3(256), 0,
                       st, static_cast<const T*>(x), w, static_cast<const T*>(dy),
                       static_cast<T*>(dx), part, D, (long)gh * gw,
                       grid_map(gh, gw, layout, out_layout), tp.rows, tp.cols, tp.ntr, tp.ntc,
                       tp.nslab);
    hipLaunchKernelGGL(dwconv_dw_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       part, (int)((long)B * tp.ntr * tp.ntc), D, dw, dbias);
    return hipGetLastError();
  }
  const hipError_t e = launch_conv_t<T, true>(B, gh, gw, D, layout, out_layout, dy, w, nullptr,
                                              dx, st);
  if (e != hipSuccess) return e;
  return launch_dw_t<T>(B, gh, gw, D, layout, out_layout, x, dy, dw, dbias, part, st);
}

hipError_t launch_dwconv_bwd(int B, int gh, int gw, int D, int bf16v, int layout, int out_layout,
                             const void* x, const float* w, const void* dy, void* dx, float* dw,
                             float* dbias, void* workspace, hipStream_t st) {
  float* part = static_cast<float*>(workspace);
  if (bf16v)
    return launch_dwconv_bwd_t<bf16>(B, gh, gw, D, layout, out_layout, x, w, dy, dx, dw, dbias,
                                     part, st);
  return launch_dwconv_bwd_t<float>(B, gh, gw, D, layout, out_layout, x, w, dy, dx, dw, dbias,
                                    part, st);
}

// The allocation-free conv backward keeps its dW/dbias partials in this array, one copy per
// GPU for the life of the process.  Every call on a GPU shares that GPU's copy (calls that
// overlap on one GPU race); each call writes every partial it later reads, so nothing needs
// clearing between calls.  Host code never passes the array's name to a kernel: it passes the
// device address hipGetSymbolAddress gives for the current device.
__device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];
namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t noalloc_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_dwconv_bwd_noalloc(int B, int gh, int gw, int D, int bf16v, int layout,
                                     int out_layout, const void* x, const float* w, const void* dy,
                                     void* dx, float* dw, float* dbias, hipStream_t st) {
  if (dwconv_bwd_workspace(B, gh, gw, D) > kNoAllocScratchBytes) return hipErrorInvalidValue;
  float* part = nullptr;
  const hipError_t e = noalloc_scratch(&part);
  if (e != hipSuccess) return e;
  return launch_dwconv_bwd(B, gh, gw, D, bf16v, layout, out_layout, x, w, dy, dx, dw, dbias, part,
                           st);
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
