// probe.hip -- measurement kernels for bench.py, built into libdig_probe.so (not part of the
// library's ABI and never called by it):
//
//   digp_contraction  the chunk kernel's contraction phases with every operand resident in
//                     LDS and no global traffic: per chunk and head, the gated Q K^T from split
//                     hi/lo operands (row tile I against key tiles J <= I), P V from the P
//                     accumulators, (q e^b) S0, and the state update S <- diag(g) S + Kbar^T V,
//                     with the forward kernel's wave roles and the same device helpers.  It
//                     isolates how busy these phases can keep the matrix cores (the chunk form
//                     of the write-up's section 3 "Efficiency Analysis": chunks computed on
//                     chip) from the memory traffic around them.
//   digp_copy         a streaming device copy (16-byte vectors, eight in flight per thread):
//                     the HBM ceiling a read-once/write-once kernel can reach.
//   digp_copy_w       the same copy with 4-, 8- or 16-byte lanes: how the byte counters read
//                     for each access width.
//   digp_head_slices  one workgroup per (head, segment) reading that head's slice of every
//                     token row of the segment, in three workgroup orders: whether the heads
//                     that share 128-byte lines meet in one XCD's L2.
//   digp_mfma_rate    bf16 MFMA instructions with operands and accumulators in registers only
//                     (independent accumulators, no memory): the rate each instruction shape
//                     can sustain, the ceiling under the contraction microbenchmark.
#include <hip/hip_runtime.h>

#include "dig_device.h"

namespace dig {
namespace {

// Head shapes: S (d_k 32, d_v 64, eight waves: four query-row waves, four state waves) and
// XL (d_k 36, d_v 72, four waves, each a query-row wave and a state wave).  Chunk 64.
template <int DK, int DV, int NW>
struct ProbeShape {
  static constexpr int C = 64, NT = C / 16;
  static constexpr int NDK = (DK + 15) / 16, NDV = (DV + 15) / 16;
  static constexpr int DKP = ((NDK * 16 + 31) / 32) * 32, DVP = NDV * 16;
  static constexpr int QKC = (DK + 3) / 4 * 4, QKP = QKC % 32 == 0 ? QKC + 4 : QKC;
  static constexpr int QP = DKP + 8, TP = C + 8;
  static constexpr int SW0 = NW > NT ? NT : 0, NSW = NW - SW0;
  static constexpr int NST = NDK * NDV, STW = (NST + NSW - 1) / NSW;
  static constexpr int O_Q = 0, O_K = O_Q + C * QKP * 4, O_KBT = O_K + C * QKP * 4;
  static constexpr int O_VT = O_KBT + 16 * NDK * TP * 2, O_S = O_VT + DVP * TP * 2;
  static constexpr int bytes = O_S + DVP * QP * 2;
  // MFMA instructions per chunk (one workgroup iteration), as issued below
  static constexpr long mfma_per_chunk() {
    long n = 0;
    const long qk = QKC == 36 ? 4 : 3 * ((QKC + 31) / 32);  // split Q K^T per tile
    const long s0 = QKC == 36 ? 1 + 2 : 2 * ((QKC + 31) / 32);  // split (q e^b) S0 per tile
    for (int I = 0; I < NT; ++I) n += (I + 1) * qk + (I / 2 + 1) * NDV + NDV * s0;
    n += (long)NST * (C / 32);  // state update
    return n;
  }
};

template <int DK, int DV, int NW>
__global__ __launch_bounds__(64 * NW) void contraction_kernel(int iters, float* sink) {
  using Sh = ProbeShape<DK, DV, NW>;
  constexpr int C = Sh::C, NT = Sh::NT, NDV = Sh::NDV, NDK = Sh::NDK, QKC = Sh::QKC;
  constexpr int QKP = Sh::QKP, QP = Sh::QP, TP = Sh::TP, SW0 = Sh::SW0, NSW = Sh::NSW;
  constexpr int NST = Sh::NST, STW = Sh::STW;
  extern __shared__ __align__(16) unsigned char smem[];
  float* sQ = reinterpret_cast<float*>(smem + Sh::O_Q);
  float* sK = reinterpret_cast<float*>(smem + Sh::O_K);
  bf16* sKbT = reinterpret_cast<bf16*>(smem + Sh::O_KBT);
  bf16* sVt = reinterpret_cast<bf16*>(smem + Sh::O_VT);
  bf16* sS = reinterpret_cast<bf16*>(smem + Sh::O_S);
  const int tid = threadIdx.x, wave = tid >> 6;
  // operands: small deterministic values (the timing does not depend on them)
  for (int i = tid; i < Sh::bytes / 4; i += 64 * NW) {
    const float v = 0.001f * (float)((i * 37 + blockIdx.x) % 97) - 0.048f;
    if (i < Sh::O_KBT / 4) reinterpret_cast<float*>(smem)[i] = v;
    else {
      reinterpret_cast<bf16*>(smem)[2 * i] = from_f<bf16>(v);
      reinterpret_cast<bf16*>(smem)[2 * i + 1] = from_f<bf16>(-v);
    }
  }
  __syncthreads();
  f32x4 oacc[NDV], sacc[STW];
#pragma unroll
  for (int E = 0; E < NDV; ++E) oacc[E] = zero4();
#pragma unroll
  for (int m = 0; m < STW; ++m) sacc[m] = zero4();
  for (int it = 0; it < iters; ++it) {
    // lane-derived LDS addresses are opaque per iteration (as in the chunk kernels), so the
    // operand reads and splits are not hoisted out of the loop
    const int lane = opaque(tid & 63);
    const int r16 = lane & 15, g4 = lane >> 4;
    // state update
#pragma unroll
    for (int m = 0; m < STW; ++m) {
      const int u = wave - SW0 + NSW * m;
      if (wave >= SW0 && u < NST) {
        const int ct = u / NDV, et = u - ct * NDV;
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[m][i] *= 0.999f;
        sacc[m] = Mma<bf16>::kc(sacc[m], sKbT, TP, 16 * ct, sVt, TP, 16 * et, C, lane);
      }
    }
    if (wave < NT) {
      const int I = wave;
      f32x4 pt[NT];
      const auto bq = split_b<QKC, QKP>(sQ, 16 * I, lane);
#pragma unroll
      for (int J = 0; J < NT; ++J)
        pt[J] = J <= I ? mm_split_pre<QKC, QKP, QKP>(zero4(), sK, 16 * J, bq, lane) : zero4();
#pragma unroll
      for (int E = 0; E < NDV; ++E)
        oacc[E] = mm_split_b<QKC, QKP, QP>(oacc[E], sQ, 16 * I, sS, 16 * E, lane);
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
            const bf16* vb = sVt + (E * 16 + r16) * TP + 32 * pp + 4 * g4;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vb);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vb + 16);
            bf16x8 bv;
#pragma unroll
            for (int i = 0; i < 4; ++i) { bv[i] = lo[i]; bv[4 + i] = hi[i]; }
            oacc[E] = mfma_bf16(a, bv, oacc[E]);
          }
        }
      }
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int E = 0; E < NDV; ++E) acc += oacc[E][0] + oacc[E][1] + oacc[E][2] + oacc[E][3];
#pragma unroll
  for (int m = 0; m < STW; ++m) acc += sacc[m][0] + sacc[m][1] + sacc[m][2] + sacc[m][3];
  sink[(long)blockIdx.x * 64 * NW + tid] = acc;
}

template <int DK, int DV, int NW>
hipError_t launch_contraction(int nwg, int iters, float* sink, hipStream_t st) {
  using Sh = ProbeShape<DK, DV, NW>;
  hipLaunchKernelGGL((contraction_kernel<DK, DV, NW>), dim3(nwg), dim3(64 * NW), Sh::bytes, st,
                     iters, sink);
  return hipGetLastError();
}

// Register-only MFMA rate: NACC independent accumulators per wave, `iters` rounds.
template <bool WIDE, int NACC>
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = from_f<bf16>(0.001f * (float)(threadIdx.x + i));
    b[i] = from_f<bf16>(0.002f * (float)i);
  }
  float s = 0.f;
  if constexpr (WIDE) {
    f32x16 c[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) c[j][v] = 0.f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NACC; ++j) c[j] = mfma32_bf16(a, b, c[j]);
#pragma unroll
    for (int j = 0; j < NACC; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += c[j][v];
  } else {
    f32x4 c[NACC];
#pragma unroll
    for (int j = 0; j < NACC; ++j) c[j] = zero4();
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < NACC; ++j) c[j] = mfma_bf16(a, b, c[j]);
#pragma unroll
    for (int j = 0; j < NACC; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  }
  sink[(long)blockIdx.x * 256 + threadIdx.x] = s;
}

// Streaming copy: every thread moves 8 16-byte vectors per step, all loads before the stores.
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, long n) {
  constexpr int U = 8;
  const long stride = (long)gridDim.x * 256 * U;
  for (long base = (long)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[min(base + 256L * u, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + 256L * u < n) dst[base + 256L * u] = v[u];
  }
}

// The same with narrower lanes (V = uint2: 8 bytes, uint32_t: 4 bytes per lane and access).
template <typename V>
__global__ __launch_bounds__(256) void copy_kernel_w(const V* __restrict__ src,
                                                     V* __restrict__ dst, long n) {
  constexpr int U = 8;
  const long stride = (long)gridDim.x * 256 * U;
  for (long base = (long)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[min(base + 256L * u, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + 256L * u < n) dst[base + 256L * u] = v[u];
  }
}

// Reads one head's d-element slice of every token row of a segment ([rows][H][d] bf16, the
// mixer's layout), one workgroup per (head, segment), and writes one sum per workgroup.  order
// 0: workgroup = head * nseg + segment (the chunk kernels' order); 1: segment * H + head;
// 2: order 0 with the segment's rows walked from a per-head offset (heads out of step).
__global__ __launch_bounds__(256) void head_slice_kernel(const unsigned* __restrict__ src,
                                                         float* __restrict__ out, int rows, int H,
                                                         int d, int nseg, int order) {
  const int blk = blockIdx.x;
  const int h = order == 1 ? blk % H : blk / nseg;
  const int seg = order == 1 ? blk / H : blk % nseg;
  const int rps = rows / nseg, pairs = d / 2;
  const int n = rps * pairs;
  float acc = 0.f;
  for (int i0 = 0; i0 < n; i0 += 256 * 4) {
    unsigned v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(i0 + 256 * u + (int)threadIdx.x, n - 1);
      int t = i / pairs;
      const int c = i - t * pairs;
      if (order == 2) t = (t + h * (rps / H)) % rps;
      v[u] = src[((long)(seg * rps + t) * H + h) * pairs + c];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += __uint_as_float(v[u] << 16);
  }
  out[(long)blk * 256 + threadIdx.x] = acc;
}

}  // namespace
}  // namespace dig

extern "C" {

// shape 0: d_k 32, d_v 64, eight waves; shape 1: d_k 36, d_v 72, four waves.  sink holds
// nwg * (64 * waves) floats.  Returns 0 or a hipError_t.
int digp_contraction(int shape, int nwg, int iters, float* sink, hipStream_t st) {
  if (nwg < 1 || iters < 1 || !sink) return (int)hipErrorInvalidValue;
  if (shape == 0) return (int)dig::launch_contraction<32, 64, 8>(nwg, iters, sink, st);
  if (shape == 1) return (int)dig::launch_contraction<36, 72, 4>(nwg, iters, sink, st);
  return (int)hipErrorInvalidValue;
}

int digp_contraction_waves(int shape) { return shape == 0 ? 8 : 4; }

// Flops of one chunk (one workgroup iteration): the algorithmic count of the chunk form,
// 2 [C (C+1)/2 (d_k + d_v) + 2 C d_k d_v] (causal gated Q K^T and P V, (q e^b) S0 and the
// state update), and the bf16 MFMA flops issued (16 x 16 x 32 x 2 per instruction).
void digp_contraction_flops(int shape, double* algorithmic, double* issued) {
  const double C = 64, dk = shape == 0 ? 32 : 36, dv = shape == 0 ? 64 : 72;
  *algorithmic = 2.0 * (C * (C + 1) / 2 * (dk + dv) + 2 * C * dk * dv);
  const long n = shape == 0 ? dig::ProbeShape<32, 64, 8>::mfma_per_chunk()
                            : dig::ProbeShape<36, 72, 4>::mfma_per_chunk();
  *issued = (double)n * 16 * 16 * 32 * 2;
}

// wide 0: 16x16x32 (16 384 flops per instruction), 1: 32x32x16 (32 768); nwg workgroups of four
// waves, iters rounds of 4 (2) independent instructions per wave; sink holds nwg * 256 floats.
int digp_mfma_rate(int wide, int nwg, int iters, float* sink, hipStream_t st) {
  if (nwg < 1 || iters < 1 || !sink) return (int)hipErrorInvalidValue;
  if (wide) hipLaunchKernelGGL((dig::mfma_rate_kernel<true, 4>), dim3(nwg), dim3(256), 0, st, sink, iters);
  else hipLaunchKernelGGL((dig::mfma_rate_kernel<false, 8>), dim3(nwg), dim3(256), 0, st, sink, iters);
  return (int)hipGetLastError();
}
double digp_mfma_rate_flops(int wide, int nwg, int iters) {
  return wide ? 4.0 * 32768 * 4 * iters * nwg : 8.0 * 16384 * 4 * iters * nwg;
}

// A streaming copy with `width`-byte lanes (4, 8 or 16): how the HBM byte counters read for
// accesses of each width.
int digp_copy_w(const void* src, void* dst, size_t bytes, int width, hipStream_t st) {
  if (!src || !dst || (width != 4 && width != 8 && width != 16) || bytes % 16)
    return (int)hipErrorInvalidValue;
  const long n = (long)(bytes / width);
  long g = (n + 256 * 8 - 1) / (256 * 8);
  if (g > 256 * 8) g = 256 * 8;
  if (g < 1) g = 1;
  if (width == 16)
    hipLaunchKernelGGL(dig::copy_kernel, dim3((unsigned)g), dim3(256), 0, st,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  else if (width == 8)
    hipLaunchKernelGGL(dig::copy_kernel_w<uint2>, dim3((unsigned)g), dim3(256), 0, st,
                       static_cast<const uint2*>(src), static_cast<uint2*>(dst), n);
  else
    hipLaunchKernelGGL(dig::copy_kernel_w<uint32_t>, dim3((unsigned)g), dim3(256), 0, st,
                       static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), n);
  return (int)hipGetLastError();
}

// src: rows * H * d bf16 (d even); out: H * nseg * 256 floats.
int digp_head_slices(const void* src, float* out, int rows, int H, int d, int nseg, int order,
                     hipStream_t st) {
  if (!src || !out || d % 2 || rows % nseg || order < 0 || order > 2)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(dig::head_slice_kernel, dim3((unsigned)(H * nseg)), dim3(256), 0, st,
                     static_cast<const unsigned*>(src), out, rows, H, d, nseg, order);
  return (int)hipGetLastError();
}

int digp_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  if (!src || !dst || bytes % 16) return (int)hipErrorInvalidValue;
  const long n = (long)(bytes / 16);
  long g = (n + 256 * 8 - 1) / (256 * 8);
  if (g > 256 * 8) g = 256 * 8;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(dig::copy_kernel, dim3((unsigned)g), dim3(256), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return (int)hipGetLastError();
}

}  // extern "C"
