// dig_device.h -- device-side building blocks shared by the gfx950 kernels of libdig:
// element types, matrix-core (MFMA) tile products, wavefront scans and reductions,
// cooperative global->LDS tile staging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dig {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return static_cast<bf16>(x); }  // RNE

// logsigmoid(z) = min(z, 0) - log1p(exp(-|z|)), no overflow for any finite z.
__device__ __forceinline__ float logsigmoid_f(float z) {
  return fminf(z, 0.0f) - log1pf(expf(-fabsf(z)));
}
__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- matrix cores
// 16x16 output tile, fp32 accumulators.  Lane l holds rows 4*(l/16)+i (i<4), column l%16.
// A operand lane layout: row l%16, K-slice owned by lane group g = l/16; B likewise with
// columns.  Any K ordering works as long as A and B use the same one.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename T> struct Mma;

// Operand access: KC ("K-contiguous") means element (row, k) sits at base[row * ld + k];
// otherwise ("row-contiguous") at base[k * ld + row].  For an A operand the row is M, for a
// B operand it is N.  KC reads are single vector loads, the other form is strided.

// bf16: K step 32; lane group g owns k = 8g..8g+7 of each step.
template <> struct Mma<bf16> {
  static constexpr int KSTEP = 32;
  template <bool KC>
  __device__ static __forceinline__ bf16x8 frag(const bf16* base, int ld, int row, int k) {
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8*>(base + row * ld + k);
    } else {
      bf16x8 v;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = base[(k + i) * ld + row];
      return v;
    }
  }
  // acc += sum_{k<K} A(m0 + m, k) * B(k, n0 + n)
  template <bool AKC, bool BKC>
  __device__ static __forceinline__ f32x4 mm(f32x4 acc, const bf16* A, int lda, int m0,
                                             const bf16* B, int ldb, int n0, int K, int lane) {
    const int r = lane & 15, g8 = (lane >> 4) * 8;

    for (int k = 0; k < K; k += 32)
      acc = mfma_bf16(frag<AKC>(A, lda, m0 + r, k + g8), frag<BKC>(B, ldb, n0 + r, k + g8), acc);
    return acc;
  }
  __device__ static __forceinline__ f32x4 kc(f32x4 acc, const bf16* A, int lda, int m0,
                                             const bf16* B, int ldb, int n0, int K, int lane) {
    return mm<true, true>(acc, A, lda, m0, B, ldb, n0, K, lane);
  }
};

// fp32: K step 4; lane group g owns k = g of each step.
template <> struct Mma<float> {
  static constexpr int KSTEP = 4;
  template <bool AKC, bool BKC>
  __device__ static __forceinline__ f32x4 mm(f32x4 acc, const float* A, int lda, int m0,
                                             const float* B, int ldb, int n0, int K, int lane) {
    const int r = lane & 15, g = lane >> 4;

    for (int k = 0; k < K; k += 4) {
      const float a = AKC ? A[(m0 + r) * lda + k + g] : A[(k + g) * lda + m0 + r];
      const float b = BKC ? B[(n0 + r) * ldb + k + g] : B[(k + g) * ldb + n0 + r];
      acc = mfma_f32(a, b, acc);
    }
    return acc;
  }
  __device__ static __forceinline__ f32x4 kc(f32x4 acc, const float* A, int lda, int m0,
                                             const float* B, int ldb, int n0, int K, int lane) {
    return mm<true, true>(acc, A, lda, m0, B, ldb, n0, K, lane);
  }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ------------------------------------------------------------ wave primitives
// Inclusive prefix sum over groups of `width` consecutive lanes (width a power of 2 <= 64).
__device__ __forceinline__ float group_inclusive_scan(float x, int width, int lane_in_group) {
  for (int off = 1; off < width; off <<= 1) {
    float y = __shfl_up(x, off, width);
    if (lane_in_group >= off) x += y;
  }
  return x;
}

// Sum over the 16 lanes that share l/16 (the lanes holding one accumulator row set).
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

// Inclusive suffix sum over groups of `width` consecutive lanes: sum of lanes >= this one.
__device__ __forceinline__ float group_inclusive_suffix(float x, int width, int lane_in_group) {
  for (int off = 1; off < width; off <<= 1) {
    float y = __shfl_down(x, off, width);
    if (lane_in_group + off < width) x += y;
  }
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// ------------------------------------------------------------ tile staging
// Copy rows [0, rows) of a token-major tile (row r at gsrc + r*gstride elements, `cols`
// elements each) into LDS dst (row pitch ld elements).  Rows >= valid are zero-filled.
// Vector width is the largest of 16/8/4/2 bytes dividing cols*sizeof(T) (rows start on that
// alignment because the base is 16-byte aligned and the stride is a multiple of cols).
template <typename T>
__device__ __forceinline__ void stage_rows(T* dst, int ld, const T* gsrc, long gstride,
                                           int rows, int valid, int cols, int tid, int nthr) {
  const int rowbytes = cols * (int)sizeof(T);
  if ((rowbytes & 15) == 0 && ((ld * (int)sizeof(T)) & 15) == 0) {
    const int nv = rowbytes >> 4;
    for (int i = tid; i < rows * nv; i += nthr) {
      int r = i / nv, c = i - r * nv;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (r < valid) val = reinterpret_cast<const uint4*>(gsrc + (long)r * gstride)[c];
      reinterpret_cast<uint4*>(dst + r * ld)[c] = val;
    }
  } else if ((rowbytes & 7) == 0 && ((ld * (int)sizeof(T)) & 7) == 0) {
    const int nv = rowbytes >> 3;
    for (int i = tid; i < rows * nv; i += nthr) {
      int r = i / nv, c = i - r * nv;
      uint2 val = make_uint2(0, 0);
      if (r < valid) val = reinterpret_cast<const uint2*>(gsrc + (long)r * gstride)[c];
      reinterpret_cast<uint2*>(dst + r * ld)[c] = val;
    }
  } else {
    for (int i = tid; i < rows * cols; i += nthr) {
      int r = i / cols, c = i - r * cols;
      T val = from_f<T>(0.f);
      if (r < valid) val = gsrc[(long)r * gstride + c];
      dst[r * ld + c] = val;
    }
  }
}

// Store rows [0, valid) of an LDS tile (pitch ld) to a token-major global tile.
template <typename T>
__device__ __forceinline__ void store_rows(T* gdst, long gstride, const T* src, int ld,
                                           int valid, int cols, int tid, int nthr) {
  const int rowbytes = cols * (int)sizeof(T);
  if ((rowbytes & 15) == 0 && ((ld * (int)sizeof(T)) & 15) == 0) {
    const int nv = rowbytes >> 4;
    for (int i = tid; i < valid * nv; i += nthr) {
      int r = i / nv, c = i - r * nv;
      reinterpret_cast<uint4*>(gdst + (long)r * gstride)[c] =
          reinterpret_cast<const uint4*>(src + r * ld)[c];
    }
  } else if ((rowbytes & 7) == 0 && ((ld * (int)sizeof(T)) & 7) == 0) {
    const int nv = rowbytes >> 3;
    for (int i = tid; i < valid * nv; i += nthr) {
      int r = i / nv, c = i - r * nv;
      reinterpret_cast<uint2*>(gdst + (long)r * gstride)[c] =
          reinterpret_cast<const uint2*>(src + r * ld)[c];
    }
  } else {
    for (int i = tid; i < valid * cols; i += nthr) {
      int r = i / cols, c = i - r * cols;
      gdst[(long)r * gstride + c] = src[r * ld + c];
    }
  }
}

__device__ __forceinline__ int round_up(int x, int m) { return (x + m - 1) / m * m; }

}  // namespace dig
