// dig_device.h -- device-side building blocks shared by the gfx950 kernels of libdig:
// element types, matrix-core (MFMA) tile products, wavefront scans and reductions,
// cooperative global->LDS tile staging.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dig_internal.h"

namespace dig {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Workgroup i of n runs on XCD i mod 8; returns the work item it takes when XCD x takes the
// x-th contiguous run of items (n / 8 items, one more for the first n mod 8 XCDs).
__device__ __forceinline__ int xcd_item(int i, int n) {
  const int q = n >> 3, r = n & 7, x = i & 7, k = i >> 3;
  return x * q + min(x, r) + k;
}

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return static_cast<bf16>(x); }  // RNE

// Hardware transcendental units (about 1 ulp): 2^x, log2(x), 1/x.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }

// log2(sigmoid(z)) = min(z, 0) log2(e) - log2(1 + 2^(-|z| log2(e))): no overflow for any z.
__device__ __forceinline__ float log2_sigmoid(float z) {
  return fminf(z, 0.f) * 1.4426950408889634f - flog2(1.f + fexp2(-fabsf(z) * 1.4426950408889634f));
}
__device__ __forceinline__ float fast_sigmoid(float z) {
  return frcp(1.f + fexp2(-z * 1.4426950408889634f));
}

// Element-type-specific math: bf16 I/O uses the hardware units above; fp32 I/O keeps the
// correctly rounded library forms so that its tighter accuracy holds on ill-conditioned rows.
template <typename T> struct Fm;
template <> struct Fm<bf16> {
  __device__ static __forceinline__ float exp2(float x) { return fexp2(x); }
  __device__ static __forceinline__ float lsig2(float z) { return log2_sigmoid(z); }
  __device__ static __forceinline__ float sig(float z) { return fast_sigmoid(z); }
};
template <> struct Fm<float> {
  __device__ static __forceinline__ float exp2(float x) { return exp2f(x); }
  __device__ static __forceinline__ float lsig2(float z) {
    return (fminf(z, 0.f) - log1pf(expf(-fabsf(z)))) * 1.4426950408889634f;
  }
  __device__ static __forceinline__ float sig(float z) { return 1.f / (1.f + expf(-z)); }
};

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
// 32 x 32 output tile, K step 16: lane l holds rows 8 (v / 4) + 4 (l / 32) + v % 4 (v < 16),
// column l % 32; A operand row l % 32, K slice 8 (l / 32)..+7, B likewise with columns.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}


template <typename T> struct Mma;

// Operand access: KC ("K-contiguous") means element (row, k) sits at base[row * ld + k];
// otherwise ("row-contiguous") at base[k * ld + row].  For an A operand the row is M, for a
// B operand it is N.  KC reads are single vector loads, the other form is strided.

// K-major tiles (element (row, k) at base[k * ld + row]) reach the MFMA lane layout through
// the gfx950 LDS transpose load: in each 16-lane group, lane L reads the four elements of
// K row k0 + L/4 at rows m0 + 4 (L % 4) .. +3 (8 bytes), and the load hands lane j the four
// K rows k0 .. k0+3 of row m0 + j.  The group reads exactly the 16 x 4 elements the lanes
// need (no other LDS address); ld and m0 are multiples of 4 and the base 8-byte aligned, so
// every 8-byte read is aligned.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* base, int ld, int m0, int k0, int r) {
  const bf16* p = base + (k0 + (r >> 2)) * ld + m0 + 4 * (r & 3);
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// bf16: K step 32; lane group g owns k = 8g..8g+7 of each step.
template <> struct Mma<bf16> {
  static constexpr int KSTEP = 32;
  // fragment of rows m0 + r (r = lane % 16), K slice k..k+7 (KC: K-contiguous rows; else a
  // K-major tile read through the transpose load)
  template <bool KC>
  __device__ static __forceinline__ bf16x8 frag(const bf16* base, int ld, int m0, int r, int k) {
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8*>(base + (m0 + r) * ld + k);
    } else {
      const bf16x4 lo = lds_tr4(base, ld, m0, k, r), hi = lds_tr4(base, ld, m0, k + 4, r);
      bf16x8 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = lo[i]; v[4 + i] = hi[i]; }
      return v;
    }
  }
  template <bool KC>
  __device__ static __forceinline__ bf16x4 frag4(const bf16* base, int ld, int m0, int r, int k) {
    if constexpr (KC) return *reinterpret_cast<const bf16x4*>(base + (m0 + r) * ld + k);
    else return lds_tr4(base, ld, m0, k, r);
  }
  template <bool KC>
  __device__ static __forceinline__ bf16x8 frag(const bf16* base, int ld, int row, int k) {
    static_assert(KC, "K-major fragments take the tile's first row");
    return *reinterpret_cast<const bf16x8*>(base + row * ld + k);
  }
  // acc += sum_{k<K} A(m0 + m, k) * B(k, n0 + n); K a multiple of 16 (a final 16 runs as a
  // 16x16x32 step with half of each lane's slots zero)
  template <bool AKC, bool BKC>
  __device__ static __forceinline__ f32x4 mm(f32x4 acc, const bf16* A, int lda, int m0,
                                             const bf16* B, int ldb, int n0, int K, int lane) {
    const int r = lane & 15, g = lane >> 4;
    int k = 0;
    for (; k + 32 <= K; k += 32)
      acc = mfma_bf16(frag<AKC>(A, lda, m0, r, k + 8 * g), frag<BKC>(B, ldb, n0, r, k + 8 * g),
                      acc);
    if (k < K) {  // K tail of 16: each lane group's 4 live k in slots 0-3, zeros in 4-7
      const bf16x4 a4 = frag4<AKC>(A, lda, m0, r, k + 4 * g);
      const bf16x4 b4 = frag4<BKC>(B, ldb, n0, r, k + 4 * g);
      bf16x8 a, b;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = a4[i];
        b[i] = b4[i];
        a[4 + i] = from_f<bf16>(0.f);
        b[4 + i] = from_f<bf16>(0.f);
      }
      acc = mfma_bf16(a, b, acc);
    }
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

// ------------------------------------------------------------ low-rank key gate
// The key gate's logits as a rank-16 product formed inside the chunk kernels: for token t and
// key column c of head h, z = bias[h d_k + c] + sum_r f[t][r] W[h d_k + c][r], with the factor
// f (16 bf16 per token) staged with the chunk's rows and the head's slice of W (bf16, out x in)
// and bias (fp32) copied once per workgroup into an LDS table: NCOLS rows of 16 bf16 (32 bytes,
// zero past d_k), then NCOLS fp32 biases.  Sums run as eight bf16 pair dot products into an
// fp32 accumulator started at the bias, in the same order in every kernel, so the forward and
// the backward see identical logits.
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int lowrank_table_bytes(int ncols) { return ncols * (kGateRank * 2 + 4); }
template <int NCOLS, int NTH>
__device__ __forceinline__ void lowrank_table_fill(unsigned char* tab, const bf16* w,
                                                   const float* bias, int h, int dk, int tid) {
  // rows of W are 32 bytes: eight 4-byte pieces each (W needs only 4-byte alignment)
  const unsigned* wsrc = reinterpret_cast<const unsigned*>(w + (long)h * dk * kGateRank);
  unsigned* wdst = reinterpret_cast<unsigned*>(tab);
  for (int i = tid; i < NCOLS * 8; i += NTH) wdst[i] = i < dk * 8 ? wsrc[i] : 0u;
  float* bdst = reinterpret_cast<float*>(tab + NCOLS * kGateRank * 2);
  for (int c = tid; c < NCOLS; c += NTH) bdst[c] = (c < dk && bias) ? bias[(long)h * dk + c] : 0.f;
}
// Logits of one token for the N key columns c0..c0+N-1 (frow: the token's 16 factor values in
// LDS, 16-byte aligned).
template <int NCOLS, int N>
__device__ __forceinline__ void lowrank_logits(float (&z)[N], const bf16* frow,
                                               const unsigned char* tab, int c0) {
  const uint4 f0 = *reinterpret_cast<const uint4*>(frow);
  const uint4 f1 = *reinterpret_cast<const uint4*>(frow + 8);
  const unsigned fp[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
  const float* btab = reinterpret_cast<const float*>(tab + NCOLS * kGateRank * 2);
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const uint4* wr = reinterpret_cast<const uint4*>(tab + (c0 + j) * kGateRank * 2);
    const uint4 w0 = wr[0], w1 = wr[1];
    const unsigned wp[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float acc = btab[c0 + j];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, fp[i]),
                                            __builtin_bit_cast(bf16x2, wp[i]), acc, false);
    z[j] = acc;
    if (j % 2 == 1) __builtin_amdgcn_sched_barrier(0);  // two columns' table reads in flight
  }
}

// ------------------------------------------------- split-precision operands on bf16 MFMA
// An fp32 operand x is carried as x_hi + x_lo, x_hi = bf16(x), x_lo = bf16(x - x_hi) (the
// difference is exact in fp32).  The pair holds about 16 significant bits, so a product
// accumulated as A_hi B_hi + A_hi B_lo + A_lo B_hi on the bf16 matrix cores is accurate to
// about 2^-16 of each term (the dropped A_lo B_lo is below that), against 2^-8 with one bf16
// rounding per operand.
struct SplitFrag {
  bf16x8 hi, lo;
};

// Split fragment of row `row`, columns k..k+7 (k a multiple of 8) of a K-contiguous fp32 tile
// with COLS stored columns (a multiple of 4) at pitch LD floats (a multiple of 4).  Columns at
// or past COLS read as zero; FULL asserts that k + 8 <= COLS for every lane.  Both 16-byte
// reads are always issued (from a clamped address where masked): no branch around them.
template <int COLS, int LD, bool FULL>
__device__ __forceinline__ SplitFrag split_frag(const float* base, int row, int k) {
  static_assert(COLS % 4 == 0 && LD % 4 == 0 && COLS <= LD, "fp32 tile layout");
  float x[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = k + 4 * h;
    const bool in = FULL || c + 4 <= COLS;
    const float4 v = *reinterpret_cast<const float4*>(base + row * LD + (in ? c : COLS - 4));
    x[4 * h + 0] = in ? v.x : 0.f;
    x[4 * h + 1] = in ? v.y : 0.f;
    x[4 * h + 2] = in ? v.z : 0.f;
    x[4 * h + 3] = in ? v.w : 0.f;
  }
  SplitFrag f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bf16 hi = from_f<bf16>(x[i]);
    f.hi[i] = hi;
    f.lo[i] = from_f<bf16>(x[i] - to_f(hi));
  }
  return f;
}

// acc += A B over one 32-wide K step from split operands (lo products first).
__device__ __forceinline__ f32x4 mfma_split(const SplitFrag& a, const SplitFrag& b, f32x4 acc) {
  acc = mfma_bf16(a.lo, b.hi, acc);
  acc = mfma_bf16(a.hi, b.lo, acc);
  return mfma_bf16(a.hi, b.hi, acc);
}

// A four-column K tail (columns 32..35) packed into one 32-wide step: the three products
// hi.hi, hi.lo and lo.hi of the four columns take 12 of the step's 32 slots.  Lane group 0
// holds A = [hi, hi], B = [hi, lo]; lane group 1 A = [lo, 0], B = [hi, 0]; the others zero.
// TAIL_B selects the B role.  (The element index inside a lane's eight slots is the K index
// within its group, so A and B only have to agree slot by slot.)
template <int LD, bool TAIL_B>
__device__ __forceinline__ bf16x8 tail4_frag(const float* base, int row, int g) {
  const float4 v = *reinterpret_cast<const float4*>(base + row * LD + 32);
  const float x[4] = {v.x, v.y, v.z, v.w};
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16 hi = from_f<bf16>(x[i]);
    const bf16 lo = from_f<bf16>(x[i] - to_f(hi));
    const bf16 z = from_f<bf16>(0.f);
    f[i] = g == 0 ? hi : (g == 1 ? (TAIL_B ? hi : lo) : z);
    f[4 + i] = g == 0 ? (TAIL_B ? lo : hi) : z;
  }
  return f;
}

// acc(m, n) += sum_k A(m0 + m, k) B(n0 + n, k) over the COLS stored columns of two K-contiguous
// fp32 tiles (pitches LDA, LDB floats), both split into hi + lo bf16 parts.
template <int COLS, int LDA, int LDB>
__device__ __forceinline__ f32x4 mm_split(f32x4 acc, const float* A, int m0, const float* B,
                                          int n0, int lane) {
  static_assert(COLS <= 64, "two K steps");
  const int r = lane & 15, g = lane >> 4;
  if constexpr (COLS == 36) {  // 32 columns split, then the packed four-column tail
    acc = mfma_bf16(tail4_frag<LDA, false>(A, m0 + r, g), tail4_frag<LDB, true>(B, n0 + r, g), acc);
    return mfma_split(split_frag<COLS, LDA, true>(A, m0 + r, 8 * g),
                      split_frag<COLS, LDB, true>(B, n0 + r, 8 * g), acc);
  }
  acc = mfma_split(split_frag<COLS, LDA, (32 <= COLS)>(A, m0 + r, 8 * g),
                   split_frag<COLS, LDB, (32 <= COLS)>(B, n0 + r, 8 * g), acc);
  if constexpr (COLS > 32)
    acc = mfma_split(split_frag<COLS, LDA, (64 <= COLS)>(A, m0 + r, 32 + 8 * g),
                     split_frag<COLS, LDB, (64 <= COLS)>(B, n0 + r, 32 + 8 * g), acc);
  return acc;
}

// The B side of mm_split for one 16-row tile, split once and reused against several A tiles
// (the same operations and order as mm_split: identical results).
template <int COLS, int LD>
struct SplitB {
  static constexpr int NS = COLS == 36 ? 1 : (COLS + 31) / 32;
  SplitFrag s[NS];
  bf16x8 tail;  // COLS == 36: the packed four-column tail
};
template <int COLS, int LD>
__device__ __forceinline__ SplitB<COLS, LD> split_b(const float* B, int n0, int lane) {
  static_assert(COLS <= 64, "two K steps");
  const int r = lane & 15, g = lane >> 4;
  SplitB<COLS, LD> b;
  if constexpr (COLS == 36) {
    b.tail = tail4_frag<LD, true>(B, n0 + r, g);
    b.s[0] = split_frag<COLS, LD, true>(B, n0 + r, 8 * g);
  } else {
    b.s[0] = split_frag<COLS, LD, (32 <= COLS)>(B, n0 + r, 8 * g);
    if constexpr (COLS > 32) b.s[1] = split_frag<COLS, LD, (64 <= COLS)>(B, n0 + r, 32 + 8 * g);
  }
  return b;
}
template <int COLS, int LDA, int LDB>
__device__ __forceinline__ f32x4 mm_split_pre(f32x4 acc, const float* A, int m0,
                                              const SplitB<COLS, LDB>& b, int lane) {
  const int r = lane & 15, g = lane >> 4;
  if constexpr (COLS == 36) {
    acc = mfma_bf16(tail4_frag<LDA, false>(A, m0 + r, g), b.tail, acc);
    return mfma_split(split_frag<COLS, LDA, true>(A, m0 + r, 8 * g), b.s[0], acc);
  }
  acc = mfma_split(split_frag<COLS, LDA, (32 <= COLS)>(A, m0 + r, 8 * g), b.s[0], acc);
  if constexpr (COLS > 32)
    acc = mfma_split(split_frag<COLS, LDA, (64 <= COLS)>(A, m0 + r, 32 + 8 * g), b.s[1], acc);
  return acc;
}

// The same with a bf16 K-contiguous B tile (pitch LDB elements): A enters as hi + lo parts, B as
// stored.  A lane group whose first column lies past COLS takes B as zero (its A part is zero);
// one whose first column lies inside reads eight B columns, so rows of B must hold
// (COLS + 7) / 8 * 8 readable, finite columns.
template <int COLS, int LDA, int LDB>
__device__ __forceinline__ f32x4 mm_split_b(f32x4 acc, const float* A, int m0, const bf16* B,
                                            int n0, int lane) {
  static_assert(COLS <= 64 && (COLS + 7) / 8 * 8 <= LDB, "bf16 operand rows");
  const int r = lane & 15, g = lane >> 4;
  if constexpr (COLS == 36) {  // packed four-column tail: lane group 0 A = [hi, lo], B = [b, b]
    const float4 v = *reinterpret_cast<const float4*>(A + (m0 + r) * LDA + 32);
    const float x[4] = {v.x, v.y, v.z, v.w};
    const bf16x4 b4 = *reinterpret_cast<const bf16x4*>(B + (n0 + r) * LDB + 32);
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16 hi = from_f<bf16>(x[i]), z = from_f<bf16>(0.f);
      a[i] = g == 0 ? hi : z;
      a[4 + i] = g == 0 ? from_f<bf16>(x[i] - to_f(hi)) : z;
      b[i] = g == 0 ? b4[i] : z;
      b[4 + i] = g == 0 ? b4[i] : z;
    }
    acc = mfma_bf16(a, b, acc);
  }
#pragma unroll
  for (int s = 0; s < (COLS == 36 ? 1 : (COLS + 31) / 32); ++s) {
    const int k = 32 * s + 8 * g;
    const bool in = k < COLS;
    bf16x8 b = *reinterpret_cast<const bf16x8*>(B + (n0 + r) * LDB + (in ? k : 0));
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = in ? b[i] : from_f<bf16>(0.f);
    const SplitFrag a = s == 0 ? split_frag<COLS, LDA, (32 <= COLS)>(A, m0 + r, k)
                               : split_frag<COLS, LDA, (64 <= COLS)>(A, m0 + r, k);
    acc = mfma_bf16(a.lo, b, acc);
    acc = mfma_bf16(a.hi, b, acc);
  }
  return acc;
}

// The same value, opaque to the optimiser (an empty asm statement that claims to modify the
// register; no instruction is emitted).  Deriving a loop body's lane-dependent LDS addresses
// from it keeps them from being hoisted out of the loop, where hundreds of them would stay
// live across every phase and spill.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The value computed here: it feeds an empty asm statement with side effects, which nothing
// moves across, so its computation cannot sink past later loads and branches (where its
// inputs would stay live across them).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// x where `on`, else +0, through a mask the optimiser cannot see (a select of an expensive
// operand, such as a logarithm, is otherwise turned into a branch around its computation,
// one per column, which also holds that computation's inputs live across the branches).
__device__ __forceinline__ float keep_if(bool on, float x) {
  const unsigned m = (unsigned)opaque(on ? -1 : 0);
  return __builtin_bit_cast(float, __builtin_bit_cast(unsigned, x) & m);
}

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

// Four elements moved as one vector: a lane's four rows of one 16 x 16 MFMA result tile.
template <typename T>
struct alignas(4 * sizeof(T)) Quad {
  T v[4];
};

// ---------------------------------------------------- DPP (register-only) lane ops
// gfx9 data-parallel primitives: row_shr:k = 0x110+k, row_ror:k = 0x120+k, row_bcast:15 =
// 0x142, row_bcast:31 = 0x143 (a "row" is 16 lanes).  Lanes whose source is outside the row,
// or whose row is masked off, read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}

// Inclusive prefix sum over groups of W consecutive lanes (W = 16, 32 or 64).
template <int W>
__device__ __forceinline__ float scan_dpp(float x) {
  static_assert(W == 16 || W == 32 || W == 64, "scan width");
  x += dpp_f<0x111>(x);
  x += dpp_f<0x112>(x);
  x += dpp_f<0x114>(x);
  x += dpp_f<0x118>(x);
  if constexpr (W >= 32) x += dpp_f<0x142, 0xa>(x);  // row r-1's last lane into rows 1, 3
  if constexpr (W == 64) x += dpp_f<0x143, 0xc>(x);  // lane 31 into rows 2, 3
  return x;
}

// Sum over the 16 lanes of this lane's row, returned in every lane of the row.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f<0x128>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x122>(x);
  x += dpp_f<0x121>(x);
  return x;
}

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Value held by the last lane of this lane's group of W consecutive lanes.
template <int W>
__device__ __forceinline__ float group_last(float x, int lane) {
  if constexpr (W == 64) {
    return readlane_f(x, 63);
  } else {
    float r = 0.f;
#pragma unroll
    for (int g = 0; g < 64 / W; ++g) {
      const float v = readlane_f(x, g * W + W - 1);
      if (lane / W == g) r = v;
    }
    return r;
  }
}

// Maximum over the whole wave (uniform result).
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_f<0x128>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  x = fmaxf(x, dpp_f<0x122>(x));
  x = fmaxf(x, dpp_f<0x121>(x));
  return fmaxf(fmaxf(readlane_f(x, 0), readlane_f(x, 16)), fmaxf(readlane_f(x, 32), readlane_f(x, 48)));
}

// N consecutive elements c0..c0+N-1 of an LDS row with `cols` elements (row pitch
// pitch_elems, default cols); columns past the row end, and every column of an invalid row,
// read as zero.  Whole 16-, 8- or 4-byte vectors when the row pitch and the range allow it
// (c0 is a multiple of N: the vectors are aligned whenever the pitch is).
template <typename T, int N>
__device__ __forceinline__ void lds_row_read(T (&out)[N], const T* row, int c0, int cols,
                                             bool valid, int pitch_elems = -1) {
  constexpr int V16 = 16 / (int)sizeof(T), V8 = 8 / (int)sizeof(T), V4 = 4 / (int)sizeof(T);
  const int pitch = (pitch_elems < 0 ? cols : pitch_elems) * (int)sizeof(T);
  if (N % V16 == 0 && (pitch & 15) == 0 && c0 + N <= cols) {
#pragma unroll
    for (int j = 0; j < N; j += V16) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + c0 + j);
      const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int i = 0; i < V16; ++i) out[j + i] = e[i];
    }
  } else if (N % V8 == 0 && (pitch & 7) == 0 && c0 + N <= cols) {
#pragma unroll
    for (int j = 0; j < N; j += V8) {
      const uint2 u = *reinterpret_cast<const uint2*>(row + c0 + j);
      const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int i = 0; i < V8; ++i) out[j + i] = e[i];
    }
  } else if (c0 >= cols) {  // wholly past the row end
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = from_f<T>(0.f);
  } else if (N % V4 == 0 && (pitch & 3) == 0 && c0 + N <= cols) {
#pragma unroll
    for (int j = 0; j < N; j += V4) {
      const unsigned u = *reinterpret_cast<const unsigned*>(row + c0 + j);
      const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int i = 0; i < V4; ++i) out[j + i] = e[i];
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = (c0 + j < cols) ? row[c0 + j] : from_f<T>(0.f);
  }
  if (!valid) {
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = from_f<T>(0.f);
  }
}

// Same with the row width known at compile time and the range inside the row (c0 + N <=
// COLS, c0 a multiple of N): whole 16-byte vectors whenever the widths allow.
template <typename T, int N, int COLS>
__device__ __forceinline__ void lds_row_read_k(T (&out)[N], const T* row, int c0, bool valid) {
  constexpr int V16 = 16 / (int)sizeof(T), V8 = 8 / (int)sizeof(T);
  constexpr int PB = COLS * (int)sizeof(T), NB = N * (int)sizeof(T);
  if constexpr (PB % 16 == 0 && NB % 16 == 0) {
#pragma unroll
    for (int j = 0; j < N; j += V16) {
      const uint4 u = *reinterpret_cast<const uint4*>(row + c0 + j);
      const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int i = 0; i < V16; ++i) out[j + i] = e[i];
    }
  } else if constexpr (PB % 8 == 0 && NB % 8 == 0) {
#pragma unroll
    for (int j = 0; j < N; j += V8) {
      const uint2 u = *reinterpret_cast<const uint2*>(row + c0 + j);
      const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int i = 0; i < V8; ++i) out[j + i] = e[i];
    }
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = row[c0 + j];
  }
  if (!valid) {
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = from_f<T>(0.f);
  }
}

// Store N consecutive elements to an LDS row at element offset c0 (16-byte vectors when
// the byte offset is 16-aligned and N fills whole vectors).
template <typename T, int N>
__device__ __forceinline__ void lds_row_write(T* row, int c0, const T (&in)[N]) {
  constexpr int V16 = 16 / (int)sizeof(T), V8 = 8 / (int)sizeof(T);
  if constexpr (N % V16 == 0) {
    if (((reinterpret_cast<uintptr_t>(row + c0)) & 15) == 0) {
#pragma unroll
      for (int j = 0; j < N; j += V16) {
        uint4 u;
        T* e = reinterpret_cast<T*>(&u);
#pragma unroll
        for (int i = 0; i < V16; ++i) e[i] = in[j + i];
        *reinterpret_cast<uint4*>(row + c0 + j) = u;
      }
      return;
    }
  }
  if constexpr (N % V8 == 0) {
    if (((reinterpret_cast<uintptr_t>(row + c0)) & 7) == 0) {
#pragma unroll
      for (int j = 0; j < N; j += V8) {
        uint2 u;
        T* e = reinterpret_cast<T*>(&u);
#pragma unroll
        for (int i = 0; i < V8; ++i) e[i] = in[j + i];
        *reinterpret_cast<uint2*>(row + c0 + j) = u;
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < N; ++j) row[c0 + j] = in[j];
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

// ------------------------------------------------------- direct global -> LDS copies
// gfx950 LDS DMA: lane i of a wave writes its PS-byte piece to (wave-uniform LDS base) + i*PS.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

template <int PS>
__device__ __forceinline__ void dma_pieces(unsigned char* lds_dst, const unsigned char* gsrc,
                                           long gstride, int ppr, int npieces, int wave,
                                           int nwaves, int lane) {
  for (int base = wave * 64; base < npieces; base += nwaves * 64) {
    const int e = base + lane;
    if (e < npieces) {
      const int r = e / ppr, c = e - r * ppr;
      gbl_ptr_t g = (gbl_ptr_t)(gsrc + (long)r * gstride + c * PS);
      lds_ptr_t l = (lds_ptr_t)(lds_dst + base * PS);
      if constexpr (PS == 16)
        __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
      else if constexpr (PS == 4)
        __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(g, l, 2, 0, 0);
    }
  }
}

// Lane -> piece mapping of a tile with `cols` elements per row, copied with one DMA
// instruction covering rpi whole rows (pieces of ps bytes, ppr pieces per row).
struct DmaMap {
  int ps, ppr, rpi, lr, lc, rowbytes;
};

template <typename T>
__device__ __forceinline__ DmaMap dma_map(int cols, int lane) {
  DmaMap m;
  m.rowbytes = cols * (int)sizeof(T);
  m.ps = (m.rowbytes & 15) == 0 ? 16 : ((m.rowbytes & 3) == 0 ? 4 : 2);
  m.ppr = m.rowbytes / m.ps;
  m.rpi = m.ppr <= 64 ? 64 / m.ppr : 0;
  m.lr = m.rpi ? lane / m.ppr : 0;
  m.lc = lane - m.lr * m.ppr;
  return m;
}

// Rows [0, valid) of a token-major tile into packed LDS rows, whole rows per instruction.
template <typename T>
__device__ __forceinline__ void dma_rows(const DmaMap& m, T* lds_dst, const T* gsrc, long gstride,
                                         int valid, int wave, int nwaves, int lane) {
  unsigned char* d = reinterpret_cast<unsigned char*>(lds_dst);
  const unsigned char* s = reinterpret_cast<const unsigned char*>(gsrc);
  const long gs = gstride * (long)sizeof(T);
  if (m.rpi == 0) {  // rows wider than one instruction: piecewise
    if (m.ps == 16) dma_pieces<16>(d, s, gs, m.ppr, valid * m.ppr, wave, nwaves, lane);
    else if (m.ps == 4) dma_pieces<4>(d, s, gs, m.ppr, valid * m.ppr, wave, nwaves, lane);
    else dma_pieces<2>(d, s, gs, m.ppr, valid * m.ppr, wave, nwaves, lane);
    return;
  }
  for (int rb = wave * m.rpi; rb < valid; rb += nwaves * m.rpi) {
    const int r = rb + m.lr;
    if (m.lr < m.rpi && r < valid) {
      gbl_ptr_t g = (gbl_ptr_t)(s + (long)r * gs + m.lc * m.ps);
      lds_ptr_t l = (lds_ptr_t)(d + rb * m.rowbytes);
      if (m.ps == 16)
        __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
      else if (m.ps == 4)
        __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(g, l, 2, 0, 0);
    }
  }
}

// Compact form of dma_rows (one loop for every row width; small code): rows [0, valid) of
// `rowbytes` bytes each, row r at gsrc + r*gstride_bytes, into packed LDS rows at lds_dst.
// Piece size 16, 4 or 2 bytes: the largest dividing the row.  Waves [0, nwaves) share the
// pieces; lane i of an instruction writes LDS at (instruction base) + i*piece.
__device__ __forceinline__ void dma_rows_c(unsigned char* lds_dst, const unsigned char* gsrc,
                                           long gstride_bytes, int rowbytes, int valid,
                                           int wave, int nwaves, int lane) {
  const int lg = (rowbytes & 15) == 0 ? 4 : ((rowbytes & 3) == 0 ? 2 : 1);
  const int ppr = rowbytes >> lg;
  const int npieces = valid * ppr;
  for (int base = wave * 64; base < npieces; base += nwaves * 64) {
    const int e = base + lane;
    if (e < npieces) {
      const int r = e / ppr, c = e - r * ppr;
      gbl_ptr_t g = (gbl_ptr_t)(gsrc + (long)r * gstride_bytes + (c << lg));
      lds_ptr_t l = (lds_ptr_t)(lds_dst + (base << lg));
      if (lg == 4)
        __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
      else if (lg == 2)
        __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(g, l, 2, 0, 0);
    }
  }
}

// Starts an asynchronous copy of rows [0, valid) of a token-major tile (row r at gsrc + r *
// gstride elements, `cols` elements per row) into LDS as packed rows (pitch = cols).  The
// caller waits with dma_wait() + a barrier, and zero-fills rows >= valid itself.
template <typename T>
__device__ __forceinline__ void dma_tile(T* lds_dst, const T* gsrc, long gstride, int valid,
                                         int cols, int wave, int nwaves, int lane) {
  const int rowbytes = cols * (int)sizeof(T);
  const long gs = gstride * (long)sizeof(T);
  unsigned char* d = reinterpret_cast<unsigned char*>(lds_dst);
  const unsigned char* s = reinterpret_cast<const unsigned char*>(gsrc);
  if ((rowbytes & 15) == 0)
    dma_pieces<16>(d, s, gs, rowbytes >> 4, valid * (rowbytes >> 4), wave, nwaves, lane);
  else if ((rowbytes & 3) == 0)
    dma_pieces<4>(d, s, gs, rowbytes >> 2, valid * (rowbytes >> 2), wave, nwaves, lane);
  else
    dma_pieces<2>(d, s, gs, rowbytes >> 1, valid * (rowbytes >> 1), wave, nwaves, lane);
}

// ------------------------------------------------------- register prefetch of raw rows
// ROWS rows of RB bytes each (row r at gsrc + r * gstride bytes) held in VGPRs, shared by NTH
// threads in pieces of 16, 8 or 4 bytes (the largest dividing RB).  load() starts ordinary
// vector loads (rows >= valid read as zero); put() writes the rows packed (pitch RB) to LDS.
// Unlike an LDS DMA, nothing in between has to wait for these loads: the wait lands at put().
template <int PB> struct PieceType;
template <> struct PieceType<16> { using type = uint4; };
template <> struct PieceType<8> { using type = uint2; };
template <> struct PieceType<4> { using type = unsigned; };

// LDS row pitch LP bytes (>= RB; a padded pitch keeps accesses that walk rows conflict-free):
// each piece is written as one store when LP keeps it aligned, else as 8- or 4-byte parts.
template <int RB, int ROWS, int NTH, int LP = RB>
struct RowRegs {
  static_assert(RB % 4 == 0 && LP % 4 == 0 && LP >= RB, "row and pitch in dwords");
  static constexpr int PB = RB % 16 == 0 ? 16 : (RB % 8 == 0 ? 8 : 4);
  static constexpr int PR = RB / PB;                     // pieces per row
  static constexpr int NPC = ROWS * PR;                  // pieces in the tile
  static constexpr int NP = (NPC + NTH - 1) / NTH;       // pieces per thread
  static constexpr int WB = LP % PB == 0 ? PB : (LP % 8 == 0 && PB % 8 == 0 ? 8 : 4);
  using P = typename PieceType<PB>::type;
  using PW = typename PieceType<WB>::type;
  P v[NP];
  // Branch-free on purpose (a branch around a load makes the compiler's wait analysis
  // pessimistic): threads past the last piece repeat it, and rows >= valid load row valid-1
  // and are replaced by zeros in put().
  __device__ __forceinline__ void load(const unsigned char* gsrc, long gstride, int valid,
                                       int tid) {
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int e = min(tid + NTH * m, NPC - 1), r = e / PR, c = e - r * PR;
      v[m] = *reinterpret_cast<const P*>(gsrc + (long)min(r, valid - 1) * gstride + c * PB);
    }
  }
  __device__ __forceinline__ void put(unsigned char* lds, int valid, int tid) const {
#pragma unroll
    for (int m = 0; m < NP; ++m) {
      const int e = min(tid + NTH * m, NPC - 1), r = e / PR, c = e - r * PR;
      P x = v[m];
      if (r >= valid) x = P{};
      const PW* xs = reinterpret_cast<const PW*>(&x);
#pragma unroll
      for (int k = 0; k < PB / WB; ++k)
        *reinterpret_cast<PW*>(lds + r * LP + c * PB + k * WB) = xs[k];
    }
  }
};

// Rows [0, valid) of a packed LDS tile (pitch RB bytes) stored to global rows `gstride`
// bytes apart, branch-free with a fixed number of stores per thread (so the compiler can
// count them when it waits for loads issued earlier): threads past the last piece repeat it
// and rows >= valid repeat row valid-1, i.e. the same bytes to the same address.
template <int RB, int ROWS, int NTH, int LP = RB>
__device__ __forceinline__ void store_rows_fixed(unsigned char* gdst, long gstride,
                                                 const unsigned char* lds, int valid, int tid) {
  using R = RowRegs<RB, ROWS, NTH, LP>;
  using P = typename R::P;
  using PW = typename R::PW;
#pragma unroll
  for (int m = 0; m < R::NP; ++m) {
    const int e = min(tid + NTH * m, R::NPC - 1), c = e % R::PR;
    const int r = min(e / R::PR, valid - 1);
    P x;
    PW* xs = reinterpret_cast<PW*>(&x);
#pragma unroll
    for (int k = 0; k < R::PB / R::WB; ++k)
      xs[k] = *reinterpret_cast<const PW*>(lds + r * LP + c * R::PB + k * R::WB);
    *reinterpret_cast<P*>(gdst + (long)r * gstride + c * R::PB) = x;
  }
}

// Row pitch (bytes, >= rb) at which one lane per row reading nb bytes of the row, with the
// widest vector reads the pitch allows (16 or 8 bytes, as lds_row_read_k does), hits distinct
// banks: P / w odd for the read width w.  Among the widths nb allows, the smallest such pitch
// (wider reads on ties); rows of other widths fall back to 4-byte alignment.
constexpr int odd_multiple_pitch(int rb, int w) {
  int p = (rb + w - 1) / w * w;
  if ((p / w) % 2 == 0) p += w;
  return p;
}
constexpr int row_pitch(int rb, int nb) {
  const int p16 = nb % 16 == 0 ? odd_multiple_pitch(rb, 16) : 1 << 30;
  const int p8 = nb % 8 == 0 ? odd_multiple_pitch(rb, 8) : 1 << 30;
  if (p16 <= p8 && p16 < (1 << 30)) return p16;
  if (p8 < (1 << 30)) return p8;
  return odd_multiple_pitch(rb, 4);
}

// Waits for this wave's outstanding memory operations (LDS DMA included).
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt = 0; s_waitcnt encoding 0xC07F leaves vmcnt/expcnt unconstrained) and keeps the
// compiler from moving memory accesses across it.  Unlike __syncthreads() it does not wait
// for this wave's global->LDS copies still in flight, so a wave that prefetches can pass it.
// Callers must not rely on it for LDS written by such copies.
__device__ __forceinline__ void barrier_lds() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Zero rows [valid, rows) of a packed LDS tile.
template <typename T>
__device__ __forceinline__ void zero_rows(T* dst, int valid, int rows, int cols, int tid,
                                          int nthr) {
  for (int i = valid * cols + tid; i < rows * cols; i += nthr) dst[i] = from_f<T>(0.f);
}

// Cross-workgroup exchange inside one launch (the GLA look-back kernels).  Every exchanged
// value goes through device-scope loads and stores, which the L2 of each
// XCD does not hold back; the stores have completed (waited for) before the flag is
// written, and the values are loaded only after the flag is seen.  No L2 write-back or
// invalidation is needed (fences would do both, over the whole L2, per wave).
constexpr unsigned kLbSpinLimit = 1u << 18;  // default bound: polls of at least ~1 us, far past any real wait
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<unsigned*>(const_cast<float*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Each launch also clears its flags before it ends: every workgroup raises a second ("done")
// flag once its own waits are over, and the last workgroup waits for all of those and then
// zeroes both arrays.  A launch therefore never sees flags raised by an earlier one, also when
// the same arguments (the same tag) are replayed, as from a captured graph; the per-call tag
// covers a workspace that has never been used.
//
// Every wait is bounded (spin_limit polls).  A wait that gives up returns true; the caller
// then records it in the sticky status word (lb_fail) and poisons what the missing values fed
// with NaN, so that the output is visibly wrong and the host can ask for the status.
//
// Waits until flags[0..count) all hold tag (lane j polls flag j; count <= 64).  Returns true
// on every lane of the wave if any lane gave up.
__device__ __forceinline__ bool lb_wait_all(const unsigned* flags, int count, unsigned tag,
                                            int lane, unsigned spin_limit) {
  bool expired = false;
  if (lane < count) {
    unsigned spins = 0;
    while (__hip_atomic_load(const_cast<unsigned*>(flags + lane), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) != tag) {
      if (++spins >= spin_limit) {
        expired = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return __any(expired);
}

// Every thread: waits until flags[0..n) all hold tag, n any size (the workgroup's threads
// share the flags; a workgroup barrier follows in the caller).  Returns true on the threads
// whose own wait gave up.
__device__ __forceinline__ bool lb_wait_each(const unsigned* flags, int n, unsigned tag, int tid,
                                             int nthreads, unsigned spin_limit) {
  bool expired = false;
  for (int i = tid; i < n; i += nthreads) {
    unsigned spins = 0;
    while (__hip_atomic_load(const_cast<unsigned*>(flags + i), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) != tag) {
      if (++spins >= spin_limit) {
        expired = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return expired;
}
__device__ __forceinline__ void lb_raise(unsigned* flag, unsigned tag) {
  __hip_atomic_store(flag, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Records an expired wait in the sticky status word (kept until the host reads and clears it).
__device__ __forceinline__ void lb_fail(unsigned* status) {
  __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace dig
