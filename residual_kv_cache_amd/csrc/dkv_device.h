// Device-side helpers of the DeltaKV kernels: storage conversions with
// exact rounding, MFMA operand types and small wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dkv {

// Word 3 of a raw buffer descriptor (gfx9 family): 32-bit data format, so
// untyped loads return the bytes as stored; a load whose offset (lane offset
// plus immediate) is at or past the size in word 2 (bytes, for stride 0)
// returns zeros.
constexpr int kBufferRsrcWord3 = 0x00020000;

// Raw buffer descriptor over `bytes` bytes from base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kBufferRsrcWord3);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bfloat16 <-> float32.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bfloat16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Moves a float32 that was rounded to nearest from an exact value x = a + err
// (|err| <= half an ulp of a) to x rounded to odd: if the rounding was
// inexact and a's last significand bit is 0, step one ulp towards x.  A value
// rounded to odd at 24 bits and then to nearest-even at 8 bits equals x
// rounded to nearest-even at 8 bits directly (no double-rounding error).
__device__ __forceinline__ float to_odd(float a, float err) {
  uint32_t u = __float_as_uint(a);
  if (err != 0.0f && (u & 1u) == 0u) {
    // step away from zero when err has a's sign, towards zero otherwise
    bool away = (err > 0.0f) == (a > 0.0f);
    u = away ? u + 1u : u - 1u;
  }
  return __uint_as_float(u);
}

// Correctly rounded bfloat16(x - y) for bfloat16-valued x and y.  When the
// exponents of x and y differ by at most 15, x - y has at most 24
// significant bits and the float32 subtraction is exact.  Otherwise the
// smaller operand is below 2^-15 of the larger one's leading bit, so both the
// exact and the float32 difference lie within 2^-8 of a bfloat16 ulp of the
// larger operand, which is itself a bfloat16 value, and round to it.  Either
// way one float32 subtraction and one rounding give the correct result.
__device__ __forceinline__ uint16_t bf16_sub_rn(float x, float y) { return f2bf(x - y); }

// Correctly rounded bfloat16 of a double.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  float a = (float)x;
  double e = x - (double)a;  // exact: a is x rounded to the nearest float
  return f2bf(to_odd(a, e > 0.0 ? 1.0f : (e < 0.0 ? -1.0f : 0.0f)));
}

// Storage types: raw bfloat16 bits or float.
struct BF16 {
  typedef uint16_t T;
  static __device__ __forceinline__ float load(T v) { return bf2f(v); }
  static __device__ __forceinline__ T from_f32(float f) { return f2bf(f); }
  static __device__ __forceinline__ T from_f64(double x) { return f64_to_bf16(x); }
  static __device__ __forceinline__ T sub_rn(float x, float y) { return bf16_sub_rn(x, y); }
};

struct F32 {
  typedef float T;
  static __device__ __forceinline__ float load(T v) { return v; }
  static __device__ __forceinline__ T from_f32(float f) { return f; }
  static __device__ __forceinline__ T from_f64(double x) { return (float)x; }
  static __device__ __forceinline__ T sub_rn(float x, float y) { return x - y; }
};

// Eight consecutive storage elements (16-byte aligned) as floats, through
// global (not flat) loads.
template <class S>
__device__ __forceinline__ void load8(const typename S::T* p, float (&v)[8]) {
  typedef const __attribute__((address_space(1))) u32x4* G4;
  if constexpr (sizeof(typename S::T) == 2) {
    const u32x4 w = *(G4)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const u32x4 a = *(G4)p, b = *((G4)p + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// 4-bit codes: element e of a row sits in byte e / 2, low nibble for even e,
// two's complement.
// ---------------------------------------------------------------------------

// Nibble k (0..7) of a 32-bit word holding elements 8w .. 8w + 7, as float.
__device__ __forceinline__ float q4_at(uint32_t word, int k) {
  return (float)((int32_t)(word << (28 - 4 * k)) >> 28);
}

// Quantized value of code c under `scale` (0 when the scale is 0).
__device__ __forceinline__ int q4_quant(float c, float scale) {
  if (!(scale > 0.f)) return 0;
  const float x = rintf(c / scale);   // IEEE division, ties to even
  return (int)fminf(fmaxf(x, -8.f), 7.f);
}

// ---------------------------------------------------------------------------
// Sorted lists of the best k candidates (score, ordinal) under the total
// order "higher score, then lower ordinal".
// ---------------------------------------------------------------------------

constexpr int kTopMax = 8;

// (s1, r1) ranks before (s2, r2): larger score, then lower ordinal.  Bitwise
// operators, so all three comparisons are evaluated and combined as lane
// masks (short-circuit forms become divergent branches).
__device__ __forceinline__ bool ranks_before(float s1, int r1, float s2, int r2) {
  return (s1 > s2) | ((s1 == s2) & (r1 < r2));
}

template <int KM>
struct TopKN {
  float s[KM];
  int r[KM];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      s[j] = -INFINITY;
      r[j] = 0x7FFFFFFF;
    }
  }
  // Insertion by compare-and-swap down the list (branch-free).
  __device__ __forceinline__ void insert(float cs, int cr, int K) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < K) {
        const bool take = ranks_before(cs, cr, s[j], r[j]);
        const float ts = s[j];
        const int tr = r[j];
        s[j] = take ? cs : s[j];
        r[j] = take ? cr : r[j];
        cs = take ? ts : cs;
        cr = take ? tr : cr;
      }
    }
  }
  // The k-th entry (selects over the fixed-size arrays: no dynamic
  // register indexing).
  __device__ __forceinline__ void kth(int K, float& ks, int& kr) const {
    ks = s[0];
    kr = r[0];
#pragma unroll
    for (int j = 1; j < KM; ++j) {
      ks = j == K - 1 ? s[j] : ks;
      kr = j == K - 1 ? r[j] : kr;
    }
  }
  // Merge with the list of lane (lane ^ mask).
  __device__ __forceinline__ void merge_xor(int mask, int K) {
    float os[KM];
    int orr[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      os[j] = __shfl_xor(s[j], mask, 64);
      orr[j] = __shfl_xor(r[j], mask, 64);
    }
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < K) insert(os[j], orr[j], K);
  }
  // The first c ordinals in ascending order (c <= K), zero after.
  __device__ __forceinline__ void sorted_ordinals(int c, int* out) const {
    int v[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) v[j] = j < c ? r[j] : 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < KM; ++i)
#pragma unroll
      for (int j = 0; j + 1 < KM - i; ++j) {
        const int lo = min(v[j], v[j + 1]), hi = max(v[j], v[j + 1]);
        v[j] = lo;
        v[j + 1] = hi;
      }
#pragma unroll
    for (int j = 0; j < KM; ++j) out[j] = j < c ? v[j] : 0;
  }
};
typedef TopKN<kTopMax> TopK;

// ---------------------------------------------------------------------------
// Wave64 reductions (butterfly; every lane ends with the result).
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Position of coded row n (non-reference tokens in position order), s >= 2.
__device__ __forceinline__ int slot_to_pos(int n, int s) { return (n / (s - 1)) * s + (n % (s - 1)) + 1; }

// Coded row of a non-reference position t.
__device__ __forceinline__ int pos_to_slot(int t, int s) { return t - t / s - 1; }

__device__ __forceinline__ uint32_t load_idx(const void* idx, size_t i, int idx_bytes) {
  return idx_bytes == 2 ? (uint32_t)((const uint16_t*)idx)[i] : ((const uint32_t*)idx)[i];
}

__device__ __forceinline__ void store_idx(void* idx, size_t i, int idx_bytes, uint32_t r) {
  if (idx_bytes == 2)
    ((uint16_t*)idx)[i] = (uint16_t)r;
  else
    ((uint32_t*)idx)[i] = r;
}

}  // namespace dkv
