// Device helpers shared by the libi8mm kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float h2f(_Float16 h) { return (float)h; }

#if defined(__HIP_DEVICE_COMPILE__)
// A raw buffer resource over `bytes` bytes at p: loads at offsets >= bytes
// return 0 without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}
#endif

// n / s with r = fl32(1/s) computed once per row: q0 = n*r, one fused
// correction step.  For n = fl32(x*127) with fp16 x, |x| <= s, s an fp16
// value (the absmax codes), and for n = fl32(c*s) / 127 with a code c (the
// dequantized outlier weights), the result equals the IEEE quotient
// fl32(n/s) -- checked exhaustively over every such pair by
// tests/native/quotient_check.c.  Saves the per-element division sequence.
__device__ __forceinline__ float div_by(float n, float s, float r) {
#pragma clang fp contract(off)
  const float q0 = n * r;
  const float e = __builtin_fmaf(-q0, s, n);
  return __builtin_fmaf(e, r, q0);
}

// Reciprocal for the absmax codes of a row with scale s: fl32(1/s), and 0
// for s == 0 (every code of such a row is 0, with no per-element test).
__device__ __forceinline__ float code_recip(float s) { return s > 0.0f ? 1.0f / s : 0.0f; }

// Absmax code of one value, |x| <= s, r = code_recip(s): round half away
// from zero of the IEEE fp32 quotient fl32(x * 127) / s (x*127 is exact for
// fp16 x).  The quotient comes from div_by; the rounding is an fp32 add of
// +-0.5 and a truncating conversion.  On its own that add can round (just
// below 0.5, for instance), but for every quotient these codes can produce
// -- every fp16 pair |x| <= s -- it equals the exact rule, as checked
// exhaustively by tests/native/quotient_check.c.  |q| <= 127, so no clamp.
__device__ __forceinline__ int absmax_code(float x, float s, float r) {
#pragma clang fp contract(off)
  const float q = div_by(x * 127.0f, s, r);
  return (int)(q + __builtin_copysignf(0.5f, q));
}

// Codes of 8 fp16 values (|v[e]| <= s), packed little-endian into 8 bytes.
__device__ __forceinline__ v2u absmax_codes8(v8h v, float s, float r) {
  v2u out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      word |= ((uint32_t)absmax_code((float)v[4 * w + b], s, r) & 0xffu) << (8 * b);
    out[w] = word;
  }
  return out;
}

// v with the elements whose bit is set in the low 8 bits of `bits` zeroed
__device__ __forceinline__ v8h zero_masked8(v8h v, uint32_t bits) {
  if (bits & 0xffu) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((bits >> e) & 1u) v[e] = (_Float16)0.0f;
  }
  return v;
}

// max |v[e]| in fp16 (exact), as float
__device__ __forceinline__ float absmax8(v8h v) {
  typedef _Float16 v2h __attribute__((ext_vector_type(2)));
  v2h m = __builtin_elementwise_abs(v2h{v[0], v[1]});
#pragma unroll
  for (int e = 2; e < 8; e += 2)
    m = __builtin_elementwise_max(m, __builtin_elementwise_abs(v2h{v[e], v[e + 1]}));
  return fmaxf((float)m[0], (float)m[1]);
}

// fp16(fl32(fl32(c * s) / 127)): a dequantized outlier weight
__device__ __forceinline__ _Float16 dequant_weight(int c, float s) {
#pragma clang fp contract(off)
  const float p = (float)c * s;  // exact: <= 8 x 11 significant bits
  return (_Float16)div_by(p, 127.0f, 1.0f / 127.0f);
}

// ---- zero-point (asymmetric) row codes ----
// Round half away from zero, exactly: v - trunc(v) is exact in fp32.
__device__ __forceinline__ float rhaz_exact(float v) {
  const float t = __builtin_truncf(v);
  return __builtin_fabsf(v - t) >= 0.5f ? t + __builtin_copysignf(1.0f, v) : t;
}

// Parameters of a row whose kept values span [lo, hi] with lo <= 0 <= hi:
// d = fl32(hi - lo), S = fl32(254 / d), Z = rhaz(fl32(lo * S)) + 127 and
// sx = d / 2 (exact); a row with hi == lo gets S = Z = sx = 0.
struct ZpRow {
  float S, sx;
  int Z;
};
__device__ __forceinline__ ZpRow zp_row(float lo, float hi) {
#pragma clang fp contract(off)
  ZpRow z{0.0f, 0.0f, 0};
  const float d = hi - lo;
  if (d > 0.0f) {
    z.S = __fdiv_rn(254.0f, d);  // correctly rounded
    z.Z = (int)rhaz_exact(lo * z.S) + 127;
    z.sx = d * 0.5f;
  }
  return z;
}

// Zero-point code of a kept value: clamp(rhaz(fl32(fl32(x * S) - Z)), +-127)
// (contraction off: the product is rounded before the subtraction, as the
// definition says, not fused into one multiply-add)
__device__ __forceinline__ int zp_code(float x, const ZpRow& z) {
#pragma clang fp contract(off)
  const float p = x * z.S;  // written out here: the pragma covers only these
  const float t = p - (float)z.Z;
  const float q = rhaz_exact(t);
  return (int)__builtin_fminf(127.0f, __builtin_fmaxf(-127.0f, q));
}

// Codes of 8 fp16 values; positions whose bit is set in the low 8 bits of
// `bits` (outlier columns) get code 0.
__device__ __forceinline__ v2u zp_codes8(v8h v, uint32_t bits, const ZpRow& z) {
  v2u out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int e = 4 * w + b;
      const int q = ((bits >> e) & 1u) ? 0 : zp_code((float)v[e], z);
      word |= ((uint32_t)q & 0xffu) << (8 * b);
    }
    out[w] = word;
  }
  return out;
}

// min and max of 8 fp16 values (exact), as floats
__device__ __forceinline__ void minmax8(v8h v, float& lo, float& hi) {
  typedef _Float16 v2h __attribute__((ext_vector_type(2)));
  v2h mn = v2h{v[0], v[1]}, mx = mn;
#pragma unroll
  for (int e = 2; e < 8; e += 2) {
    mn = __builtin_elementwise_min(mn, v2h{v[e], v[e + 1]});
    mx = __builtin_elementwise_max(mx, v2h{v[e], v[e + 1]});
  }
  lo = fminf(lo, fminf((float)mn[0], (float)mn[1]));
  hi = fmaxf(hi, fmaxf((float)mx[0], (float)mx[1]));
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Block-wide max of non-negative values; every thread gets the result.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* lds /* NT/64 floats */) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (NT > kWave) {
    if (l == 0) lds[w] = v;
    __syncthreads();
    v = lds[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) v = fmaxf(v, lds[i]);
    __syncthreads();
  }
  return v;
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Raises a kernel's dynamic-LDS limit to `bytes` once per process, on its
// first launch (later calls return the first call's status without a HIP
// call); `bytes` must be the most the kernel is ever launched with.
template <auto Kern>
inline hipError_t lds_limit(size_t bytes) {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  return e;
}

}  // namespace i8mm
