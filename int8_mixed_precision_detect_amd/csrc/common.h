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

// Absmax code of one value: round half away from zero of the IEEE fp32
// quotient fl32(x * 127) / s (x*127 is exact for fp16 x); 0 when s == 0.
// r must be fl32(1/s) (any value when s == 0).
__device__ __forceinline__ int8_t absmax_code(float x, float s, float r) {
#pragma clang fp contract(off)
  if (s == 0.0f) return 0;
  float q = div_by(x * 127.0f, s, r);
  q = __builtin_roundf(q);               // half away from zero
  q = fminf(fmaxf(q, -127.0f), 127.0f);  // no-op for |x| <= s
  return (int8_t)(int)q;
}

// fp16(fl32(fl32(c * s) / 127)): a dequantized outlier weight
__device__ __forceinline__ _Float16 dequant_weight(int c, float s) {
#pragma clang fp contract(off)
  const float p = (float)c * s;  // exact: <= 8 x 11 significant bits
  return (_Float16)div_by(p, 127.0f, 1.0f / 127.0f);
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

}  // namespace i8mm
