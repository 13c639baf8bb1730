// Internal launchers of libi8mm (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

void launch_wquant(const _Float16* W, int64_t N, int64_t K, int8_t* CB, float* SCB, bool vec,
                   hipStream_t st);
// Outlier detection: per-row-block column flags, and (for the stage entry
// point) their compaction into mask, O and counts.
void launch_detect_partial(const _Float16* X, int64_t T, int64_t K, float thr, uint32_t* partial,
                           int64_t rows_per_block, int64_t nrb, bool vec, hipStream_t st);
void launch_detect_compact(const uint32_t* partial, int64_t nrb, int64_t K, uint32_t* mask,
                           int32_t* O, int32_t* counts, int64_t max_o, hipStream_t st);

// Step 2 preparation in one launch (see k_prep): rebuilds the outlier set
// from `partial` (nrb row blocks of ceil(K/32) words; a final mask is nrb 1),
// optionally publishes mask/O/counts, quantizes rows (Xq != null) and builds
// the dequantized outlier weights (Wo != null; only when the outlier set is
// larger than small_tail).
struct PrepArgs {
  const _Float16* X;
  int64_t T, K;
  const uint32_t* partial;
  int64_t nrb;
  uint32_t* mask_out;  // published by workgroup 0 when counts != null
  int32_t* O_out;
  int32_t* counts;
  int64_t max_o;
  int8_t* Xq;
  int64_t ldq;
  float* sx;
  _Float16* Xo;
  int64_t ldo;
  const int8_t* CB;
  const float* SCB;
  int64_t N;
  _Float16* Wo;
  int64_t small_tail;  // Wo is built only when n_use > small_tail
  int64_t ocap;        // O-list capacity in LDS for the Wo workgroups
  bool stage_rows;     // stage CB rows in LDS for the Wo gather
  bool vec;            // 16-byte aligned rows of X (K % 8 == 0)
};
size_t prep_lds_bytes(int64_t K, int64_t ocap, bool stage_rows);
void launch_prep(const PrepArgs& p, hipStream_t st);
void launch_fill_bias(_Float16* Y, int64_t T, int64_t N, const _Float16* bias, int32_t* counts,
                      hipStream_t st);

// Fused product: Y = fp16(acc*sx*SCB/127^2 + Xo.Wo^T + bias), acc = Xq.CB^T.
struct GemmArgs {
  const int8_t* A;  // CB [N][lda] (features)
  int64_t lda;
  const int8_t* B;  // Xq [T][ldb] (tokens)
  int64_t ldb;
  int64_t N, T, K;
  // fused epilogue
  const float* sx;
  const float* SCB;
  const _Float16* Wo;
  const _Float16* Xo;
  int64_t ldo;
  const int32_t* counts;
  int64_t max_o;
  const _Float16* bias;
  _Float16* Y;
  // int32 output instead of the epilogue
  int32_t* C;
  // fp32 [T][N] product over a large outlier set (more than kSmallTail
  // columns); only read or written in that case
  float* P;
};

// Outlier columns the aligned fused kernel handles inside its epilogue
// (3 slices of 32, staged in LDS); beyond that a separate fp16 launch writes
// P first.
constexpr int64_t kSmallTail = 96;

// Any shape and alignment: register-staged, byte-granular loads.
hipError_t launch_gemm_fused(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_s32(const GemmArgs& a, hipStream_t st);

// 16-byte aligned operands (K, lda, ldb multiples of 16): the pipelined
// gfx950 kernel.
bool gemm_i8_supported(const GemmArgs& a);
hipError_t launch_gemm_i8_fused(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_i8_s32(const GemmArgs& a, hipStream_t st);

}  // namespace i8mm
