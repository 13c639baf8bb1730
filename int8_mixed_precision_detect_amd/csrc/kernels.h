// Internal launchers of libi8mm (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

void launch_wquant(const _Float16* W, int64_t N, int64_t K, int8_t* CB, float* SCB, bool vec,
                   hipStream_t st);
// Outlier detection: OR the column flags |x| >= thr of row blocks into
// mask[ceil(K/32)], which must be zero on entry (clear: zero it first, with
// one more launch -- the stage entry point; the forward's mask is left zero
// by the previous call's product kernel).
void launch_detect(const _Float16* X, int64_t T, int64_t K, float thr, uint32_t* mask, bool clear,
                   bool vec, hipStream_t st);
// zero words [0, n) of p (a fill kernel: no memset node in a captured graph)
void launch_zero_words(uint32_t* p, int64_t n, hipStream_t st);
// mask -> ascending O (first max_o entries), counts {n_o, overflow, 0, 0}.
void launch_compact(const uint32_t* mask, int64_t K, int32_t* O, int32_t* counts, int64_t max_o,
                    hipStream_t st);

// Step 2 preparation in one launch (see k_prep): the outlier set from the
// mask, optionally published as O/counts (counts != null), rows of X
// quantized (Xq != null) and the dequantized outlier weights (Wo != null).
struct PrepArgs {
  const _Float16* X;
  int64_t T, K;
  const uint32_t* mask;
  int32_t* O_out;  // written by workgroup 0 when counts != null
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
  int64_t ocap;     // outlier-list capacity in LDS (entries)
  int64_t wo_skip;  // Wo is built only when the outlier set exceeds this
  bool vec;         // 16-byte aligned rows of X (K % 8 == 0)
  // fp16 weight [N][K]: Wo copies W16[:, O] instead of dequantizing CB
  const _Float16* W16 = nullptr;
  // zero-point row codes: the offsets Z [T] out (non-null selects the
  // scheme) and the per-channel sums of the outlier codes [N] out
  int32_t* zp = nullptr;
  int32_t* osum = nullptr;
};
// rsum[j] = sum_k CB[j, k] (int32), once per weight (zero-point layer)
void launch_rowsum(const int8_t* CB, int64_t N, int64_t K, int32_t* rsum, hipStream_t st);
// LDS of the step-2 kernel: mask[KW], pref[KW + 1], O[ocap]
constexpr size_t prep_lds_bytes(int64_t K, int64_t ocap) {
  return (size_t)((2 * ((K + 31) / 32) + 1 + ocap) * 4);
}
// Largest K the forward takes (an LDS copy of its outlier bit mask, 32 KB)
// and the largest outlier list kept in LDS.
constexpr int64_t kMaxK = (int64_t)1 << 18;
constexpr int64_t kMaxOcap = 4096;
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
  const int32_t* O;  // ascending outlier list (few-token calls)
  int64_t max_o;
  const _Float16* bias;
  _Float16* Y;
  // int32 output instead of the epilogue
  int32_t* C;
  // split K (fused product only): `splits` workgroups a tile each walk a
  // contiguous range of K and store their int32 accumulators in `part`
  // (splits x tiles x BM x BN); a second launch adds them and runs the
  // epilogue.
  int64_t splits;
  int64_t cfg;  // tile configuration of the plan (see plan_gemm_i8); -1: choose
  int32_t* part;
  // Wo is already in the workspace (the few-token tiles must not rebuild it
  // from CB: the fp16-weight variant takes it from W)
  bool wo_ready;
  // the forward's outlier mask (clear_words words), zeroed by the first
  // workgroup of the call's first product launch: step 2 has read it, and
  // the next call's detection starts from zero
  uint32_t* clear_mask;
  int64_t clear_words;
  // zero-point activations (zp non-null): acc + zp[t] * (rsum[j] - osum[j])
  // is the int8 part (osum read only when there are outlier columns)
  const int32_t* zp;
  const int32_t* rsum;
  const int32_t* osum;
  // Wo is not built (steps 1-2 ran as k_rows): the few-token products take
  // the codes of every outlier set from CB themselves, whatever its width
  bool wo_gather;
};

// Any shape and alignment: register-staged, byte-granular loads.
hipError_t launch_gemm_fused(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_s32(const GemmArgs& a, hipStream_t st);

// 16-byte aligned operands (K, lda, ldb multiples of 16): the pipelined
// gfx950 kernel.
bool gemm_i8_supported(const GemmArgs& a);
// The tile configuration and K split the fused product takes for a shape on
// this device, and the workspace it needs for them.
struct GemmPlan {
  int64_t cfg;         // tile configuration (few-token tiles: -1)
  int64_t splits;      // 1: no split
  int64_t tiles;       // output tiles
  int64_t part_elems;  // int32 elements of partial accumulators
};
GemmPlan plan_gemm_i8(int64_t T, int64_t N, int64_t K);
// Process-wide override of the K split (0: the plan's own choice); a test
// and tuning control.
void set_split_override(int64_t splits);
int64_t split_override();
// Process-wide choice of the wide tile configuration (-1: the plan's own).
void set_tile_override(int64_t cfg);
hipError_t launch_gemm_i8_fused(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_i8_s32(const GemmArgs& a, hipStream_t st);

// Few tokens (1 <= T <= kFewT, aligned operands): launch_gemm_i8_* run thin
// tiles with one token tile, and the fused one extracts the outlier weights of
// sets of at most kFewOcap columns itself (the step-2 kernel then skips Wo).
constexpr int64_t kFewT = 32;
constexpr int64_t kFewOcap = 128;
// 1 <= T <= 4: the row-streaming kernel (1 KB of a weight row per load,
// VALU dot products)
bool gemv_supported(const GemmArgs& a);
hipError_t launch_gemv(const GemmArgs& a, bool fused, hipStream_t st);
// Up to kRowsMaxT rows of X (1 <= T <= 8, K % 8 == 0, K <= kRow1MaxK,
// 16-byte aligned): steps 1-2 in one launch of one workgroup -- counts, O,
// sx, Xq (ldq) and Xo (ldo), the same values k_detect + k_prep write (the
// mask is not used); Wo is left to the product (wo_gather).
constexpr int64_t kRow1MaxK = 16384;
constexpr int kRowsMaxT = 8;
void launch_rows(const _Float16* X, int64_t T, int64_t K, float thr, int32_t* O, int32_t* counts,
                 int64_t max_o, int8_t* Xq, int64_t ldq, float* sx, _Float16* Xo, int64_t ldo,
                 hipStream_t st);

}  // namespace i8mm
