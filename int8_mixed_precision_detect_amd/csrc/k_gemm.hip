// The product of the LLM.int8() layer on gfx950 int8 matrix cores.
//
// acc = Xq . CB^T in exact int32 (v_mfma_i32_16x16x64_i8), then in the same
// registers: scale to fp32 by sx[i] * SCB[j] / 127^2, add the fp16 outlier
// product Xo . Wo^T (v_mfma_f32_16x16x32_f16 over the padded outlier
// columns), add the bias and store fp16.  This is step 2 (int8 product of the
// non-outlier dims, fp16 product of the outlier dims) and step 3 (dequantize
// and sum) of "LLM.int8() の核心アイデア" on the Hugging Face summary page.
//
// Roles: the MFMA "A" side is the weight (rows = output channels j), the
// "B" side the activations (rows = tokens i), so a lane's four accumulator
// values are four consecutive output channels of one token and the fp16
// store is one 8-byte write per lane.
//
// This is the general kernel: any K, any leading dimension, any alignment
// (byte-granular loads), any number of outlier columns.  16-byte aligned
// operands take the pipelined kernel in k_gemm_i8.hip instead.
//
// Tiling: a workgroup owns a BM x BN (channels x tokens) output tile, split
// among waves of WM x WN, and walks K in 64-byte slices staged through LDS
// (two buffers, register staged).  LDS rows are 64 bytes (4 chunks of 16); chunk cc of row r is
// stored at chunk cc ^ ((r>>1)&3), which keeps the 16-byte fragment reads
// free of bank conflicts on gfx950 (measured with SQ_LDS_BANK_CONFLICT).
#include "common.h"
#include "kernels.h"

namespace i8mm {

__device__ __forceinline__ int lds_off(int r, int cc) {
  return r * 64 + ((cc ^ ((r >> 1) & 3)) << 4);
}

// 16 bytes at byte offset k0 + kc of a row (p = row start); zero past Kb.
template <bool VEC>
__device__ __forceinline__ v4i load16(const char* p, int64_t k0, int kc, int64_t Kb) {
  if (VEC) {
    // Kb is a multiple of 16 here, so a chunk is wholly in or out; a chunk
    // that is out reads the row's first 16 bytes (always valid) and selects
    // zero, which keeps the tail free of branches.
    const bool ok = k0 + kc < Kb;
    v4i v = *(const v4i*)(p + (ok ? k0 + kc : 0));
    return ok ? v : v4i{0, 0, 0, 0};
  } else {
    v4u v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t k = k0 + kc + e;
      const uint32_t b = (k < Kb) ? (uint32_t)(uint8_t)p[k] : 0u;
      v[e >> 2] |= b << (8 * (e & 3));
    }
    return __builtin_bit_cast(v4i, v);
  }
}

template <int BM, int BN, int WM, int WN, bool FUSED, bool VEC>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm(GemmArgs a) {
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int LA = BM * 4 / NT, LB = BN * 4 / NT;
  static_assert((BM * 4) % NT == 0 && (BN * 4) % NT == 0, "tile/thread mismatch");
  constexpr int STAGE = (BM + BN) * 64;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / NWN) * WM, wn0 = (wave % NWN) * WN;
  // the forward's outlier mask: step 2 is done with it; zero it for the next
  // call's detection
  if (a.clear_mask && blockIdx.x == 0)
    for (int64_t w = tid; w < a.clear_words; w += NT) a.clear_mask[w] = 0u;

  // tile order: blocks are dealt to the 8 XCDs round-robin; give each XCD a
  // contiguous run of tiles, consecutive tiles sharing one weight tile.
  const int64_t tiles_m = ceil_div(a.N, BM), tiles_n = ceil_div(a.T, BN);
  const int64_t ntiles = tiles_m * tiles_n;
  int64_t bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  const int64_t tn = bid % tiles_n, tm = bid / tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const char* pa[LA];
  const char* pb[LB];
  int la[LA], lb[LB], ka[LA], kb[LB];
  auto setup = [&](const char* A, int64_t ldab, const char* B, int64_t ldbb) {
#pragma unroll
    for (int s = 0; s < LA; ++s) {
      const int c = tid + s * NT, r = c >> 2, cc = c & 3;
      const int64_t g = min(m0 + r, a.N - 1);
      pa[s] = A + g * ldab;
      la[s] = lds_off(r, cc);
      ka[s] = cc * 16;
    }
#pragma unroll
    for (int s = 0; s < LB; ++s) {
      const int c = tid + s * NT, r = c >> 2, cc = c & 3;
      const int64_t g = min(n0 + r, a.T - 1);
      pb[s] = B + g * ldbb;
      lb[s] = BM * 64 + lds_off(r, cc);
      kb[s] = cc * 16;
    }
  };
  v4i ra[LA], rb[LB];
  auto gload = [&](int64_t k0, int64_t Kb) {
#pragma unroll
    for (int s = 0; s < LA; ++s) ra[s] = load16<VEC>(pa[s], k0, ka[s], Kb);
#pragma unroll
    for (int s = 0; s < LB; ++s) rb[s] = load16<VEC>(pb[s], k0, kb[s], Kb);
  };
  auto sstore = [&](int buf) {
    char* base = lds + buf * STAGE;
#pragma unroll
    for (int s = 0; s < LA; ++s) *(v4i*)(base + la[s]) = ra[s];
#pragma unroll
    for (int s = 0; s < LB; ++s) *(v4i*)(base + lb[s]) = rb[s];
  };
  const int lo = lds_off(lane & 15, lane >> 4);

  v4i acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  // ---- int8 main loop ----
  setup((const char*)a.A, a.lda, (const char*)a.B, a.ldb);
  const int64_t nk = ceil_div(a.K, 64);
  if (nk > 0) {
    gload(0, a.K);
    sstore(0);
  }
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nk) gload((kt + 1) * 64, a.K);
    const char* As = lds + cur * STAGE;
    const char* Bs = As + BM * 64;
    v4i fa[MI], fb[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[i] = *(const v4i*)(As + (wm0 + i * 16) * 64 + lo);
#pragma unroll
    for (int j = 0; j < NI; ++j) fb[j] = *(const v4i*)(Bs + (wn0 + j * 16) * 64 + lo);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  const int lrow = 4 * (lane >> 4);  // first of the 4 channels this lane holds
  const int lcol = lane & 15;        // token within a 16-wide block

  if constexpr (!FUSED) {
    const bool cvec = ((a.N & 3) == 0) && ((((uintptr_t)a.C) & 15) == 0);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t f = m0 + wm0 + i * 16 + lrow;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int64_t t = n0 + wn0 + j * 16 + lcol;
        if (t >= a.T) continue;
        int32_t* dst = a.C + t * a.N + f;
        if (cvec && f + 3 < a.N) {
          *(v4i*)dst = acc[i][j];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (f + r < a.N) dst[r] = acc[i][j][r];
        }
      }
    }
    return;
  } else {
    // ---- dequantize in registers: acc * sx[i] * SCB[j] / 127^2 ----
    float sxv[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t t = n0 + wn0 + j * 16 + lcol;
      sxv[j] = (t < a.T) ? a.sx[t] : 0.0f;
    }
    // the fp32 values reuse the int32 accumulator storage (bit casts), so one
    // 256-register array lives in the accumulation registers throughout
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t f = m0 + wm0 + i * 16 + lrow + r;
        sc[r] = (f < a.N) ? a.SCB[f] * (1.0f / 16129.0f) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        v4f v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (float)acc[i][j][r] * (sxv[j] * sc[r]);
        acc[i][j] = __builtin_bit_cast(v4i, v);
      }
    }

    // ---- fp16 product over the outlier columns, same registers ----
    const int64_t n_o = a.counts[0];
    const int64_t n_use = n_o < a.max_o ? n_o : a.max_o;
    const int64_t nt = ceil_div(n_use, 32);  // 32 halves = 64 bytes per slice
    if (nt > 0) {
      const int64_t Kb = nt * 64;
      setup((const char*)a.Wo, a.ldo * 2, (const char*)a.Xo, a.ldo * 2);
      gload(0, Kb);
      sstore(0);
      __syncthreads();
      for (int64_t kt = 0; kt < nt; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nt) gload((kt + 1) * 64, Kb);
        const char* As = lds + cur * STAGE;
        const char* Bs = As + BM * 64;
        v8h fa[MI], fb[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = *(const v8h*)(As + (wm0 + i * 16) * 64 + lo);
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[j] = *(const v8h*)(Bs + (wn0 + j * 16) * 64 + lo);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
            acc[i][j] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb[j],
                                                            __builtin_bit_cast(v4f, acc[i][j]), 0, 0, 0));
        if (kt + 1 < nt) sstore(cur ^ 1);
        __syncthreads();
      }
    }

    // ---- bias, fp16 round-to-nearest-even, store ----
    // (zero-point activations: plus the offset part of the int8 product,
    // (sx Z / 127) (SCB (rsum - osum) / 127), a rank-1 fp32 term)
    const bool yvec = ((a.N & 3) == 0) && ((((uintptr_t)a.Y) & 7) == 0);
    float ut[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t t = n0 + wn0 + j * 16 + lcol;
      ut[j] = (a.zp && t < a.T) ? a.sx[t] * (float)a.zp[t] * (1.0f / 127.0f) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t f = m0 + wm0 + i * 16 + lrow;
      float bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = (a.bias && f + r < a.N) ? h2f(a.bias[f + r]) : 0.0f;
      float vr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vr[r] = (a.zp && f + r < a.N)
                    ? a.SCB[f + r] * (float)(a.rsum[f + r] - (nt > 0 ? a.osum[f + r] : 0)) *
                          (1.0f / 127.0f)
                    : 0.0f;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int64_t t = n0 + wn0 + j * 16 + lcol;
        if (t >= a.T) continue;
        _Float16* dst = a.Y + t * a.N + f;
        const v4f v = __builtin_bit_cast(v4f, acc[i][j]);
        v4h y;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          y[r] = (_Float16)(a.zp ? v[r] + bv[r] + ut[j] * vr[r] : v[r] + bv[r]);
        if (yvec && f + 3 < a.N) {
          *(v4h*)dst = y;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (f + r < a.N) dst[r] = y[r];
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool FUSED>
static hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
  const int64_t ntiles = ceil_div(a.N, BM) * ceil_div(a.T, BN);
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  constexpr size_t LDS = 2 * (size_t)(BM + BN) * 64;
  const bool vec = (a.K % 16 == 0) && (a.lda % 16 == 0) && (a.ldb % 16 == 0) &&
                   ((((uintptr_t)a.A) & 15) == 0) && ((((uintptr_t)a.B) & 15) == 0);
  hipError_t e;
  if (vec) {
    auto kern = k_gemm<BM, BN, WM, WN, FUSED, true>;
    e = lds_limit<k_gemm<BM, BN, WM, WN, FUSED, true>>(LDS);
    if (e != hipSuccess) return e;
    kern<<<dim3((unsigned)ntiles), dim3(NT), LDS, st>>>(a);
  } else {
    auto kern = k_gemm<BM, BN, WM, WN, FUSED, false>;
    e = lds_limit<k_gemm<BM, BN, WM, WN, FUSED, false>>(LDS);
    if (e != hipSuccess) return e;
    kern<<<dim3((unsigned)ntiles), dim3(NT), LDS, st>>>(a);
  }
  return hipGetLastError();
}

// 256 x 256 tile, 8 waves of 128 x 64 (two waves per SIMD): the fused
// epilogue, with its in-register fp16 loop over any number of outlier
// columns, fits the register file without spilling at this wave tile.
hipError_t launch_gemm_fused(const GemmArgs& a, hipStream_t st) {
  return launch_cfg<256, 256, 128, 64, true>(a, st);
}

hipError_t launch_gemm_s32(const GemmArgs& a, hipStream_t st) {
  return launch_cfg<256, 256, 128, 64, false>(a, st);
}

}  // namespace i8mm
