// The products of the LLM.int8() layer, tuned for gfx950 (16-byte aligned
// operands).
//
// Step 2 of "LLM.int8() の核心アイデア" (Hugging Face summary page) multiplies
// the non-outlier dims in int8 and the outlier dims in fp16; step 3
// dequantizes the int8 result and adds the fp16 one.  Here:
//
//   k_gemm_i8<..., MODE_I32>    C = Xq . CB^T (exact int32)
//   k_gemm_i8<..., MODE_FUSED>  Y = fp16(acc*sx*SCB/127^2 + Xo.Wo^T + bias):
//       the int8 slices of K, then the accumulators are scaled to fp32 in
//       place and the fp16 outlier slices (Xo/Wo rows, 64 halves a slice)
//       stream through the same LDS pipeline into them with
//       v_mfma_f32_16x16x32_f16, then bias and one fp16 rounding.
//
// Workgroup: a BM x BN output tile (channels x tokens) split over waves of
// WM x WN, each an array of 16 x 16 v_mfma_i32_16x16x64_i8 blocks.  K is
// walked in slices of KB bytes per row (KB/64 MFMA k-steps each); S slices
// are in flight in LDS, loaded with buffer_load_dwordx4 ... lds (no staging
// registers), one barrier per slice.
//
// Load efficiency: a load instruction fills 1 KB of LDS, i.e. 1024/KB rows
// of KB bytes.  With KB = 128 every instruction reads whole 128-byte lines;
// with 64-byte rows each instruction touches twice the lines for the same
// bytes, and the memory pipeline alone of that variant took ~190 us of a
// 261 us 13B-scale product.
//
// LDS rows are KB bytes (KB/16 chunks of 16); chunk c of row r sits at
// chunk c ^ sw(r), sw(r) = (r>>1)&3 for 64-byte rows, r&7 for 128-byte rows.
// Measured on gfx950 with the SQ_LDS_BANK_CONFLICT counter, both keep the
// fragment reads (16 consecutive rows x 4 chunks per wave) conflict-free at
// every row offset used here (~4 LDS cycles per 16-byte-per-lane read; an
// XOR that also folds in row bit 3 on 64-byte rows costs twice that).  A
// load instruction writes consecutive lane addresses, so the swizzle is
// applied on the global side: lane i fetches the chunk that belongs at its
// LDS position.  Chunks past the end of K read as zeros (their offset points
// past the buffer's range), so any K that is a multiple of 16 is exact.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace i8mm {

namespace {

constexpr int MODE_I32 = 0, MODE_FUSED = 1;
using I8Slices = std::false_type;
using F16Slices = std::true_type;

template <int KB>
__device__ __forceinline__ int swz(int r) {
  return KB == 64 ? ((r >> 1) & 3) : (r & 7);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// wait until at most n*PW of this wave's loads are outstanding (n < 4)
template <int PW>
__device__ __forceinline__ void wait_slices(int n) {
  if (n >= 3)
    wait_vm<3 * PW < 64 ? 3 * PW : 63>();
  else if (n == 2)
    wait_vm<2 * PW>();
  else if (n == 1)
    wait_vm<PW>();
  else
    wait_vm<0>();
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

}  // namespace

template <int BM, int BN, int WM, int WN, int S, int KB, int MODE>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm_i8(GemmArgs a) {
  // The body uses amdgcn-only types (buffer resources); the host pass only
  // needs the kernel's signature to emit its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int NWN = BN / WN, NWAVE = (BM / WM) * NWN;
  constexpr int STAGE = (BM + BN) * KB;          // bytes of one slice
  constexpr int RPP = 1024 / KB;                 // rows per 1 KB load instruction
  constexpr int CPR = KB / 16;                   // 16-byte chunks per row
  constexpr int ACH = BM / RPP, BCH = BN / RPP;  // load instructions per slice
  constexpr int PW = (ACH + BCH) / NWAVE;        // ... per wave
  constexpr int KS = KB / 64;                    // MFMA k-steps per slice
  static_assert(KB == 64 || KB == 128, "slice width");
  static_assert(S >= 2 && S <= 4 && (S - 1) * PW < 64, "slices in flight");
  static_assert((ACH + BCH) % NWAVE == 0, "slice pieces must split evenly over waves");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / NWN) * WM, wn0 = (wave % NWN) * WN;

  // tile order: workgroups are dealt to the 8 XCDs round-robin; give each XCD
  // a contiguous run of tiles, consecutive tiles sharing one weight tile.
  const int64_t tiles_m = ceil_div(a.N, BM), tiles_n = ceil_div(a.T, BN);
  const int64_t ntiles = tiles_m * tiles_n;
  int64_t bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  const int64_t tn = bid % tiles_n, tm = bid / tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  // Slice loads: buffer_load_dwordx4 ... lds.  The operand is a buffer
  // resource (base in SGPRs), a lane's 32-bit offset (row * ld + its chunk)
  // is fixed for the whole K loop and the K position goes in the scalar
  // offset, so a load costs no per-lane address arithmetic.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  __amdgpu_buffer_rsrc_t rsA, rsB;
  uint32_t voff[PW];
  // a lane's chunk within its row: rows of a piece start at multiples of
  // RPP (8 or 16), so the swizzle of row rr depends only on the lane
  const int kc = ((lane % CPR) ^ swz<KB>(lane / CPR)) * 16;
  auto setup = [&](const char* A, int64_t ldab, int64_t rowsA, const char* B, int64_t ldbb,
                   int64_t rowsB) {
    rsA = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)(rowsA * ldab), 0x00020000);
    rsB = __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, (int)(rowsB * ldbb), 0x00020000);
    // an opaque copy of the lane index: the row indices of a later setup
    // (the outlier operands index the same channels) are recomputed rather
    // than kept live across the K loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int j = wv * PW + u;  // piece: RPP rows of A, then of B (wave-uniform)
      const bool isA = j < ACH;
      const int rr = (isA ? j : j - ACH) * RPP + ln / CPR;
      static_assert(RPP % 8 == 0, "swizzle period");
      const int64_t g = isA ? min(m0 + rr, a.N - 1) : min(n0 + rr, a.T - 1);
      voff[u] = (uint32_t)(g * (isA ? ldab : ldbb) + kc);
    }
  };
  auto lds_dst = [&](int buf, int u) {
    const int j = wv * PW + u;
    const int off = (j < ACH) ? j * 1024 : BM * KB + (j - ACH) * 1024;
    return (__attribute__((address_space(3))) void*)(lds + buf * STAGE + off);
  };
  auto issue = [&](int buf, int64_t k0, int64_t Kb) {
    if (k0 + KB <= Kb) {
#pragma unroll
      for (int u = 0; u < PW; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wv * PW + u < ACH ? rsA : rsB, lds_dst(buf, u), 16,
                                                 voff[u], (int)k0, 0, 0);
    } else {
#pragma unroll
      for (int u = 0; u < PW; ++u) {
        const uint32_t vo = (k0 + kc < Kb) ? voff[u] : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wv * PW + u < ACH ? rsA : rsB, lds_dst(buf, u), 16,
                                                 vo, (int)k0, 0, 0);
      }
    }
  };
  // fragment of 16 rows at k-step h of a slice: lane -> row (lane & 15),
  // chunk (lane >> 4) + 4h
  const int lr = lane & 15;
  auto frag_off = [&](int row0, int h) {
    const int r = row0 + lr;
    return r * KB + ((((lane >> 4) + 4 * h) ^ swz<KB>(r)) << 4);
  };

  v4i acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  auto mma = [&](auto f16, int i, int j, v4i x, v4i y) {
    if constexpr (decltype(f16)::value) {
      acc[i][j] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x),
                                                      __builtin_bit_cast(v8h, y),
                                                      __builtin_bit_cast(v4f, acc[i][j]), 0, 0, 0));
    } else {
      acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x, y, acc[i][j], 0, 0, 0);
    }
  };
  // the MFMAs of one slice; the other waves of the SIMD cover LDS latency
  auto compute = [&](auto f16, int buf) {
    const char* As = lds + buf * STAGE;
    const char* Bs = As + BM * KB;
#pragma unroll
    for (int h = 0; h < KS; ++h) {
      if constexpr (MI * NI <= 32) {
        // small wave tile: the compiler schedules the fragment reads freely
        v4i fa[MI], fb[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = *(const v4i*)(As + frag_off(wm0 + i * 16, h));
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[j] = *(const v4i*)(Bs + frag_off(wn0 + j * 16, h));
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) mma(f16, i, j, fa[i], fb[j]);
      } else {
        // wide wave tile: token fragments once per k-step, channel fragments
        // one ahead of their NI MFMAs, in a fixed order, so that the live
        // fragments stay at NI + 2 registers of 4
        v4i fb[NI], fa0, fa1;
#pragma unroll
        for (int j = 0; j < NI; ++j) fb[j] = *(const v4i*)(Bs + frag_off(wn0 + j * 16, h));
        fa0 = *(const v4i*)(As + frag_off(wm0, h));
        __builtin_amdgcn_sched_group_barrier(0x100, NI + 1, 0);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (i + 1 < MI) {
            fa1 = *(const v4i*)(As + frag_off(wm0 + (i + 1) * 16, h));
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
#pragma unroll
          for (int j = 0; j < NI; ++j) mma(f16, i, j, fa0, fb[j]);
          __builtin_amdgcn_sched_group_barrier(0x008, NI, 0);
          fa0 = fa1;
        }
      }
    }
  };

  // K loop over Kb bytes of the operands set up last: S slices in flight,
  // one barrier per slice.  LDS must be free of earlier readers on entry.
  auto run = [&](auto f16, int64_t Kb) {
    const int64_t nk = ceil_div(Kb, KB);
    if (nk <= 0) return;
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s < nk) issue(s, s * KB, Kb);
    for (int64_t kt = 0; kt < nk; ++kt) {
      // Slice kt must have landed.  Issued so far: slices up to
      // min(kt + S - 2, nk - 1) (up to S - 1 before the loop); the ones
      // after kt may stay in flight.
      const int64_t last = kt == 0 ? (S - 1 < nk - 1 ? S - 1 : nk - 1)
                                   : (kt + S - 2 < nk - 1 ? kt + S - 2 : nk - 1);
      wait_slices<PW>((int)(last - kt));
      // one barrier: slice kt is visible to every wave, and every wave is
      // done with slice kt-1, whose buffer is refilled with slice kt-1+S
      __builtin_amdgcn_s_barrier();
      if (kt >= 1 && kt - 1 + S < nk) issue((int)((kt - 1) % S), (kt - 1 + S) * KB, Kb);
      compute(f16, (int)(kt % S));
      // keeps the epilogue's loads (scales, bias) below the loop instead of
      // hoisted above it, where they would hold registers throughout
      asm volatile("" ::: "memory");
    }
  };

  setup((const char*)a.A, a.lda, a.N, (const char*)a.B, a.ldb, a.T);
  run(I8Slices{}, a.K);

  const int lrow = 4 * (lane >> 4);  // first of the 4 channels a lane holds
  const int lcol = lane & 15;        // token within a 16-wide block

  if constexpr (MODE == MODE_I32) {
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
  } else {
    // ---- fused epilogue ----
    const int64_t n_o = a.counts[0];
    const int64_t n_use = n_o < a.max_o ? n_o : a.max_o;
    const int64_t Kt = round_up(n_use, 32) * 2;  // bytes of an Xo / Wo row in use
    float sxv[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t t = n0 + wn0 + j * 16 + lcol;
      sxv[j] = (t < a.T) ? a.sx[t] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t f = m0 + wm0 + i * 16 + lrow + r;
        const float sc = f < a.N ? a.SCB[f] * (1.0f / 16129.0f) : 0.0f;
        // int32 accumulator -> fp32 acc * sx * SCB / 127^2, in place
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j][r] = __builtin_bit_cast(int, (float)acc[i][j][r] * (sxv[j] * sc));
      }
    if (Kt > 0) {
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();  // every wave is done with the int8 slices
      setup((const char*)a.Wo, a.ldo * 2, a.N, (const char*)a.Xo, a.ldo * 2, a.T);
      run(F16Slices{}, Kt);
    }
    const bool yvec = ((a.N & 3) == 0) && ((((uintptr_t)a.Y) & 7) == 0);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t f = m0 + wm0 + i * 16 + lrow;  // 4 consecutive channels
      float bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = (a.bias && f + r < a.N) ? h2f(a.bias[f + r]) : 0.0f;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int64_t t = n0 + wn0 + j * 16 + lcol;
        if (t >= a.T) continue;
        const v4f v = __builtin_bit_cast(v4f, acc[i][j]);
        v4h y;
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = (_Float16)(v[r] + bv[r]);
        _Float16* dst = a.Y + t * a.N + f;
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
#endif  // __HIP_DEVICE_COMPILE__
}

namespace {
template <int BM, int BN, int WM, int WN, int S, int KB, int MODE>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  constexpr size_t LDS = (size_t)S * (BM + BN) * KB;
  hipError_t e = hipFuncSetAttribute((const void*)k_gemm_i8<BM, BN, WM, WN, S, KB, MODE>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS);
  if (e != hipSuccess) return e;
  const int64_t ntiles = ceil_div(a.N, BM) * ceil_div(a.T, BN);
  k_gemm_i8<BM, BN, WM, WN, S, KB, MODE><<<dim3((unsigned)ntiles), dim3(NT), LDS, st>>>(a);
  return hipGetLastError();
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Tile configurations (channels x tokens per workgroup, per wave, slices
// in flight, slice bytes per row), one workgroup per CU (LDS-bound):
//   A: 256 x 256, 8 waves of 64 x 128, two 128-byte slices (128 KB LDS)
//   B: 320 x 256, 8 waves of 80 x 128, two 128-byte slices (144 KB LDS)
// The workgroups run in waves of one per CU, so a launch costs about
// ceil(tiles / CUs) times the time of one tile.  The host takes the
// configuration with the smaller ceil(tiles / CUs) * tile area (ties go to
// A): on the 13B-scale layer (20480 x 2048 outputs) A needs 640 tiles, 2.5
// waves, and B 512 tiles, 2 full waves.
template <int MODE>
hipError_t launch_mode(const GemmArgs& a, hipStream_t st) {
  const int64_t cus = cu_count();
  auto cost = [&](int64_t bm, int64_t bn) {
    return ceil_div(ceil_div(a.N, bm) * ceil_div(a.T, bn), cus) * bm * bn;
  };
  if (cost(320, 256) < cost(256, 256)) return launch_cfg<320, 256, 80, 128, 2, 128, MODE>(a, st);
  return launch_cfg<256, 256, 64, 128, 2, 128, MODE>(a, st);
}
}  // namespace

bool gemm_i8_supported(const GemmArgs& a) {
  // 16-byte aligned rows, and every operand addressable with 31-bit offsets
  const int64_t lim = (int64_t)1 << 31;
  return (a.K % 16 == 0) && (a.lda % 16 == 0) && (a.ldb % 16 == 0) &&
         ((((uintptr_t)a.A) & 15) == 0) && ((((uintptr_t)a.B) & 15) == 0) &&
         ((a.ldo * 2) % 16 == 0) && a.N * a.lda < lim && a.T * a.ldb < lim &&
         a.N * a.ldo * 2 < lim && a.T * a.ldo * 2 < lim;
}

hipError_t launch_gemm_i8_s32(const GemmArgs& a, hipStream_t st) {
  return launch_mode<MODE_I32>(a, st);
}

hipError_t launch_gemm_i8_fused(const GemmArgs& a, hipStream_t st) {
  return launch_mode<MODE_FUSED>(a, st);
}

}  // namespace i8mm
