// The int8 product of the LLM.int8() layer, tuned for gfx950 (16-byte
// aligned operands), and the fp16 product over a large outlier set.
//
// Step 2 of "LLM.int8() の核心アイデア" (Hugging Face summary page) multiplies
// the non-outlier dims in int8 and the outlier dims in fp16; step 3
// dequantizes the int8 result and adds the fp16 one.  Here:
//
//   k_gemm_i8<..., MODE_I32>    C = Xq . CB^T (exact int32)
//   k_gemm_i8<..., MODE_FUSED>  Y = fp16(acc*sx*SCB/127^2 + Xo.Wo^T + bias)
//   k_gemm_i8<..., MODE_F16>    P = Xo . Wo^T in fp32, only when the outlier
//                                   set is too large for the fused epilogue
//                                   (more than kSmallTail columns)
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
#include "common.h"
#include "kernels.h"

namespace i8mm {

namespace {

constexpr int MODE_I32 = 0, MODE_FUSED = 1, MODE_F16 = 2;

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

  // the outlier-product launch only has work for a large outlier set
  int64_t nt_tail = 0;  // 32-column (64-byte) k-steps of the outlier operands
  if constexpr (MODE != MODE_I32) {
    const int64_t n_o = a.counts[0];
    const int64_t n_use = n_o < a.max_o ? n_o : a.max_o;
    nt_tail = ceil_div(n_use, 32);
    if constexpr (MODE == MODE_F16) {
      if (nt_tail <= kSmallTail / 32) return;
    }
  }

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
  int kc[PW];
  auto setup = [&](const char* A, int64_t ldab, int64_t rowsA, const char* B, int64_t ldbb,
                   int64_t rowsB) {
    rsA = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)(rowsA * ldab), 0x00020000);
    rsB = __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, (int)(rowsB * ldbb), 0x00020000);
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int j = wv * PW + u;  // piece: RPP rows of A, then of B (wave-uniform)
      const bool isA = j < ACH;
      const int rr = (isA ? j : j - ACH) * RPP + lane / CPR;
      const int c = (lane % CPR) ^ swz<KB>(rr);
      const int64_t g = isA ? min(m0 + rr, a.N - 1) : min(n0 + rr, a.T - 1);
      voff[u] = (uint32_t)(g * (isA ? ldab : ldbb) + c * 16);
      kc[u] = c * 16;
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
        const uint32_t vo = (k0 + kc[u] < Kb) ? voff[u] : 0x80000000u;
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

  auto mfma = [&](int i, int j, v4i x, v4i y) {
    if constexpr (MODE == MODE_F16) {
      acc[i][j] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x),
                                                      __builtin_bit_cast(v8h, y),
                                                      __builtin_bit_cast(v4f, acc[i][j]), 0, 0, 0));
    } else {
      acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x, y, acc[i][j], 0, 0, 0);
    }
  };
  // the MFMAs of one slice; the other waves of the SIMD cover LDS latency
  auto compute = [&](int buf) {
    const char* As = lds + buf * STAGE;
    const char* Bs = As + BM * KB;
#pragma unroll
    for (int h = 0; h < KS; ++h) {
      v4i fa[MI], fb[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[i] = *(const v4i*)(As + frag_off(wm0 + i * 16, h));
#pragma unroll
      for (int j = 0; j < NI; ++j) fb[j] = *(const v4i*)(Bs + frag_off(wn0 + j * 16, h));
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) mfma(i, j, fa[i], fb[j]);
    }
  };

  int64_t Kb;
  if constexpr (MODE == MODE_F16) {
    setup((const char*)a.Wo, a.ldo * 2, a.N, (const char*)a.Xo, a.ldo * 2, a.T);
    Kb = nt_tail * 64;
  } else {
    setup((const char*)a.A, a.lda, a.N, (const char*)a.B, a.ldb, a.T);
    Kb = a.K;
  }
  const int64_t nk = ceil_div(Kb, KB);

  if (nk > 0) {
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
      compute((int)(kt % S));
    }
  }

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
  } else if constexpr (MODE == MODE_F16) {
    const bool pvec = ((a.N & 3) == 0) && ((((uintptr_t)a.P) & 15) == 0);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int64_t f = m0 + wm0 + i * 16 + lrow;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int64_t t = n0 + wn0 + j * 16 + lcol;
        if (t >= a.T) continue;
        float* dst = a.P + t * a.N + f;
        const v4f v = __builtin_bit_cast(v4f, acc[i][j]);
        if (pvec && f + 3 < a.N) {
          *(v4f*)dst = v;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (f + r < a.N) dst[r] = v[r];
        }
      }
    }
  } else {
    // ---- fused epilogue ----
    // small outlier sets: stage Xo/Wo (<= kSmallTail columns) in LDS and run
    // the fp16 MFMAs per output block into a fresh accumulator; large ones:
    // the fp32 product P was written by the MODE_F16 launch before.
    const bool small = nt_tail <= kSmallTail / 32;
    const int64_t Kt = nt_tail * 64;        // bytes of a tail row
    const int ntl = (int)ceil_div(Kt, KB);  // tail slices
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();  // every wave is done with the int8 slices
    if (small && nt_tail > 0) {
      static_assert(S * KB >= kSmallTail * 2, "the small tail must fit the slice buffers");
      setup((const char*)a.Wo, a.ldo * 2, a.N, (const char*)a.Xo, a.ldo * 2, a.T);
      for (int s = 0; s < S; ++s)
        if (s < ntl) issue(s, s * KB, Kt);
      wait_vm<0>();
      __builtin_amdgcn_s_barrier();
    }
    float sxv[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t t = n0 + wn0 + j * 16 + lcol;
      sxv[j] = (t < a.T) ? a.sx[t] : 0.0f;
    }
    const bool yvec = ((a.N & 3) == 0) && ((((uintptr_t)a.Y) & 7) == 0);
    const bool pvec = ((a.N & 3) == 0) && ((((uintptr_t)a.P) & 15) == 0);
    float scv[MI][4], bvv[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t f = m0 + wm0 + i * 16 + lrow + r;
        const bool in = f < a.N;
        scv[i][r] = in ? a.SCB[f] * (1.0f / 16129.0f) : 0.0f;
        bvv[i][r] = (a.bias && in) ? h2f(a.bias[f]) : 0.0f;
      }
    v8h ta[MI];
    if (small && nt_tail == 1) {
#pragma unroll
      for (int i = 0; i < MI; ++i) ta[i] = *(const v8h*)(lds + frag_off(wm0 + i * 16, 0));
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t t = n0 + wn0 + j * 16 + lcol;
      v8h tb = {};
      if (small && nt_tail == 1) tb = *(const v8h*)(lds + BM * KB + frag_off(wn0 + j * 16, 0));
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int64_t f = m0 + wm0 + i * 16 + lrow;
        v4f p = {0.0f, 0.0f, 0.0f, 0.0f};
        if (small) {
          if (nt_tail == 1) {
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(ta[i], tb, p, 0, 0, 0);
          } else {
            for (int64_t q = 0; q < nt_tail; ++q) {  // 64-byte k-steps of the tail
              const char* base = lds + (int)(q / KS) * STAGE;
              const int h = (int)(q % KS);
              const v8h xa = *(const v8h*)(base + frag_off(wm0 + i * 16, h));
              const v8h xb = *(const v8h*)(base + BM * KB + frag_off(wn0 + j * 16, h));
              p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, xb, p, 0, 0, 0);
            }
          }
        } else if (t < a.T) {
          const float* src = a.P + t * a.N + f;
          if (pvec && f + 3 < a.N) {
            p = *(const v4f*)src;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = (f + r < a.N) ? src[r] : 0.0f;
          }
        }
        if (t >= a.T) continue;
        v4h y;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          y[r] = (_Float16)((float)acc[i][j][r] * (sxv[j] * scv[i][r]) + p[r] + bvv[i][r]);
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

#ifndef I8MM_CFG
#define I8MM_CFG 20
#endif

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

// tile configurations: channels x tokens per workgroup, per wave, slices in
// flight, slice bytes per row.  Configuration 20 (256 x 256, 8 waves of
// 64 x 128, two 128-byte slices in flight, 128 KB of LDS) measured fastest
// on the first feed-forward shapes (13B: 242 us against 275 us for the
// 64-byte, four-slice configuration 3).
template <int MODE>
hipError_t launch_mode(const GemmArgs& a, hipStream_t st) {
#if I8MM_CFG == 3
  return launch_cfg<256, 256, 64, 128, 4, 64, MODE>(a, st);
#elif I8MM_CFG == 20
  return launch_cfg<256, 256, 64, 128, 2, 128, MODE>(a, st);
#elif I8MM_CFG == 21
  return launch_cfg<256, 128, 64, 64, 3, 128, MODE>(a, st);
#elif I8MM_CFG == 22
  return launch_cfg<256, 256, 128, 64, 2, 128, MODE>(a, st);
#elif I8MM_CFG == 23
  return launch_cfg<128, 256, 64, 64, 3, 128, MODE>(a, st);
#elif I8MM_CFG == 24
  return launch_cfg<256, 256, 64, 64, 2, 128, MODE>(a, st);
#else
#error "unknown I8MM_CFG"
#endif
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
  // the fp16 product of a large outlier set first (returns at once otherwise)
  hipError_t e = launch_mode<MODE_F16>(a, st);
  if (e != hipSuccess) return e;
  return launch_mode<MODE_FUSED>(a, st);
}

}  // namespace i8mm
