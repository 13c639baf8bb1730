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
// Workgroup: 4 waves (one per SIMD), 256 x 256 output tile (channels x
// tokens), 128 x 128 per wave = 8 x 8 blocks of v_mfma_i32_16x16x64_i8.  K is
// walked in 64-byte slices; S slices are in flight in LDS, loaded with
// buffer_load_dwordx4 ... lds (no staging registers), so a slice is
// requested S slices ahead of its use.  Operand fragments are double-buffered in
// registers: while the 64 MFMAs of slice k issue, the 16 LDS reads of slice
// k+1 are interleaved between them.  One barrier per slice.
//
// LDS rows are 64 bytes (4 chunks of 16); chunk cc of row r sits at chunk
// cc ^ ((r>>1)&3).  Measured on gfx950 with the SQ_LDS_BANK_CONFLICT counter,
// this makes the fragment reads (16 consecutive rows x 4 chunks per wave)
// conflict-free at every row offset the kernel uses, ~4 LDS cycles per
// 16-byte-per-lane read; an XOR that also folds in bit 3 of the row costs
// twice that.  A load instruction writes 1 KB of LDS
// at consecutive lane addresses, so the swizzle is applied on the global side
// (lane i fetches the chunk that belongs at its LDS position).  Chunks past
// the end of K read as zeros, so any K that is a multiple of 16 is exact.
#include "common.h"
#include "kernels.h"

namespace i8mm {

namespace {

constexpr int MODE_I32 = 0, MODE_FUSED = 1, MODE_F16 = 2;

__device__ __forceinline__ int swz_off(int r, int cc) {
  return r * 64 + ((cc ^ ((r >> 1) & 3)) << 4);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

}  // namespace

template <int BM, int BN, int WM, int WN, int S, bool DBUF, int MODE>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void k_gemm_i8(GemmArgs a) {
  // The body uses amdgcn-only types (buffer resources); the host pass only
  // needs the kernel's signature to emit its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int NWN = BN / WN, NWAVE = (BM / WM) * NWN;
  constexpr int STAGE = (BM + BN) * 64;            // bytes of one slice
  constexpr int PW = (BM / 16 + BN / 16) / NWAVE;  // 1 KB load instructions per wave per slice
  static_assert((BM / 16 + BN / 16) % NWAVE == 0, "slice pieces must split evenly over waves");
  static_assert((BM / 16) % PW == 0, "each wave loads pieces of one operand only");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / NWN) * WM, wn0 = (wave % NWN) * WN;

  // the outlier-product launch only has work for a large outlier set
  int64_t nt_tail = 0;
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
  // offset, so a load costs no per-lane address arithmetic.  A chunk past the
  // end of K gets an offset beyond the buffer's range, which the hardware
  // reads as zeros.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[PW], vtail[PW];
  int kc[PW];
  auto setup = [&](const char* A, int64_t ldab, int64_t rowsA, const char* B, int64_t ldbb,
                   int64_t rowsB) {
    const bool isA = wv * PW < BM / 16;  // a wave's pieces are all A or all B
    const char* base = isA ? A : B;
    const int64_t ld = isA ? ldab : ldbb;
    const int64_t rows = isA ? rowsA : rowsB;
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(rows * ld), 0x00020000);
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int j = wv * PW + u;  // 1 KB piece: 16 rows of A, then of B
      const int rr = (isA ? j : j - BM / 16) * 16 + (lane >> 2);
      const int cc = (lane & 3) ^ ((rr >> 1) & 3);
      const int64_t g = isA ? min(m0 + rr, a.N - 1) : min(n0 + rr, a.T - 1);
      voff[u] = (uint32_t)(g * ld + cc * 16);
      kc[u] = cc * 16;
    }
  };
  auto lds_dst = [&](int buf, int u) {
    const int j = wv * PW + u;
    const int off = (j < BM / 16) ? j * 1024 : BM * 64 + (j - BM / 16) * 1024;
    return (__attribute__((address_space(3))) void*)(lds + buf * STAGE + off);
  };
  auto issue = [&](int buf, int64_t k0, int64_t Kb) {
    if (k0 + 64 <= Kb) {
#pragma unroll
      for (int u = 0; u < PW; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_dst(buf, u), 16, voff[u], (int)k0, 0, 0);
    } else {
#pragma unroll
      for (int u = 0; u < PW; ++u) {
        const uint32_t vo = (k0 + kc[u] < Kb) ? voff[u] : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_dst(buf, u), 16, vo, (int)k0, 0, 0);
      }
    }
  };
  const int lo = swz_off(lane & 15, lane >> 4);

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
  auto read_frags = [&](int buf, v4i (&fa)[MI], v4i (&fb)[NI]) {
    const char* As = lds + buf * STAGE;
    const char* Bs = As + BM * 64;
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[i] = *(const v4i*)(As + (wm0 + i * 16) * 64 + lo);
#pragma unroll
    for (int j = 0; j < NI; ++j) fb[j] = *(const v4i*)(Bs + (wn0 + j * 16) * 64 + lo);
  };
  // 64 MFMAs on (ca, cb); one LDS read of the next slice after every 4th
  auto step = [&](const v4i (&ca)[MI], const v4i (&cb)[NI], v4i (&na)[MI], v4i (&nb)[NI],
                  int nbuf) {
    const char* As = lds + nbuf * STAGE;
    const char* Bs = As + BM * 64;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        mfma(i, j, ca[i], cb[j]);
        if ((j & 3) == 3) {
          const int f = (i * NI + j) >> 2;
          if (f < MI)
            na[f] = *(const v4i*)(As + (wm0 + f * 16) * 64 + lo);
          else
            nb[f - MI] = *(const v4i*)(Bs + (wn0 + (f - MI) * 16) * 64 + lo);
        }
      }
    }
  };
  auto last = [&](const v4i (&ca)[MI], const v4i (&cb)[NI]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) mfma(i, j, ca[i], cb[j]);
  };

  int64_t nk, Kb;
  if constexpr (MODE == MODE_F16) {
    setup((const char*)a.Wo, a.ldo * 2, a.N, (const char*)a.Xo, a.ldo * 2, a.T);
    nk = nt_tail;
    Kb = nt_tail * 64;
  } else {
    setup((const char*)a.A, a.lda, a.N, (const char*)a.B, a.ldb, a.T);
    nk = ceil_div(a.K, 64);
    Kb = a.K;
  }
  // make slice kt+1 visible to every wave and start loading slice kt+S into
  // the buffer slice kt used (its fragments are already in registers)
  auto sync_next = [&](int64_t kt) {
    wait_lgkm0();
    if (kt + S - 1 <= nk - 1)
      wait_vm<(S - 2) * PW>();
    else
      wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + S < nk) issue((int)(kt % S), (kt + S) * 64, Kb);
  };

  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s < nk) issue(s, s * 64, Kb);
    if (nk >= S)
      wait_vm<(S - 1) * PW>();
    else
      wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (DBUF) {
      // fragments double-buffered in registers: the reads of slice k+1
      // interleave with the MFMAs of slice k
      v4i fa0[MI], fb0[NI], fa1[MI], fb1[NI];
      read_frags(0, fa0, fb0);
      int64_t kt = 0;
      for (; kt + 2 < nk; kt += 2) {
        sync_next(kt);
        step(fa0, fb0, fa1, fb1, (int)((kt + 1) % S));
        sync_next(kt + 1);
        step(fa1, fb1, fa0, fb0, (int)((kt + 2) % S));
      }
      if (nk - kt == 2) {
        sync_next(kt);
        step(fa0, fb0, fa1, fb1, (int)((kt + 1) % S));
        last(fa1, fb1);
      } else {
        last(fa0, fb0);
      }
    } else {
      // one fragment set; the other waves of the SIMD cover the LDS latency
      for (int64_t kt = 0; kt < nk; ++kt) {
        if (kt > 0) {
          // slice kt must have landed; the buffer of slice kt-1 is free
          if (kt + S - 2 <= nk - 1)
            wait_vm<(S - 2) * PW>();
          else
            wait_vm<0>();
          __builtin_amdgcn_s_barrier();
          if (kt - 1 + S < nk) issue((int)((kt - 1) % S), (kt - 1 + S) * 64, Kb);
        }
        v4i fa[MI], fb[NI];
        read_frags((int)(kt % S), fa, fb);
        last(fa, fb);
      }
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
    // small outlier sets: stage Xo/Wo (<= S slices of 32 columns) in LDS and
    // run the fp16 MFMAs per output block into a fresh accumulator; large
    // ones: the fp32 product P was written by the MODE_F16 launch before.
    const bool small = nt_tail <= kSmallTail / 32;
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();  // every wave is done with the int8 slices
    if (small && nt_tail > 0) {
      setup((const char*)a.Wo, a.ldo * 2, a.N, (const char*)a.Xo, a.ldo * 2, a.T);
      static_assert(S * 32 >= kSmallTail, "the small tail must fit the slice buffers");
      for (int s = 0; s < S; ++s)
        if (s < nt_tail) issue(s, s * 64, nt_tail * 64);
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
      for (int i = 0; i < MI; ++i) ta[i] = *(const v8h*)(lds + (wm0 + i * 16) * 64 + lo);
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int64_t t = n0 + wn0 + j * 16 + lcol;
      v8h tb = {};
      if (small && nt_tail == 1) tb = *(const v8h*)(lds + BM * 64 + (wn0 + j * 16) * 64 + lo);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int64_t f = m0 + wm0 + i * 16 + lrow;
        v4f p = {0.0f, 0.0f, 0.0f, 0.0f};
        if (small) {
          if (nt_tail == 1) {
            p = __builtin_amdgcn_mfma_f32_16x16x32_f16(ta[i], tb, p, 0, 0, 0);
          } else {
            for (int64_t s = 0; s < nt_tail; ++s) {
              const char* base = lds + s * STAGE;
              const v8h xa = *(const v8h*)(base + (wm0 + i * 16) * 64 + lo);
              const v8h xb = *(const v8h*)(base + BM * 64 + (wn0 + j * 16) * 64 + lo);
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
#define I8MM_CFG 3
#endif

namespace {
template <int BM, int BN, int WM, int WN, int S, bool DBUF, int MODE>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  constexpr size_t LDS = (size_t)S * (BM + BN) * 64;
  hipError_t e = hipFuncSetAttribute((const void*)k_gemm_i8<BM, BN, WM, WN, S, DBUF, MODE>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS);
  if (e != hipSuccess) return e;
  const int64_t ntiles = ceil_div(a.N, BM) * ceil_div(a.T, BN);
  k_gemm_i8<BM, BN, WM, WN, S, DBUF, MODE><<<dim3((unsigned)ntiles), dim3(NT), LDS, st>>>(a);
  return hipGetLastError();
}

// tile configurations: channels x tokens per workgroup, per wave, slices in
// flight, register double-buffering of fragments.  Configuration 3 (256 x 256,
// 8 waves of 64 x 128, 4 slices, single-buffered) measured fastest on the
// first feed-forward shapes.
template <int MODE>
hipError_t launch_mode(const GemmArgs& a, hipStream_t st) {
#if I8MM_CFG == 0
  return launch_cfg<256, 256, 128, 64, 4, false, MODE>(a, st);
#elif I8MM_CFG == 1
  return launch_cfg<256, 256, 128, 128, 4, true, MODE>(a, st);
#elif I8MM_CFG == 3
  return launch_cfg<256, 256, 64, 128, 4, false, MODE>(a, st);
#elif I8MM_CFG == 4
  return launch_cfg<256, 128, 128, 64, 3, false, MODE>(a, st);
#elif I8MM_CFG == 5
  return launch_cfg<256, 256, 128, 64, 3, false, MODE>(a, st);
#elif I8MM_CFG == 6
  return launch_cfg<128, 256, 64, 128, 3, false, MODE>(a, st);
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
