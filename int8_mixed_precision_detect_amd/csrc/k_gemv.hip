// The LLM.int8() product for few tokens (decode: T <= 32), gfx950.
//
// Step 2 of "LLM.int8() の核心アイデア" (Hugging Face summary page): the
// non-outlier dims in int8, the outlier dims in fp16; step 3 adds them after
// dequantizing.  With T <= 32 the work is reading CB once from HBM: 2*T ops
// per weight byte, far below what int8 MFMA can absorb, so this kernel is
// built to stream CB, not to fill matrix cores.
//
// One wave per workgroup owns 16*FA output channels (FA 16-row A fragments
// of v_mfma_i32_16x16x64_i8) over all of K, and all T tokens (NB 16-token B
// fragments, Xq read through L2: it is T*K bytes, re-read by every wave).
// CB goes straight from HBM into the A-fragment registers with 16-byte
// buffer loads, U k-steps (64 bytes of K each) in flight in a ring of
// registers.  Loads past the end of K are still issued, with out-of-range
// offsets: they return zeros without touching memory, so every wait in the
// loop is the same constant.
//
// The outlier weights need no separate pass for small outlier sets: O is
// ascending, so while a k-step's CB bytes sit in registers the wave checks
// whether the next outlier column falls inside it; the 16 lanes holding that
// column (one per row) dequantize their byte, fp16(fl32(fl32(c*SCB)/127)),
// into an LDS row of Wo (also written to the workspace's Wo rows, as the
// other product paths leave them).  After the int8 loop the accumulators are scaled to
// fp32 (acc*sx*SCB/127^2) and the fp16 outlier product runs into them with
// v_mfma_f32_16x16x32_f16 (Xo from the step-2 kernel, Wo from LDS); then
// bias and one fp16 rounding.  Larger outlier sets take Wo from the
// workspace, where the step-2 kernel built it.
#include "common.h"
#include "kernels.h"

namespace i8mm {

namespace {
constexpr int kU = 8;  // k-steps in flight

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
}  // namespace

// FA 16-row A fragments (output channels) per wave, NB 16-token B fragments
template <int FA, int NB, bool FUSED>
__global__ __launch_bounds__(64) void k_gemv_i8(GemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int kRows = 16 * FA;  // output channels per wave
  constexpr int LPS = FA + NB;    // loads per k-step
  static_assert((kU - 1) * LPS < 64, "loads in flight");
  __shared__ _Float16 swo[kRows][kGemvOcap + 8];  // dequantized outlier weights
  __shared__ int32_t sO[kGemvOcap];
  const int lane = threadIdx.x;
  const int lr = lane & 15, lq = lane >> 4;
  const int64_t j0 = (int64_t)blockIdx.x * kRows;
  const int64_t rows = min((int64_t)kRows, a.N - j0);

  // A: CB rows j0 .. j0+rows-1 (rows past N read 0); B: Xq rows 0..T-1
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(a.A + j0 * a.lda, (uint32_t)(rows * a.lda));
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(a.B, (uint32_t)(a.T * a.ldb));
  uint32_t vA[FA], vB[NB];
#pragma unroll
  for (int f = 0; f < FA; ++f) vA[f] = (uint32_t)((lr + 16 * f) * a.lda + 16 * lq);
#pragma unroll
  for (int b = 0; b < NB; ++b) vB[b] = (uint32_t)((lr + 16 * b) * a.ldb + 16 * lq);
  const int64_t nsteps = ceil_div(a.K, 64);
  const uint32_t kOOB = 0x80000000u;

  // outlier list for the in-loop Wo extraction
  int64_t n_use = 0;
  bool inloop = false;
  if constexpr (FUSED) {
    const int64_t n_o = a.counts[0];
    n_use = n_o < a.max_o ? n_o : a.max_o;
    inloop = n_use <= kGemvOcap;
    if (inloop)
      for (int64_t o = lane; o < n_use; o += 64) sO[o] = a.O[o];
  }

  // Every wave walks the k-steps in rotated order, starting at s_rot: the
  // waves of an XCD would otherwise request the same Xq lines at the same
  // moment (one L2 channel serving them all); the int32 sums do not depend
  // on the order.  Step number s (0 .. nsteps-1 in walking order) is k-step
  // kstep(s) = (s_rot + s) mod nsteps.
  const int64_t s_rot = nsteps > 0 ? ((int64_t)(blockIdx.x >> 3) * 37) % nsteps : 0;
  auto kstep = [&](int64_t s) { return s_rot + s < nsteps ? s_rot + s : s_rot + s - nsteps; };

  v4i ring[kU][LPS];
  auto issue = [&](int slot, int64_t s) {
    // a lane's 16 bytes sit at k = 64 kstep(s) + 16 lq; past K, and for the
    // steps past the end of the walk, they read as zero
    const int64_t ks = kstep(s);
    const int64_t k = 64 * ks + 16 * lq;
    const bool in = s < nsteps && k < a.K;
#pragma unroll
    for (int f = 0; f < FA; ++f)
      ring[slot][f] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(rsA, in ? vA[f] + (uint32_t)(64 * ks) : kOOB,
                                                     0, 0));
#pragma unroll
    for (int b = 0; b < NB; ++b)
      ring[slot][FA + b] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(rsB, in ? vB[b] + (uint32_t)(64 * ks) : kOOB,
                                                     0, 0));
  };

  v4i acc[FA][NB];
#pragma unroll
  for (int f = 0; f < FA; ++f)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[f][b] = v4i{0, 0, 0, 0};

  float sj[FA] = {};           // SCB of the rows this lane holds in A
  int64_t nxt = 0;             // next outlier (index into sO) not yet extracted
  int nextc = 0x7fffffff;      // its column (wave-uniform)
  if constexpr (FUSED) {
#pragma unroll
    for (int f = 0; f < FA; ++f) sj[f] = lr + 16 * f < rows ? a.SCB[j0 + lr + 16 * f] : 0.0f;
    __syncthreads();  // sO visible
    if (inloop) {
      // the walk starts at k-step s_rot: first outlier at or after it
      while (nxt < n_use && sO[nxt] < 64 * s_rot) ++nxt;
      nextc = nxt < n_use ? __builtin_amdgcn_readfirstlane(sO[nxt]) : 0x7fffffff;
    }
  }

#pragma unroll
  for (int u = 0; u < kU; ++u) issue(u, u);
  // steps past the end hold zeros (their loads were out of range), so the
  // loop runs whole groups of kU steps without a per-step test
  for (int64_t s0 = 0; s0 < nsteps; s0 += kU) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t s = s0 + u;
      // step s landed: the (kU-1) steps issued after it may stay in flight
      wait_vm<(kU - 1) * LPS>();
#pragma unroll
      for (int f = 0; f < FA; ++f)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[f][b] =
              __builtin_amdgcn_mfma_i32_16x16x64_i8(ring[u][f], ring[u][FA + b], acc[f][b], 0, 0, 0);
      if constexpr (FUSED) {
        // outlier columns inside this k-step (rare): pick their CB bytes
        const int ks = (int)kstep(s);
        if (s_rot > 0 && ks == 0 && inloop) {
          // the walk wrapped to column 0: the outliers before s_rot remain
          nxt = 0;
          nextc = n_use > 0 ? __builtin_amdgcn_readfirstlane(sO[0]) : 0x7fffffff;
        }
        if (s < nsteps && nextc < 64 * ks + 64) {
          do {
            const int off = nextc - 64 * ks;  // 0..63
            if (lq == (off >> 4)) {
              const int sh = 8 * (off & 3), wsel = (off >> 2) & 3;
#pragma unroll
              for (int f = 0; f < FA; ++f) {
                const int cb = (int)(int8_t)(ring[u][f][wsel] >> sh);
                swo[lr + 16 * f][nxt] = dequant_weight(cb, sj[f]);
              }
            }
            ++nxt;
            nextc = nxt < n_use ? __builtin_amdgcn_readfirstlane(sO[nxt]) : 0x7fffffff;
          } while (nextc < 64 * ks + 64);
        }
      }
      issue(u, s + kU);
    }
  }
  wait_vm<0>();

  const int lrow = 4 * lq;  // first of the 4 channels a lane holds in D
  const int lcol = lr;      // token within a 16-token block
  if constexpr (!FUSED) {
#pragma unroll
    for (int f = 0; f < FA; ++f) {
      const int64_t j = j0 + 16 * f + lrow;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int64_t t = 16 * b + lcol;
        if (t >= a.T) continue;
        int32_t* dst = a.C + t * a.N + j;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j + r < a.N) dst[r] = acc[f][b][r];
      }
    }
  } else {
    // int32 -> fp32 acc * sx * SCB / 127^2, in place
    float sxv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) sxv[b] = 16 * b + lcol < a.T ? a.sx[16 * b + lcol] : 0.0f;
#pragma unroll
    for (int f = 0; f < FA; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t j = j0 + 16 * f + lrow + r;
        const float sc = j < a.N ? a.SCB[j] * (1.0f / 16129.0f) : 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[f][b][r] = __builtin_bit_cast(int, (float)acc[f][b][r] * (sxv[b] * sc));
      }
    // fp16 outlier product, 32 outlier columns (64 bytes of a row) a step
    const int64_t nt = ceil_div(n_use, 32);
    if (nt > 0) {
      if (inloop) {
        // zero the pad columns of this wave's Wo rows, then make the
        // extracted values visible to every lane
        for (int64_t o = n_use + lane; o < 32 * nt; o += 64)
#pragma unroll
          for (int rr = 0; rr < kRows; ++rr) swo[rr][o] = (_Float16)0.0f;
        __syncthreads();
        // the workspace keeps the same Wo rows as the other product paths
        const int64_t c8 = 4 * nt;  // 16-byte pieces of a row in use
        for (int64_t idx = lane; idx < kRows * c8; idx += 64) {
          const int64_t r = idx / c8, c = idx - r * c8;
          if (r < rows) *(v8h*)(a.Wo + (j0 + r) * a.ldo + 8 * c) = *(const v8h*)&swo[r][8 * c];
        }
      }
      const __amdgpu_buffer_rsrc_t rsX = make_rsrc(a.Xo, (uint32_t)(a.T * a.ldo * 2));
      const __amdgpu_buffer_rsrc_t rsW =
          make_rsrc(a.Wo + j0 * a.ldo, (uint32_t)(rows * a.ldo * 2));
      for (int64_t q = 0; q < nt; ++q) {
        v8h xb[NB], wa[FA];
#pragma unroll
        for (int b = 0; b < NB; ++b)
          xb[b] = __builtin_bit_cast(
              v8h, __builtin_amdgcn_raw_buffer_load_b128(
                       rsX, (uint32_t)(((lr + 16 * b) * a.ldo + 32 * q + 8 * lq) * 2), 0, 0));
#pragma unroll
        for (int f = 0; f < FA; ++f) {
          if (inloop) {
            wa[f] = *(const v8h*)&swo[lr + 16 * f][32 * q + 8 * lq];
          } else {
            wa[f] = __builtin_bit_cast(
                v8h, __builtin_amdgcn_raw_buffer_load_b128(
                         rsW, (uint32_t)(((lr + 16 * f) * a.ldo + 32 * q + 8 * lq) * 2), 0, 0));
          }
        }
#pragma unroll
        for (int f = 0; f < FA; ++f)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            acc[f][b] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_mfma_f32_16x16x32_f16(
                         wa[f], xb[b], __builtin_bit_cast(v4f, acc[f][b]), 0, 0, 0));
      }
    }
    const bool yvec = ((a.N & 3) == 0) && ((((uintptr_t)a.Y) & 7) == 0);
#pragma unroll
    for (int f = 0; f < FA; ++f) {
      const int64_t j = j0 + 16 * f + lrow;
      float bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = (a.bias && j + r < a.N) ? h2f(a.bias[j + r]) : 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int64_t t = 16 * b + lcol;
        if (t >= a.T) continue;
        const v4f v = __builtin_bit_cast(v4f, acc[f][b]);
        v4h y;
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = (_Float16)(v[r] + bv[r]);
        _Float16* dst = a.Y + t * a.N + j;
        if (yvec && j + 3 < a.N) {
          *(v4h*)dst = y;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (j + r < a.N) dst[r] = y[r];
        }
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

bool gemv_i8_supported(const GemmArgs& a) {
  // 16-byte aligned rows; every offset the kernel forms fits 31 bits
  const int64_t lim = (int64_t)1 << 31;
  return a.T >= 1 && a.T <= kGemvMaxT && (a.K % 16 == 0) && (a.lda % 16 == 0) &&
         (a.ldb % 16 == 0) && ((((uintptr_t)a.A) & 15) == 0) && ((((uintptr_t)a.B) & 15) == 0) &&
         64 * a.lda + ceil_div(a.K, 64) * 64 + 64 * kU < lim && a.T * a.ldb < lim &&
         (a.ldo * 2) % 16 == 0 && a.T * a.ldo * 2 < lim && 64 * a.ldo * 2 < lim;
}

namespace {
template <bool FUSED>
hipError_t launch_gemv(const GemmArgs& a, hipStream_t st) {
  // 64 channels a wave: each Xq fragment read from L2 serves 4 weight
  // fragments (Xq is re-read by every wave, T*K bytes each time).  On the
  // 175B-width decode shapes (K = 12288, N = 49152) this measured 120 / 126
  // / 156 us for T = 1 / 8 / 32 against 123 / 135 / 194 us with 32 channels.
  constexpr int FA = 4;
  const dim3 g((unsigned)ceil_div(a.N, 16 * FA)), b(64);
  if (a.T <= 16)
    k_gemv_i8<FA, 1, FUSED><<<g, b, 0, st>>>(a);
  else
    k_gemv_i8<FA, 2, FUSED><<<g, b, 0, st>>>(a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemv_i8_fused(const GemmArgs& a, hipStream_t st) { return launch_gemv<true>(a, st); }
hipError_t launch_gemv_i8_s32(const GemmArgs& a, hipStream_t st) { return launch_gemv<false>(a, st); }

}  // namespace i8mm
