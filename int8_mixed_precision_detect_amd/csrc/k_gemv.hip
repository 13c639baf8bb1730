// The LLM.int8() product for one to four tokens on gfx950: the decode
// calls, where each weight byte is used once and the call lasts as long as
// the weight CB takes to stream from HBM.
//
// Step 2 of "LLM.int8() の核心アイデア" (Hugging Face summary page) multiplies
// the non-outlier dims in int8 and the outlier dims in fp16; step 3
// dequantizes the int8 result and adds the fp16 one.
//
// How fast HBM delivers a weight depends on how many bytes of each row one
// pass asks for.  Streaming 604 MB of weight rows (49152 x 12288) measured
// on MI355X: 87 us when every load instruction reads 1 KB of one row (the
// rate of a plain contiguous copy, 6.9 TB/s), 121 us with the 16-row x
// 128-byte slices of the tiled kernel, 140 us with MFMA-fragment-shaped
// loads (16 rows x 64 bytes an instruction).  So here a wave owns R channel
// rows and walks K in 1 KB pieces: each load instruction is one row's piece
// (lane l holds bytes 16l .. 16l+15), D pieces in flight in registers (no
// LDS), non-temporal.  The matching 16 bytes of each token's Xq row (small,
// L2-resident) come with each piece.  With that layout the products are
// VALU dot products (v_dot4 on int8: one instruction a lane per 4 codes and
// token), per-lane partial sums over the lane's columns; the 64 lanes' sums
// are added once, after the K loop, by a butterfly that leaves each lane one
// (channel, token) total.  int32 sums are exact in any order, so the int8
// part equals the MFMA one bit for bit.
//
// Outlier weights (up to kFewOcap columns): O is ascending, so a pointer
// follows the piece walk; for an outlier column in the current piece, the
// lane holding that byte copies it for its R rows to LDS.  After the loop
// the codes give Wo (dequantized, written to the workspace) and the fp16
// products sum_o X[t, o] Wo[j, o] in fp32, in increasing o.  Wider sets,
// and the layers whose step 2 already built Wo, stream Wo and Xo through
// the same loop with fp16 dot products instead -- except calls whose steps
// 1-2 ran as k_rows, which builds no Wo: their codes are gathered from CB
// after the loop, 128 columns at a time, and summed the same way as the
// extracted ones.
//
// Measured at 49152 x 12288 (HIP events around the product): 109 us at
// T = 1 and 116 us at T = 4 against 124 us for the tiled few-token kernel;
// from T = 6 on the tiled kernel is faster (the dot products grow with T,
// the MFMAs do not), so this kernel takes T <= 4.  It stays short of the
// contiguous-read rate: the compiler's wait analysis does not follow the
// register ring through the extraction's control flow and waits for each
// slot's loads at its first use (without the extraction: 106 us), and the
// per-wave register budget bounds the bytes in flight.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace i8mm {

namespace {

constexpr int kGvPiece = 1024;  // bytes of a row a load instruction reads

template <int N_>
__device__ __forceinline__ void gv_wait_vm() {
  static_assert(N_ >= 0 && N_ < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N_ & 15) | ((N_ >> 4) << 14) | (7 << 4) | (15 << 8));
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Butterfly over the 64 lanes: v[0 .. V) per lane in, and lane l out with
// the sum over all lanes of entry l >> (6 - log2 V) in v[0].  Each step
// halves the entries a lane keeps (the partner, lane ^ s, keeps the other
// half), then the last lane bits are plain sums.
template <int V, int S = 32, typename X>
__device__ __forceinline__ void butterfly(X (&v)[V], int lane) {
  if constexpr (S >= 1) {
    constexpr int C = (V >> ilog2(32 / S)) > 0 ? (V >> ilog2(32 / S)) : 1;  // entries held
    if constexpr (C > 1) {
      constexpr int H = C / 2;
      const bool up = (lane & S) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const X send = up ? v[i] : v[i + H];
        const X keep = up ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, S, 64);
      }
    } else {
      v[0] += __shfl_xor(v[0], S, 64);
    }
    butterfly<V, S / 2>(v, lane);
  }
}

}  // namespace

// TT: token capacity (T <= TT); R channel rows a workgroup (one wave); D
// pieces in flight, in a ring of registers.  FUSED: the layer (Y); else
// C = Xq . CB^T (int32).  ZP: zero-point activations (the offset term in the
// epilogue).
template <int TT, int R, int D, bool FUSED, bool ZP>
__global__ __launch_bounds__(64) void k_gemv(GemmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int V = R * TT, LV = ilog2(V);
  static_assert((1 << LV) == V && V <= 64, "R * TT: a power of two, at most 64");
  static_assert((D - 1) * (R + TT) < 64, "vmcnt range");
  __shared__ int32_t sO[kFewOcap];
  __shared__ _Float16 sXo[kFewOcap * TT];
  __shared__ int8_t sC[kFewOcap * R];
  const int lane = threadIdx.x;
  const uint32_t lo = (uint32_t)lane * 16;  // the lane's bytes of a piece
  if (a.clear_mask && blockIdx.x == 0)
    for (int64_t w = lane; w < a.clear_words; w += 64) a.clear_mask[w] = 0u;
  const int64_t m0 = (int64_t)blockIdx.x * R;
  const int64_t ra = a.N - m0 < R ? a.N - m0 : R;

  __amdgpu_buffer_rsrc_t rsA, rsB;
  uint32_t lda32 = 0, ldb32 = 0;
  auto setup = [&](const void* A, int64_t lda, const void* B, int64_t ldb) {
    rsA = make_rsrc((const char*)A + m0 * lda, (uint32_t)(ra * lda));
    rsB = make_rsrc(B, (uint32_t)(a.T * ldb));
    lda32 = (uint32_t)lda;
    ldb32 = (uint32_t)ldb;
  };
  v4i w[D][R], x[D][TT];
  // piece p of rows ending at byte Kb into ring slot d: the TT token rows
  // and the R weight rows.  Lanes past Kb, rows past the operand, tokens past
  // T and pieces past the end read zeros (out-of-range offsets: no memory
  // traffic), so every piece is the same R + TT loads.
  auto issue = [&](int d, int64_t p, int64_t Kb) {
    const int64_t k0 = p * kGvPiece;
    const bool ok = (int64_t)lo < Kb - k0;
    // (uniform; said so, or the compiler loops over lanes for it)
    const int so = __builtin_amdgcn_readfirstlane(k0 < Kb ? (int)k0 : 0);
#pragma unroll
    for (int t = 0; t < TT; ++t)
      x[d][t] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(
                   rsB, (ok && t < a.T) ? (uint32_t)t * ldb32 + lo : 0x80000000u, so, 0));
#pragma unroll
    for (int r = 0; r < R; ++r)
      w[d][r] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(
                   rsA, (ok && r < ra) ? (uint32_t)r * lda32 + lo : 0x80000000u, so, 2));
  };

  // ---- outlier set (fused) ----
  int64_t n_use = 0, nxt = 0;
  bool inloop = false;
  int nextc = 0x7fffffff;
  if constexpr (FUSED) {
    const int64_t n_o = a.counts[0];
    n_use = n_o < a.max_o ? n_o : a.max_o;
    inloop = n_use <= kFewOcap && !a.wo_ready;
  }
  // the outlier list and the tile's X[:, O] values to LDS: run once the
  // first pieces are in flight (done before them, its loads held every
  // workgroup's stream back by a load latency: about 10 us a call at T = 1)
  auto stage_outliers = [&]() {
    if constexpr (FUSED) {
      if (inloop) {
        for (int64_t o = lane; o < n_use; o += 64) {
          sO[o] = a.O[o];
#pragma unroll
          for (int t = 0; t < TT; ++t)
            sXo[o * TT + t] = t < a.T ? a.Xo[t * a.ldo + o] : (_Float16)0.0f;
        }
        __syncthreads();
        if (n_use > 0) nextc = __builtin_amdgcn_readfirstlane(sO[0]);
      }
    }
  };
  // the codes of the outlier columns in int8 piece p (weights w): the lane
  // holding column o copies its byte of each of the R rows to sC[idx][.]
  auto extract = [&](const v4i (&w)[R], int64_t p) {
    const int64_t kend = (p + 1) * kGvPiece;
    while (nextc < kend) {
      const int off = nextc & (kGvPiece - 1);
      if (lane == (off >> 4)) {
        const int comp = (off >> 2) & 3, sh = (off & 3) * 8;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int word = comp == 0 ? w[r][0] : comp == 1 ? w[r][1] : comp == 2 ? w[r][2] : w[r][3];
          sC[nxt * R + r] = (int8_t)(word >> sh);
        }
      }
      ++nxt;
      nextc = nxt < n_use ? __builtin_amdgcn_readfirstlane(sO[nxt]) : 0x7fffffff;
    }
  };

  // ---- the K loop over bytes [0, Kb): wait for piece p (pieces p+1 ..
  // p+D-1 may stay in flight), use it, refill its slot with piece p+D.  The
  // scheduling barriers keep the loads in this order: the compiler's own
  // waits then follow the ring (with the loads moved, it waits for them
  // all at each use). ----
  auto run = [&](auto f16, int64_t Kb, auto& acc, auto&& primed) {
    const int64_t P = Kb > 0 ? ceil_div(Kb, kGvPiece) : 1;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      issue(d, d, Kb);
      __builtin_amdgcn_sched_barrier(0);
    }
    primed();
    for (int64_t p0 = 0; p0 < P; p0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int64_t p = p0 + d;
        if (p >= P) break;
        gv_wait_vm<(D - 1) * (R + TT)>();
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              // (each element through a scalar first: clang's bit_cast of a
              // vector element reads element 0)
              const int wi = w[d][r][c], xi = x[d][t][c];
              if constexpr (decltype(f16)::value) {
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                acc[r * TT + t] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, wi),
                                                         __builtin_bit_cast(h2, xi),
                                                         acc[r * TT + t], false);
              } else {
                acc[r * TT + t] = __builtin_amdgcn_sdot4(wi, xi, acc[r * TT + t], false);
              }
            }
        if constexpr (FUSED && !decltype(f16)::value) {
          if (inloop) extract(w[d], p);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(d, p + D, Kb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    gv_wait_vm<0>();
  };

  int acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0;
  setup(a.A, a.lda, a.B, a.ldb);
  run(std::false_type{}, a.K, acc, stage_outliers);
  butterfly<V>(acc, lane);

  // this lane's (channel row, token); the 64 / V lanes of a group agree
  const int idx = lane >> (6 - LV);
  const int r = idx / TT, t = idx % TT;
  const bool lead = (lane & ((64 >> LV) - 1)) == 0;
  const int64_t f = m0 + r;
  const bool valid = r < ra && t < a.T;
  if constexpr (!FUSED) {
    if (lead && valid) a.C[t * a.N + f] = acc[0];
  } else {
    const float sxt = valid ? a.sx[t] : 0.0f;
    const float sj = valid ? a.SCB[f] : 0.0f;
    float y = (float)acc[0] * (sxt * (sj * (1.0f / 16129.0f)));
    const int64_t npad = round_up(n_use, 32);
    // wider sets whose Wo no step-2 kernel built (wo_gather: steps 1-2 were
    // one workgroup): their codes are gathered from CB, kFewOcap columns at
    // a time, and go the same way
    const bool gather = FUSED && a.wo_gather && !inloop && n_use > 0;
    if (inloop || gather) {
      // Wo rows of this tile (zeros up to the 32-column pad), and the fp16
      // products in increasing o
      float px = 0.0f;
      for (int64_t o0 = 0; o0 < npad; o0 += kFewOcap) {
        const int64_t cnt = npad - o0 < kFewOcap ? npad - o0 : kFewOcap;
        if (gather) {
          __syncthreads();  // done with the previous columns
          for (int64_t o = lane; o < cnt && o0 + o < n_use; o += 64) {
            const int col = a.O[o0 + o];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
              sXo[o * TT + tt] = tt < a.T ? a.Xo[tt * a.ldo + o0 + o] : (_Float16)0.0f;
#pragma unroll
            for (int rr = 0; rr < R; ++rr) sC[o * R + rr] = rr < ra ? a.A[(m0 + rr) * a.lda + col] : 0;
          }
          __syncthreads();
        }
        const int64_t cb = inloop ? o0 : 0;  // first column of the chunk in sC / sXo
        for (int64_t i = lane; i < R * cnt; i += 64) {
          const int rr = (int)(i / cnt);
          const int64_t o = i % cnt;
          if (rr < ra) {
            const _Float16 v = o0 + o < n_use
                                   ? dequant_weight(sC[(cb + o) * R + rr], a.SCB[m0 + rr])
                                   : (_Float16)0.0f;
            ((_Float16*)a.Wo)[(m0 + rr) * a.ldo + o0 + o] = v;
          }
        }
        for (int64_t o = 0; o < cnt && o0 + o < n_use; ++o)
          px += (float)sXo[(cb + o) * TT + t] * (float)dequant_weight(sC[(cb + o) * R + r], sj);
      }
      y += px;
    } else if (npad > 0) {
      // wide outlier sets, or Wo built by step 2: fp16 rows of the workspace
      float pf[V];
#pragma unroll
      for (int i = 0; i < V; ++i) pf[i] = 0.0f;
      setup(a.Wo, a.ldo * 2, a.Xo, a.ldo * 2);
      run(std::true_type{}, npad * 2, pf, [] {});
      butterfly<V>(pf, lane);
      y += pf[0];
    }
    float bv = 0.0f, zt = 0.0f;
    if (a.bias && valid) bv = h2f(a.bias[f]);
    if constexpr (ZP) {
      if (valid) {
        const int os = npad > 0 ? a.osum[f] : 0;
        zt = (sxt * (float)a.zp[t] * (1.0f / 127.0f)) *
             (sj * (float)(a.rsum[f] - os) * (1.0f / 127.0f));
      }
    }
    const float v = y + bv;
    if (lead && valid) a.Y[t * a.N + f] = (_Float16)(ZP ? v + zt : v);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

namespace {
template <int TT, int R, int D, bool FUSED, bool ZP>
hipError_t launch_gemv_t(const GemmArgs& a, hipStream_t st) {
  k_gemv<TT, R, D, FUSED, ZP><<<dim3((unsigned)ceil_div(a.N, R)), dim3(64), 0, st>>>(a);
  return hipGetLastError();
}
template <bool FUSED, bool ZP>
hipError_t launch_gemv_z(const GemmArgs& a, hipStream_t st) {
  // 4 rows a workgroup: the fewest registers for the most loads in flight
  // per CU (T = 1, per call at 49152 x 12288: 4 rows x 4 pieces 111 us,
  // 8 x 4 116 us, 16 x 2 128 us, 1 x 8 131 us)
  if (a.T <= 1) return launch_gemv_t<1, 4, 4, FUSED, ZP>(a, st);
  if (a.T <= 2) return launch_gemv_t<2, 4, 4, FUSED, ZP>(a, st);
  return launch_gemv_t<4, 4, 3, FUSED, ZP>(a, st);
}
}  // namespace

bool gemv_supported(const GemmArgs& a) {
  const int64_t lim = (int64_t)1 << 31;
  return a.T >= 1 && a.T <= 4 && a.N >= 1 && 4 * a.lda < lim && 4 * a.ldo * 2 < lim &&
         a.T * a.ldb < lim && a.T * a.ldo * 2 < lim;
}

hipError_t launch_gemv(const GemmArgs& a, bool fused, hipStream_t st) {
  if (!fused) return launch_gemv_z<false, false>(a, st);
  if (a.zp) return launch_gemv_z<true, true>(a, st);
  return launch_gemv_z<true, false>(a, st);
}

}  // namespace i8mm
