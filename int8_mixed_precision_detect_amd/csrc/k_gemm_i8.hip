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
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace i8mm {

namespace {

// MODE_FUSED_X: the fused product for few tokens (one token tile, one wave
// owning every channel row of its tile), which also extracts the outlier
// weights itself -- see the int8 loop.
// Split K (MODE_PART then MODE_COMBINE): splits workgroups a tile each walk
// a range of K and store their int32 accumulators in a.part; one combine
// workgroup a tile loads and adds them (exact) and runs the fused epilogue.
constexpr int MODE_I32 = 0, MODE_FUSED = 1, MODE_FUSED_X = 2, MODE_PART = 3, MODE_COMBINE = 4;
struct NoDma {
  __device__ void operator()(int) const {}
};
// LDS beyond the slices for MODE_FUSED_X: the outlier list and the tile's
// X[:, O] values ([kFewStage][BN] halves), kFewStage outlier columns at a
// time: 48 rather than all kFewOcap the tiles take keeps 8 (32 x 16) or 4
// (64 x 32) workgroups on a CU instead of 7 or 3
constexpr int64_t kFewStage = 48;
constexpr size_t few_lds(int BN) { return (size_t)kFewStage * 4 + (size_t)kFewStage * BN * 2; }
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
// wait until at most n*PW of this wave's loads are outstanding
template <int PW>
__device__ __forceinline__ void wait_slices(int n) {
  if (n >= 5)
    wait_vm<5 * PW < 64 ? 5 * PW : 63>();
  else if (n == 4)
    wait_vm<4 * PW < 64 ? 4 * PW : 63>();
  else if (n == 3)
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

// NTA: the weight operand's slice loads are non-temporal (streamed once: the
// few-token shapes, where each weight byte is used by one workgroup).
// ZP: zero-point activations -- the epilogue adds the offset part of the
// int8 product, (sx Z / 127)(SCB (rsum - osum) / 127), before the store.
template <int BM, int BN, int WM, int WN, int S, int KB, int MODE, bool NTA, bool ZP>
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
  // wide tiles issue each slice refill among the MFMAs of the slice before
  constexpr bool kInterleave = MODE != MODE_FUSED_X && (WM / 16) * (WN / 16) > 32;
  static_assert(KB == 64 || KB == 128, "slice width");
  static_assert(S >= 2 && S <= 6 && (S - 1) * PW < 64, "slices in flight");
  static_assert(MODE != MODE_FUSED_X || (NWAVE == 1 && BM <= 64), "one wave, one lane a row");
  static_assert((ACH + BCH) % NWAVE == 0, "slice pieces must split evenly over waves");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / NWN) * WM, wn0 = (wave % NWN) * WN;
  // the forward's outlier mask: step 2 is done with it; zero it for the next
  // call's detection (the first workgroup of the call's first product launch)
  if (a.clear_mask && blockIdx.x == 0)
    for (int64_t w = tid; w < a.clear_words; w += (BM / WM) * (BN / WN) * 64) a.clear_mask[w] = 0u;

  // work items (split, tile), split-major.  Workgroups are dealt to the 8
  // XCDs round-robin; give each XCD a contiguous run of items, consecutive
  // tiles sharing one weight tile.
  const int64_t tiles_m = ceil_div(a.N, BM), tiles_n = ceil_div(a.T, BN);
  const int64_t ntiles = tiles_m * tiles_n;
  const int64_t splits = MODE == MODE_PART ? a.splits : 1;
  const int64_t items = ntiles * splits;
  int64_t bid = blockIdx.x;
  if ((items & 7) == 0) bid = (bid & 7) * (items >> 3) + (bid >> 3);
  const int64_t split = bid / ntiles, tile = bid % ntiles;
  const int64_t tn = tile % tiles_n, tm = tile / tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  // this split's range of K: whole slices, the last range ragged
  const int64_t ksplit = round_up(ceil_div(a.K, splits), KB);
  const int64_t kbeg = split * ksplit < a.K ? split * ksplit : a.K;
  const int64_t kend = kbeg + ksplit < a.K ? kbeg + ksplit : a.K;

  // Slice loads: buffer_load_dwordx4 ... lds.  The operand is a buffer
  // resource (base in SGPRs), a lane's 32-bit offset (row * ld + its chunk)
  // is fixed for the whole K loop and the K position goes in the scalar
  // offset, so a load costs no per-lane address arithmetic.
  const int wv = NWAVE == 1 ? 0 : __builtin_amdgcn_readfirstlane(wave);
  __amdgpu_buffer_rsrc_t rsA, rsB;
  uint32_t voff[PW];
  // a lane's chunk within its row: rows of a piece start at multiples of
  // RPP (8 or 16), so the swizzle of row rr depends only on the lane
  const int kc = ((lane % CPR) ^ swz<KB>(lane / CPR)) * 16;
  // The resources start at the tile's first row and span its rows only, so
  // an operand of any size is addressed with 32-bit offsets as long as
  // BM (BN) rows of it fit in 2^31 bytes, which the host checks.
  auto setup = [&](const char* A, int64_t ldab, int64_t rowsA, const char* B, int64_t ldbb,
                   int64_t rowsB) {
    const int64_t ra = rowsA - m0 < BM ? rowsA - m0 : BM;
    const int64_t rb = rowsB - n0 < BN ? rowsB - n0 : BN;
    rsA = __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * ldab), (short)0,
                                            (int)(ra > 0 ? ra * ldab : 0), 0x00020000);
    rsB = __builtin_amdgcn_make_buffer_rsrc((void*)(B + n0 * ldbb), (short)0,
                                            (int)(rb > 0 ? rb * ldbb : 0), 0x00020000);
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
      // 32-bit arithmetic (the offset within the tile's rows), which keeps
      // fewer registers live across the K loop.  Rows past the operand (a
      // ragged last tile, the token rows of a few-token tile beyond T) get
      // an out-of-range offset: they read zeros without touching memory
      // (their results are never stored; a clamped row made every such
      // lane re-read one line of the last row)
      const int64_t gr = isA ? m0 + rr : n0 + rr;
      voff[u] = gr < (isA ? a.N : a.T)
                    ? (uint32_t)rr * (uint32_t)(isA ? ldab : ldbb) + (uint32_t)kc
                    : 0x80000000u;
    }
  };
  auto lds_dst = [&](int buf, int u) {
    const int j = wv * PW + u;
    const int off = (j < ACH) ? j * 1024 : BM * KB + (j - ACH) * 1024;
    return (__attribute__((address_space(3))) void*)(lds + buf * STAGE + off);
  };
  // one 1 KB piece; the cache policy is an immediate, hence the two calls
  // (the A/B choice is wave-uniform)
  auto dma = [&](int u, void* dst, uint32_t vo, int64_t k0) {
    auto d = (__attribute__((address_space(3))) void*)dst;
    if (wv * PW + u < ACH)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, d, 16, vo, (int)k0, 0, NTA ? 2 : 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, d, 16, vo, (int)k0, 0, 0);
  };
  auto issue = [&](int buf, int64_t k0, int64_t Kb) {
    if (k0 + KB <= Kb) {
#pragma unroll
      for (int u = 0; u < PW; ++u) dma(u, (void*)lds_dst(buf, u), voff[u], k0);
    } else {
      const int rem = (int)(Kb - k0);  // bytes of the slice inside [k0, Kb)
#pragma unroll
      for (int u = 0; u < PW; ++u)
        dma(u, (void*)lds_dst(buf, u), kc < rem ? voff[u] : 0x80000000u, k0);
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
  // the MFMAs of one slice; the other waves of the SIMD cover LDS latency.
  // dma(u), when given, issues piece u of a slice refill: the wide tiles
  // interleave the PW pieces with the first MFMAs of the slice, one piece per
  // NI/2 MFMAs, so that a wave keeps its MFMA pipe busy while the CU's
  // address unit works through the workgroup's refill queue (issued in one
  // burst, the pieces held every wave's MFMAs back until its own were
  // accepted).
  auto compute = [&](auto f16, int buf, auto&& dma_piece) {
    constexpr bool kDma = !std::is_same_v<std::decay_t<decltype(dma_piece)>, NoDma>;

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
          if constexpr (kDma) {
            static_assert(NI % 2 == 0 && 2 * MI * KS >= PW, "refill slots");
#pragma unroll
            for (int jh = 0; jh < 2; ++jh) {
#pragma unroll
              for (int j = jh * (NI / 2); j < (jh + 1) * (NI / 2); ++j) mma(f16, i, j, fa0, fb[j]);
              __builtin_amdgcn_sched_group_barrier(0x008, NI / 2, 0);
              const int slot = (h * MI + i) * 2 + jh;
              if (slot < PW) {
                dma_piece(slot);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
              }
            }
          } else {
#pragma unroll
            for (int j = 0; j < NI; ++j) mma(f16, i, j, fa0, fb[j]);
            __builtin_amdgcn_sched_group_barrier(0x008, NI, 0);
          }
          fa0 = fa1;
        }
      }
    }
  };

  // Few tokens (MODE_FUSED_X): the outlier weights come out of the CB bytes
  // this workgroup stages anyway.  O is ascending, so one pointer follows the
  // k walk: when slice kt holds the next outlier column, the lane owning each
  // channel row reads that byte from LDS, dequantizes it and adds its
  // products with the tile's X[:, O] values (staged in LDS) to px, one fp32
  // sum per token.  The lane also shifts the value into wb, a window of the
  // last 64 columns of its Wo row held in registers, which goes to the
  // workspace after the K loop (and every 64th column for wider sets).  The
  // K loop loads and stores nothing in global memory but the slices: a store
  // there, waited for with the slices, costs about a slice's time.  O and
  // X[:, O] are staged kFewStage columns at a time (sets up to kFewOcap
  // columns, or any width when no step-2 kernel built Wo); each restaging
  // waits for the slices in flight, which only sets wider than kFewStage
  // columns pay.
  int64_t n_use = 0;
  bool inloop = false;
  int64_t nxt = 0;
  int nextc = 0x7fffffff;
  float sjx = 0.0f;
  constexpr int PX = MODE == MODE_FUSED_X ? BN : 1;  // (nothing of this in other modes)
  float px[PX];
#pragma unroll
  for (int t = 0; t < PX; ++t) px[t] = 0.0f;
  int32_t* sO = (int32_t*)(lds + S * STAGE);                                   // [kFewStage]
  _Float16* sXo = (_Float16*)(lds + S * STAGE + kFewStage * 4);                // [kFewStage][BN]
  int64_t sbase = 0;  // the first outlier column staged
  constexpr int WB = MODE == MODE_FUSED_X ? 32 : 1;  // dwords of the window
  uint32_t wb[WB];
#pragma unroll
  for (int q = 0; q < WB; ++q) wb[q] = 0u;
  // window shifts down by one half, h comes in at the top
  auto wb_push = [&](uint32_t h) {
#pragma unroll
    for (int q = 0; q < WB; ++q)
      wb[q] = __builtin_amdgcn_alignbit(q + 1 < WB ? wb[q + 1] : h, wb[q], 16);
  };
  // ... by d halves (uniform, 0 <= d < 2 * WB), zeros in at the top
  auto wb_shift = [&](int d) {
    if (d & 1) {
#pragma unroll
      for (int q = 0; q < WB; ++q)
        wb[q] = __builtin_amdgcn_alignbit(q + 1 < WB ? wb[q + 1] : 0u, wb[q], 16);
    }
#pragma unroll
    for (int b = 1; (1 << b) < 2 * WB; ++b) {
      if (d & (1 << b)) {
        const int w = 1 << (b - 1);  // dwords
#pragma unroll
        for (int q = 0; q < WB; ++q) wb[q] = q + w < WB ? wb[q + w] : 0u;
      }
    }
  };
  // the window holds Wo columns o0 .. o0 + 2 WB - 1 of this lane's row; the
  // 8-column pieces below lim go out
  auto wb_store = [&](int64_t o0, int64_t lim) {
    if (m0 + lane < a.N) {
      _Float16* dst = (_Float16*)a.Wo + (m0 + lane) * a.ldo + o0;
#pragma unroll
      for (int q = 0; q < WB / 4; ++q)
        if (o0 + 8 * q < lim) *(v4u*)(dst + 8 * q) = v4u{wb[4 * q], wb[4 * q + 1], wb[4 * q + 2], wb[4 * q + 3]};
    }
  };
  // columns o0 .. o0 + kFewStage - 1 of O and of the tile's X[:, O] rows into
  // sO / sXo (one wave: its LDS accesses stay in order)
  auto stage_o = [&](int64_t o0) {
    if constexpr (MODE == MODE_FUSED_X) {
      const int64_t cnt = n_use - o0 < kFewStage ? n_use - o0 : kFewStage;
      for (int64_t o = lane; o < cnt; o += 64) {
        sO[o] = a.O[o0 + o];
        // unconditional loads (rows clamped), so that they are all in flight at once
        _Float16 xv[BN];
#pragma unroll
        for (int t = 0; t < BN; ++t) {
          const int64_t tt = n0 + t < a.T ? n0 + t : a.T - 1;
          xv[t] = a.Xo[tt * a.ldo + o0 + o];
        }
#pragma unroll
        for (int t = 0; t < BN; ++t) sXo[o * BN + t] = n0 + t < a.T ? xv[t] : (_Float16)0.0f;
      }
    }
  };
  // run while the first slices are in flight
  auto few_setup = [&]() {
    if constexpr (MODE == MODE_FUSED_X) {
      const int64_t n_o = a.counts[0];
      n_use = n_o < a.max_o ? n_o : a.max_o;
      // sets built by no step-2 kernel (wo_gather: steps 1-2 were one
      // workgroup) are walked whatever their width, kFewOcap columns of O
      // and X[:, O] staged at a time
      inloop = !a.wo_ready && (n_use <= kFewOcap || a.wo_gather);
      if (inloop) stage_o(0);
      if (lane < BM && m0 + lane < a.N) sjx = a.SCB[m0 + lane];
      asm volatile("" ::"v"(sjx));  // waited for here rather than inside the K loop
      __syncthreads();
      if (inloop && n_use > 0) nextc = __builtin_amdgcn_readfirstlane(sO[0]);
    }
  };
  auto extract = [&](int buf, int64_t kbase) {
    while (nextc < kbase + KB) {
      const int off = nextc - (int)kbase;  // 0 .. KB-1
      if (lane < BM) {
        const int chunk = (off >> 4) ^ swz<KB>(lane);
        const int c = (int8_t)lds[buf * STAGE + lane * KB + chunk * 16 + (off & 15)];
        const _Float16 wo = dequant_weight(c, sjx);
        wb_push(__builtin_bit_cast(uint16_t, wo));
        if ((nxt & 63) == 63) wb_store(nxt - 63, n_use);
        const float wf = (float)wo;
        const _Float16* xr = sXo + (nxt - sbase) * BN;
#pragma unroll
        for (int t = 0; t < PX; ++t) px[t] += (float)xr[t] * wf;
      }
      ++nxt;
      if (nxt < n_use && nxt - sbase == kFewStage) {
        // the next kFewStage columns (its loads wait for the slices in
        // flight too)
        __syncthreads();
        stage_o(nxt);
        sbase = nxt;
        __syncthreads();
      }
      nextc = nxt < n_use ? __builtin_amdgcn_readfirstlane(sO[nxt - sbase]) : 0x7fffffff;
    }
  };

  // The fused epilogue's fp16 outlier operands (Xo/Wo rows of kt_f16 bytes):
  // when they fit one slice (up to 64 outlier columns) that slice is issued
  // into a slice buffer the int8 loop no longer needs, during its last
  // slice, so that its latency overlaps the end of the loop and the scaling.
  int64_t kt_f16 = 0;
  if constexpr (MODE == MODE_FUSED || MODE == MODE_FUSED_X || MODE == MODE_COMBINE) {
    const int64_t n_o = a.counts[0];
    kt_f16 = round_up(n_o < a.max_o ? n_o : a.max_o, 32) * 2;
  }
  const bool tail_pre = (MODE == MODE_FUSED || MODE == MODE_COMBINE) && kt_f16 > 0 && kt_f16 <= KB;
  int tail_buf = 0;
  auto tail_prefetch = [&](int buf) {
    setup((const char*)a.Wo, a.ldo * 2, a.N, (const char*)a.Xo, a.ldo * 2, a.T);
    issue(buf, 0, kt_f16);
    tail_buf = buf;
  };

  // K loop over bytes [kb, ke) of the operands set up last: S slices in
  // flight, one barrier per slice.  LDS must be free of earlier readers on
  // entry.  primed() runs once the first slices are issued.
  // Slice kt goes to buffer (b0 + kt) % S; the first `pre` slices were
  // issued before the call.
  auto run = [&](auto f16, int64_t kb, int64_t Kb, auto&& primed, int b0 = 0, int pre = 0) {
    const int64_t nk = ceil_div(Kb - kb, KB);
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (s >= pre && s < nk) issue((b0 + s) % S, kb + s * KB, Kb);
    primed();
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
      const bool refill = kt >= 1 && kt - 1 + S < nk;
      if constexpr (!kInterleave) {
        if (refill) issue((int)((b0 + kt - 1) % S), kb + (kt - 1 + S) * KB, Kb);
      }
      if constexpr (MODE == MODE_FUSED && !decltype(f16)::value) {
        // the last slice: buffer (kt + 1) % S held slice kt + 1 - S, done.
        // (An opaque copy of the flag, so that the compiler does not version
        // the whole loop on it.)
        int pre = tail_pre && kt == nk - 1;
        asm volatile("" : "+v"(pre));
        if (__builtin_amdgcn_readfirstlane(pre)) tail_prefetch((int)((b0 + kt + 1) % S));
      }
      if constexpr (MODE == MODE_FUSED_X && !decltype(f16)::value)
        extract((int)((b0 + kt) % S), kb + kt * KB);
      if constexpr (kInterleave) {
        // The refill of slice kt-1+S goes out among the MFMAs of slice kt (a
        // ragged last slice reads zeros past Kb).  Iterations without one
        // issue the same pieces as no-ops -- out-of-range offsets, which
        // read nothing, into a spare 1 KB of LDS -- so that the loop body
        // is one block.
        const int64_t k0 = kb + (kt - 1 + S) * KB;
        const int rem = !refill ? 0 : k0 + KB <= Kb ? KB : (int)(Kb - k0);
        const int rb = (int)((b0 + kt - 1 + S) % S);
        compute(f16, (int)((b0 + kt) % S), [&](int u) {
          void* dst = refill ? (void*)lds_dst(rb, u) : (void*)(lds + S * STAGE);
          dma(u, dst, kc < rem ? voff[u] : 0x80000000u, refill ? k0 : 0);
        });
      } else {
        compute(f16, (int)((b0 + kt) % S), NoDma{});
      }
      // keeps the epilogue's loads (scales, bias) below the loop instead of
      // hoisted above it, where they would hold registers throughout
      asm volatile("" ::: "memory");
    }
  };

  // int32 partial tiles of split K, in the accumulators' register layout:
  // block (i, j) of wave w at ((w * MI + i) * NI + j) * 64 + lane, 16 bytes
  // a lane (coalesced 1 KB per block)
  auto part_at = [&](int64_t sp) {
    return (v4i*)(a.part + (sp * ntiles + tile) * ((int64_t)BM * BN)) +
           (int64_t)wave * (MI * NI * 64) + lane;
  };
  if constexpr (MODE == MODE_COMBINE) {
    if (tail_pre) tail_prefetch(0);
    // acc = the sum of the splits' partial tiles (exact int32)
#pragma unroll
    for (int64_t sp = 0; sp < a.splits; ++sp) {
      const v4i* src = part_at(sp);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] += src[(i * NI + j) * 64];
    }
  } else {
    setup((const char*)a.A, a.lda, a.N, (const char*)a.B, a.ldb, a.T);
    run(I8Slices{}, kbeg, kend, few_setup);
  }
  if constexpr (MODE == MODE_PART) {
    v4i* dst = part_at(split);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) dst[(i * NI + j) * 64] = acc[i][j];
    return;
  }

  // (opaque copies of the lane's position: the epilogue's indices are
  // computed here and again after the outlier loop, not hoisted above the
  // loops and kept -- spilled -- across them)
  int lrow = 4 * (lane >> 4);  // first of the 4 channels a lane holds
  int lcol = lane & 15;        // token within a 16-wide block
  asm volatile("" : "+v"(lrow), "+v"(lcol));
  const int m0i = (int)m0, n0i = (int)n0;  // T, N < 2^31

  if constexpr (MODE == MODE_I32) {
    const bool cvec = ((a.N & 3) == 0) && ((((uintptr_t)a.C) & 15) == 0);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int f = m0i + wm0 + i * 16 + lrow;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int t = n0i + wn0 + j * 16 + lcol;
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
    const int64_t Kt = kt_f16;  // bytes of an Xo / Wo row in use
    float sxv[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int t = n0i + wn0 + j * 16 + lcol;
      // clamped, unconditional loads: all in flight together
      const float v = a.sx[t < a.T ? t : a.T - 1];
      sxv[j] = (t < a.T) ? v : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f = m0i + wm0 + i * 16 + lrow + r;
        const float sv = a.SCB[f < a.N ? f : a.N - 1];
        const float sc = f < a.N ? sv * (1.0f / 16129.0f) : 0.0f;
        // int32 accumulator -> fp32 acc * sx * SCB / 127^2, in place
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j][r] = __builtin_bit_cast(int, (float)acc[i][j][r] * (sxv[j] * sc));
      }
    if (MODE == MODE_FUSED_X && inloop) {
      // the outlier products were summed per (channel row, token) in px:
      // through LDS into the accumulator layout.  The window's last columns
      // go out, shifted to the bottom, with zeros up to the 32-column pad.
      if (lane < BM) {
        const int rem = (int)(n_use & 63);
        if (rem > 0) {
          wb_shift(2 * WB - rem);
          wb_store(n_use - rem, round_up(n_use, 32));
        }
      }
      __syncthreads();          // done with the int8 slices
      float* sp = (float*)lds;  // [BM][BN]
      if (lane < BM) {
#pragma unroll
        for (int t = 0; t < PX; ++t) sp[lane * BN + t] = px[t];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = wm0 + i * 16 + lrow + r, t = wn0 + j * 16 + lcol;
            // the element goes through a scalar first: clang's bit_cast of
            // a vector element reads element 0
            const int bits = acc[i][j][r];
            acc[i][j][r] = __builtin_bit_cast(int, __builtin_bit_cast(float, bits) + sp[row * BN + t]);
          }
    } else if (Kt > 0) {
      if (!tail_pre) {
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();  // every wave is done with the int8 slices
        setup((const char*)a.Wo, a.ldo * 2, a.N, (const char*)a.Xo, a.ldo * 2, a.T);
      }
      // (prefetched: its one slice is in flight in buffer tail_buf)
      run(F16Slices{}, 0, Kt, [] {}, tail_buf, tail_pre ? 1 : 0);
    }
    asm volatile("" : "+v"(lrow), "+v"(lcol));
    const bool yvec = ((a.N & 3) == 0) && ((((uintptr_t)a.Y) & 7) == 0);
    const bool bvec = a.bias && ((((uintptr_t)a.bias) & 7) == 0);
    // Zero-point activations: the offset part of the int8 product,
    // (sx Z / 127) (SCB R / 127) with R the channel's kept-column code sum,
    // is a rank-1 term; it is added here in fp32, one factor per token and
    // one per channel, rather than to the int32 accumulators (where its
    // extra registers would not fit the widest tile).
    float ut[ZP ? NI : 1];
    if constexpr (ZP) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int t = n0i + wn0 + j * 16 + lcol;
        const int64_t tc = t < a.T ? t : a.T - 1;
        const float sxt = a.sx[tc];
        const int z = a.zp[tc];
        ut[j] = t < a.T ? sxt * (float)z * (1.0f / 127.0f) : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int f = m0i + wm0 + i * 16 + lrow;  // 4 consecutive channels
      float vr[ZP ? 4 : 1];
      if constexpr (ZP) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t fc = f + r < a.N ? f + r : a.N - 1;
          const int rs = a.rsum[fc];
          const int os = Kt > 0 ? a.osum[fc] : 0;
          const float sv = a.SCB[fc];
          vr[r] = f + r < a.N ? sv * (float)(rs - os) * (1.0f / 127.0f) : 0.0f;
        }
      }
      float bv[4];
      if constexpr (MODE == MODE_FUSED_X) {
        // short kernels: clamped, unconditional loads, all four in flight
        // together (the wide tiles keep the conditional form below, with
        // which they do not spill in the K loop)
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[r] = 0.0f;
        if (a.bias) {
          _Float16 hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) hv[r] = a.bias[f + r < a.N ? f + r : a.N - 1];
#pragma unroll
          for (int r = 0; r < 4; ++r) bv[r] = f + r < a.N ? h2f(hv[r]) : 0.0f;
        }
      } else if (bvec && f + 3 < a.N) {
        // 4 consecutive channels: one 8-byte load
        const v4h hv = *(const v4h*)(a.bias + f);
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[r] = h2f(hv[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[r] = (a.bias && f + r < a.N) ? h2f(a.bias[f + r]) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const v4f v = __builtin_bit_cast(v4f, acc[i][j]);
        v4f w;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (ZP)
            w[r] = v[r] + bv[r] + ut[j] * vr[r];
          else
            w[r] = v[r] + bv[r];
        }
        acc[i][j] = __builtin_bit_cast(v4i, w);
      }
    }
    // Wide tiles with N a multiple of 8: Y goes out through LDS, 64 tokens
    // of the tile at a time, as whole 16-byte chunks of token rows, so that
    // every line of Y is written completely by one workgroup at once.
    bool staged = false;
    if constexpr (MODE != MODE_FUSED_X) {
      staged = ((a.N & 7) == 0) && ((((uintptr_t)a.Y) & 15) == 0);
      if (staged) {
        constexpr int JP = 2, RW = NWN * JP * 16, LDH = BM + 8, CH = BM / 8, TOT = RW * CH;
        static_assert(NI % JP == 0 && TOT % (NWAVE * 64) == 0, "staging passes");
        static_assert(RW * LDH * 2 <= S * STAGE, "staging fits the slice buffers");
        _Float16* sy = (_Float16*)lds;
        __syncthreads();  // every wave is done with the slices in LDS
#pragma unroll
        for (int q = 0; q < NI / JP; ++q) {
#pragma unroll
          for (int jj = 0; jj < JP; ++jj) {
            const int row = (wave % NWN) * (JP * 16) + jj * 16 + lcol;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
              const v4f v = __builtin_bit_cast(v4f, acc[i][q * JP + jj]);
              v4h y;
#pragma unroll
              for (int r = 0; r < 4; ++r) y[r] = (_Float16)v[r];
              *(v4h*)(sy + row * LDH + wm0 + i * 16 + lrow) = y;
            }
          }
          __syncthreads();
#pragma unroll
          for (int c0 = 0; c0 < TOT; c0 += NWAVE * 64) {
            const int c = c0 + tid, row = c / CH, ch = c % CH;
            const int64_t t = n0 + (row / (JP * 16)) * WN + q * (JP * 16) + row % (JP * 16);
            const int64_t f = m0 + ch * 8;
            const v4i val = *(const v4i*)(sy + row * LDH + ch * 8);
            if (t < a.T && f < a.N) *(v4i*)(a.Y + t * a.N + f) = val;
          }
          __syncthreads();
        }
      }
    }
    // otherwise: a token's channels of the wave tile (the MI 32-byte pieces
    // of its row segment) go out back to back, so that each line of Y is
    // complete in the cache before it is written back
    if (!staged)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int t = n0i + wn0 + j * 16 + lcol;
      if (t >= a.T) continue;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int f = m0i + wm0 + i * 16 + lrow;
        const v4f v = __builtin_bit_cast(v4f, acc[i][j]);
        v4h y;
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = (_Float16)v[r];
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
template <int BM, int BN, int WM, int WN, int S, int KB, int MODE, bool NTA = false,
          bool ZP = false>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  constexpr bool kWide = MODE != MODE_FUSED_X && (WM / 16) * (WN / 16) > 32;
  constexpr size_t LDS = (size_t)S * (BM + BN) * KB + (MODE == MODE_FUSED_X ? few_lds(BN) : 0) +
                         (kWide ? 1024 : 0);  // the no-op refills' target
  auto kern = k_gemm_i8<BM, BN, WM, WN, S, KB, MODE, NTA, ZP>;
  const hipError_t e = lds_limit<k_gemm_i8<BM, BN, WM, WN, S, KB, MODE, NTA, ZP>>(LDS);
  if (e != hipSuccess) return e;
  const int64_t items = ceil_div(a.N, BM) * ceil_div(a.T, BN) * (MODE == MODE_PART ? a.splits : 1);
  kern<<<dim3((unsigned)items), dim3(NT), LDS, st>>>(a);
  return hipGetLastError();
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

std::atomic<int64_t> g_split_override{0};
std::atomic<int64_t> g_tile_override{-1};

// Tile configurations of the wide tiles (channels x tokens per workgroup,
// per wave, slices in flight, slice bytes per row), one workgroup per CU
// (LDS-bound):
//   0: 320 x 256, 8 waves of 80 x 128, two 128-byte slices (144 KB LDS)
//   1: 256 x 256, 8 waves of 64 x 128, two 128-byte slices (128 KB LDS)
//   2: 192 x 256, 8 waves of 48 x 128, two 128-byte slices (112 KB LDS):
//      more tiles for narrow layers (N = 5120: 216 tiles instead of 160)
//   3: 320 x 128, 8 waves of 80 x 64, two 128-byte slices (112 KB LDS):
//      narrow layers as exactly one tile a CU (N = 5120, T = 2048: 256
//      tiles), without splitting K
constexpr int kCfgs = 4;
constexpr int64_t kCfgBM[kCfgs] = {320, 256, 192, 320}, kCfgBN[kCfgs] = {256, 256, 256, 128};
constexpr int64_t kMaxSplits = 4;
constexpr int64_t kMinSplitK = 1024;  // bytes of K a split walks at least

// Planner: a modelled duration (microseconds) for each configuration and
// split count, the smallest taken (ties: fewer splits, then the narrower
// tile).  The workgroups run in rounds of one per CU; one walks
// ceil(slices / splits) 128-byte slices of K at kSliceUs each, plus kItemUs
// of set-up and epilogue; a round that fills every CU runs kFullRound times
// slower (the workgroups share the last-level cache and fabric).  Splitting
// K adds the partial tiles: written once per round of the split launch
// (kPartWriteUs a KB), read back by the combine launch, whose ceil(tiles /
// CUs) rounds each read `splits` partial tiles per CU (kPartReadUs a KB).
// The constants are fitted to the measured durations of the three tiles on
// MI355X over 21 shapes, T = 64-4096, K = 4096-20480, N = 4096-49152 and
// 1-4 splits (least squares, then tuned so that the choice is the fastest
// measured one: it is on 17 shapes, within 5.7 % on the other four); the
// 320 x 128 tile's, to its durations on 14 shapes measured beside the
// others (its single-round shapes give 1.09 us a slice, 10.1 us of set-up
// and 1.04-1.07 for a full round; over the 14 the planner's choices take
// 0.8 % longer than the fastest measured ones, at most 7 % on one shape,
// T = 512, K = N = 4096).  So the 13B first feed-forward layer (20480 x 2048
// outputs, K = 5120) runs 512 tiles of configuration 0 in two rounds, the
// down projection (5120 x 2048, K = 20480) splits K in two over 128 of
// them, and the attention projection (5120 x 2048, K = 5120) runs 256
// tiles of configuration 3, one a CU (57 us against 59 us for 216 of
// configuration 2).
constexpr double kSliceUs[kCfgs] = {1.44, 1.45, 1.131, 1.09}, kItemUs[kCfgs] = {16.44, 11.23, 10.85, 10.1};
constexpr double kFullRound[kCfgs] = {1.213, 1.123, 1.040, 1.04};
constexpr double kPartWriteUs = 0.0409, kPartReadUs = 0.0293;

double plan_cost(int64_t T, int64_t N, int64_t K, int c, int64_t sp, int64_t cus) {
  const int64_t tiles = ceil_div(N, kCfgBM[c]) * ceil_div(T, kCfgBN[c]);
  const int64_t items = tiles * sp;
  const int64_t slices = ceil_div(K, 128) > 0 ? ceil_div(K, 128) : 1;
  const double rounds = (double)ceil_div(items, cus);
  double t = rounds * ((double)ceil_div(slices, sp) * kSliceUs[c] + kItemUs[c]) *
             (items >= cus ? kFullRound[c] : 1.0);
  if (sp > 1) {
    const double tile_kb = (double)(kCfgBM[c] * kCfgBN[c] * 4) / 1024.0;
    t += rounds * tile_kb * kPartWriteUs +
         (double)ceil_div(tiles, cus) * (double)sp * tile_kb * kPartReadUs;
  }
  return t;
}

void choose_wide(int64_t T, int64_t N, int64_t K, bool allow_split,
                 int64_t* cfg, int64_t* splits) {
  const int64_t cus = cu_count();
  const int64_t slices = ceil_div(K, 128) > 0 ? ceil_div(K, 128) : 1;
  const int64_t ovr = allow_split ? g_split_override.load() : 1;
  // an override is clamped to [1, min(slices, kMaxSplits)]
  int64_t want = ovr < slices ? ovr : slices;
  want = want < kMaxSplits ? want : kMaxSplits;
  double best = 0.0;
  *cfg = 1;
  *splits = 1;
  bool first = true;
  for (int64_t sp = 1; sp <= kMaxSplits; ++sp) {
    if (ovr > 0 && sp != want) continue;
    if (ovr == 0 && sp > 1 && (ceil_div(K, sp) < kMinSplitK || sp > slices)) continue;
    const int64_t tov = g_tile_override.load();
    for (int c = kCfgs - 1; c >= 0; --c) {
      if (tov >= 0 && tov < kCfgs && c != tov) continue;
      const double cost = plan_cost(T, N, K, c, sp, cus);
      if (first || cost < best) {
        best = cost;
        *cfg = c;
        *splits = sp;
        first = false;
      }
    }
  }
}

template <int MODE, bool ZP>
hipError_t launch_mode_z(const GemmArgs& a0, hipStream_t st) {
  // Few tokens: one wave a workgroup, a thin tile (32 or 64 channels x 16 or
  // 32 tokens), three 128-byte slices in flight, weight loads non-temporal.
  // Three slices rather than four keep 7 (32 x 16) or 3 (64 x 32) workgroups
  // on a CU (LDS-bound), so that the 175B-width decode shapes (N = 49152)
  // run in a single wave of workgroups.
  constexpr int FM = MODE == MODE_FUSED ? MODE_FUSED_X : MODE;
  if (a0.T <= 4 && gemv_supported(a0)) return launch_gemv(a0, MODE == MODE_FUSED, st);
  if (a0.T <= 16) return launch_cfg<32, 16, 32, 16, 3, 128, FM, true, ZP>(a0, st);
  if (a0.T <= kFewT) return launch_cfg<64, 32, 64, 32, 3, 128, FM, true, ZP>(a0, st);
  GemmArgs a = a0;
  if (MODE != MODE_FUSED || a.splits < 1 || !a.part) a.splits = 1;
  int64_t cfg = a.cfg, sp = 1;
  if (cfg < 0 || cfg >= kCfgs) {  // no plan: the best unsplit configuration
    choose_wide(a.T, a.N, a.K, false, &cfg, &sp);
    a.splits = 1;
  }
  if constexpr (MODE == MODE_FUSED) {
    if (a.splits > 1) {  // split K: partial tiles, then one combine launch
      hipError_t e;
      GemmArgs c = a;  // (the partial launch clears the mask)
      c.clear_mask = nullptr;
      if (cfg == 0) {
        e = launch_cfg<320, 256, 80, 128, 2, 128, MODE_PART>(a, st);
        return e != hipSuccess ? e : launch_cfg<320, 256, 80, 128, 2, 128, MODE_COMBINE, false, ZP>(c, st);
      }
      if (cfg == 2) {
        e = launch_cfg<192, 256, 48, 128, 2, 128, MODE_PART>(a, st);
        return e != hipSuccess ? e : launch_cfg<192, 256, 48, 128, 2, 128, MODE_COMBINE, false, ZP>(c, st);
      }
      if (cfg == 3) {
        e = launch_cfg<320, 128, 80, 64, 2, 128, MODE_PART>(a, st);
        return e != hipSuccess ? e : launch_cfg<320, 128, 80, 64, 2, 128, MODE_COMBINE, false, ZP>(c, st);
      }
      e = launch_cfg<256, 256, 64, 128, 2, 128, MODE_PART>(a, st);
      return e != hipSuccess ? e
                             : launch_cfg<256, 256, 64, 128, 2, 128, MODE_COMBINE, false, ZP>(c, st);
    }
  }
  if (cfg == 0) return launch_cfg<320, 256, 80, 128, 2, 128, MODE, false, ZP>(a, st);
  if (cfg == 2) return launch_cfg<192, 256, 48, 128, 2, 128, MODE, false, ZP>(a, st);
  if (cfg == 3) return launch_cfg<320, 128, 80, 64, 2, 128, MODE, false, ZP>(a, st);
  return launch_cfg<256, 256, 64, 128, 2, 128, MODE, false, ZP>(a, st);
}

template <int MODE>
hipError_t launch_mode(const GemmArgs& a, hipStream_t st) {
  if constexpr (MODE == MODE_FUSED) {
    if (a.zp) return launch_mode_z<MODE, true>(a, st);
  }
  return launch_mode_z<MODE, false>(a, st);
}
}  // namespace

void set_split_override(int64_t splits) { g_split_override.store(splits > 0 ? splits : 0); }
void set_tile_override(int64_t cfg) { g_tile_override.store(cfg >= 0 && cfg < kCfgs ? cfg : -1); }
int64_t split_override() { return g_split_override.load(); }

GemmPlan plan_gemm_i8(int64_t T, int64_t N, int64_t K) {
  GemmPlan p{-1, 1, 0, 0};
  if (T <= kFewT || K % 16 != 0 || K <= 0) return p;
  choose_wide(T, N, K, true, &p.cfg, &p.splits);
  p.tiles = ceil_div(N, kCfgBM[p.cfg]) * ceil_div(T, kCfgBN[p.cfg]);
  if (p.splits > 1) p.part_elems = p.splits * p.tiles * kCfgBM[p.cfg] * kCfgBN[p.cfg];
  return p;
}

bool gemm_i8_supported(const GemmArgs& a) {
  // 16-byte aligned rows and operands (Wo, Xo null for the int32 product),
  // the rows of one tile (at most 512 of an operand) addressable with 31-bit
  // offsets; the operands themselves may exceed 2^32 bytes
  const int64_t lim = (int64_t)1 << 31, rows = 512;
  return (a.K % 16 == 0) && (a.lda % 16 == 0) && (a.ldb % 16 == 0) &&
         ((((uintptr_t)a.A) & 15) == 0) && ((((uintptr_t)a.B) & 15) == 0) &&
         ((((uintptr_t)a.Wo) & 15) == 0) && ((((uintptr_t)a.Xo) & 15) == 0) &&
         ((a.ldo * 2) % 16 == 0) && rows * a.lda < lim && rows * a.ldb < lim &&
         rows * a.ldo * 2 < lim;
}

hipError_t launch_gemm_i8_s32(const GemmArgs& a, hipStream_t st) {
  return launch_mode<MODE_I32>(a, st);
}

hipError_t launch_gemm_i8_fused(const GemmArgs& a, hipStream_t st) {
  return launch_mode<MODE_FUSED>(a, st);
}

}  // namespace i8mm
