// Bandwidth-bound kernels of the LLM.int8() layer on gfx950:
//   k_wquant    weight -> CB/SCB (absmax per output channel)
//   k_zero_words zero-fills a workspace head (outlier mask) at init
//   k_detect    column flags |x| >= threshold, OR-ed into the mask
//   k_compact   mask -> ascending outlier list O and counts (stage entry)
//   k_prep      outlier list from the mask, masked row absmax, int8 codes,
//               X[:,O] gather, dequantized weight rows CB[:,O]*SCB/127
//   k_rows      steps 1-2 of up to 8 rows (one- to eight-token calls) in one launch
//
// The method: Hugging Face LLM.int8() summary (agentlenshq.com), section
// "LLM.int8() の核心アイデア" steps 1-2; absmax rule from its section
// "量子化の仕組み"; CB/SCB storage from "transformers への統合".
#include <cstring>

#include "common.h"
#include "kernels.h"

namespace i8mm {

// ---------------------------------------------------------------------------
// Weight quantization: one workgroup per output channel j (row of W[N,K]).
// Pass 1 takes the row absmax (exact: the max of fp16 magnitudes), pass 2
// writes the codes.  A thread keeps up to kWqCache 16-byte chunks of the row
// in registers between the passes (K <= 16384), all requested at once
// (buffer loads: chunks past the row read 0); chunks beyond are read again.
// ---------------------------------------------------------------------------
constexpr int kWqCache = 8;
template <bool VEC>
__global__ __launch_bounds__(256) void k_wquant(const _Float16* __restrict__ W, int64_t K,
                                                int8_t* __restrict__ CB, float* __restrict__ SCB) {
  // (buffer resources are amdgcn-only; the host pass needs the signature)
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ float red[4];
  const int64_t j = blockIdx.x;
  const _Float16* row = W + j * K;
  int8_t* out = CB + j * K;
  float m = 0.0f;
  v8h cache[VEC ? kWqCache : 1];
  if (VEC) {
    const int64_t nc = K / 8;
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(row, (uint32_t)(nc * 16));
#pragma unroll
    for (int u = 0; u < kWqCache; ++u)
      cache[u] = __builtin_bit_cast(
          v8h, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)(threadIdx.x + 256 * u) * 16, 0, 0));
#pragma unroll
    for (int u = 0; u < kWqCache; ++u) m = fmaxf(m, absmax8(cache[u]));
    for (int64_t c = threadIdx.x + 256 * kWqCache; c < nc; c += 256)
      m = fmaxf(m, absmax8(*(const v8h*)(row + c * 8)));
  } else {
    for (int64_t k = threadIdx.x; k < K; k += 256) m = fmaxf(m, fabsf(h2f(row[k])));
  }
  const float s = block_max<256>(m, red);
  const float r = code_recip(s);
  if (threadIdx.x == 0) SCB[j] = s;
  if (VEC) {
    const int64_t nc = K / 8;
#pragma unroll
    for (int u = 0; u < kWqCache; ++u) {
      const int64_t c = threadIdx.x + 256 * u;
      if (c < nc) *(v2u*)(out + c * 8) = absmax_codes8(cache[u], s, r);
    }
    for (int64_t c = threadIdx.x + 256 * kWqCache; c < nc; c += 256)
      *(v2u*)(out + c * 8) = absmax_codes8(*(const v8h*)(row + c * 8), s, r);
  } else {
    for (int64_t k = threadIdx.x; k < K; k += 256)
      out[k] = (int8_t)absmax_code(h2f(row[k]), s, r);
  }
#endif
}

// One wave per row (16-byte aligned rows of up to 64 * 8 * CPL values): the
// whole row in registers (lane l holds chunks l, l + 64, ...: each load
// instruction reads 1 KB of the row), the absmax across the wave with no
// barrier, codes written 512 bytes an instruction.  A 256-thread workgroup
// per row spent its time in the block reduction's barriers and in its
// dependent load-reduce-store chain: 20480 x 5120 took 70 us (4.5 TB/s of
// reads and writes), 16384 x 4096 58 us; one wave per row with exactly the
// row's chunks in registers: 54 us (5.8 TB/s, 72 % of HBM) and 42 us.
template <int CPL>
__global__ __launch_bounds__(256) void k_wquant_rows(const _Float16* __restrict__ W, int64_t N,
                                                     int64_t K, int8_t* __restrict__ CB,
                                                     float* __restrict__ SCB) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= N) return;  // (wave-uniform)
  const int64_t nc = K / 8;
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(W + j * K, (uint32_t)(nc * 16));
  v8h c[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u)
    c[u] = __builtin_bit_cast(
        v8h, __builtin_amdgcn_raw_buffer_load_b128(rr, (lane + 64 * u) * 16, 0, 2));
  float m = 0.0f;
#pragma unroll
  for (int u = 0; u < CPL; ++u) m = fmaxf(m, absmax8(c[u]));
  const float s = wave_max(m);
  const float r = code_recip(s);
  if (lane == 0) SCB[j] = s;
  int8_t* out = CB + j * K;
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int64_t ci = lane + 64 * u;
    if (ci < nc) *(v2u*)(out + ci * 8) = absmax_codes8(c[u], s, r);
  }
#endif
}

template <int CPL>
bool launch_wquant_rows(const _Float16* W, int64_t N, int64_t K, int8_t* CB, float* SCB,
                        hipStream_t st) {
  if (ceil_div(K / 8, 64) > CPL) return false;
  k_wquant_rows<CPL><<<dim3((unsigned)ceil_div(N, 4)), dim3(256), 0, st>>>(W, N, K, CB, SCB);
  return true;
}

void launch_wquant(const _Float16* W, int64_t N, int64_t K, int8_t* CB, float* SCB, bool vec,
                   hipStream_t st) {
  // (rows longer than 12288 values: the workgroup-per-row kernel, whose
  // registers do not grow with K, measured faster -- K = 20480: 64 against
  // 69 us)
  if (vec && (launch_wquant_rows<8>(W, N, K, CB, SCB, st) ||
              launch_wquant_rows<10>(W, N, K, CB, SCB, st) ||
              launch_wquant_rows<12>(W, N, K, CB, SCB, st) ||
              launch_wquant_rows<16>(W, N, K, CB, SCB, st) ||
              launch_wquant_rows<24>(W, N, K, CB, SCB, st)))
    return;
  if (vec)
    k_wquant<true><<<dim3((unsigned)N), dim3(256), 0, st>>>(W, K, CB, SCB);
  else
    k_wquant<false><<<dim3((unsigned)N), dim3(256), 0, st>>>(W, K, CB, SCB);
}

// ---------------------------------------------------------------------------
// Outlier detection.  k_detect takes a slab of 512 columns (a lane owns 8
// consecutive ones: one 16-byte load per row) over a block of rows (the 4
// waves split the rows, every load of a lane issued before the first
// compare) and ORs the non-zero flag words of its slab into the global mask.
// Outlier columns are rare, so are the atomics; OR is order-independent, so
// the mask is the same whatever the schedule.  Blocks of 16 rows: a 21 MB
// read (2048 x 5120) measured 5.1 us from HBM against 7.2 us with 32-row
// blocks (more workgroups in flight at once).
// ---------------------------------------------------------------------------
__global__ void k_zero_words(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

void launch_zero_words(uint32_t* p, int64_t n, hipStream_t st) {
  if (n > 0) k_zero_words<<<dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st>>>(p, n);
}

constexpr int64_t kDetectRows = 16;

template <bool VEC>
__global__ __launch_bounds__(256) void k_detect(const _Float16* __restrict__ X, int64_t T,
                                                int64_t K, int64_t rows_per_block, float thr,
                                                uint32_t* __restrict__ mask, int64_t KW) {
  __shared__ uint32_t fl[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * 512 + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(T, r0 + rows_per_block);
  uint32_t f = 0;
  if (VEC) {
    if (c0 < K) {
      const _Float16* p = X + c0;
#pragma unroll 4
      for (int64_t r = r0 + w; r < r1; r += 4) {
        v8h v = *(const v8h*)(p + r * K);
#pragma unroll
        for (int e = 0; e < 8; ++e) f |= (uint32_t)(fabsf(h2f(v[e])) >= thr) << e;
      }
    }
  } else {
    for (int64_t r = r0 + w; r < r1; r += 4)
      for (int e = 0; e < 8; ++e)
        if (c0 + e < K) f |= (uint32_t)(fabsf(h2f(X[r * K + c0 + e])) >= thr) << e;
  }
  fl[w][lane] = f;
  __syncthreads();
  if (w == 0) {
    const uint32_t g = fl[0][lane] | fl[1][lane] | fl[2][lane] | fl[3][lane];
    uint32_t word = g << (8 * (lane & 3));
    word |= __shfl_xor(word, 1, 64);
    word |= __shfl_xor(word, 2, 64);
    const int64_t wi = ((int64_t)blockIdx.x * 512 + lane * 8) / 32;
    if ((lane & 3) == 0 && wi < KW && word) atomicOr(&mask[wi], word);
  }
}

void launch_detect(const _Float16* X, int64_t T, int64_t K, float thr, uint32_t* mask, bool clear,
                   bool vec, hipStream_t st) {
  const int64_t KW = ceil_div(K, 32);
  if (clear) launch_zero_words(mask, KW, st);
  if (T <= 0 || K <= 0) return;
  const int64_t rpb = kDetectRows;
  dim3 g((unsigned)ceil_div(K, 512), (unsigned)ceil_div(T, rpb));
  if (vec)
    k_detect<true><<<g, dim3(256), 0, st>>>(X, T, K, rpb, thr, mask, KW);
  else
    k_detect<false><<<g, dim3(256), 0, st>>>(X, T, K, rpb, thr, mask, KW);
}

// ---------------------------------------------------------------------------
// The outlier set from its bit mask, inside one workgroup of NT threads:
// smask[KW] <- mask, spref[w] = number of set bits in words < w (an
// exclusive scan of popcounts in ascending word order), spref[KW] = n_o.
// The o-th outlier column is then the q-th set bit of the word with
// spref[w] <= o < spref[w+1], so enumerating words in order yields O
// ascending, without duplicates and without sorting.
// ---------------------------------------------------------------------------
// The same, with smask[KW] already filled by the calling threads (not yet
// synchronized).
template <int NT>
__device__ int outlier_scan_lds(int64_t KW, uint32_t* smask, int32_t* spref, int32_t* wsum) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __syncthreads();
  const int64_t per = ceil_div(KW, NT);
  const int64_t w0 = tid * per, w1 = min(KW, w0 + per);
  int run = 0;
  for (int64_t w = w0; w < w1; ++w) run += __popc(smask[w]);
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, n_o = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    base += i < wave ? wsum[i] : 0;
    n_o += wsum[i];
  }
  int acc = base + incl - run;
  for (int64_t w = w0; w < w1; ++w) {
    spref[w] = acc;
    acc += __popc(smask[w]);
  }
  if (tid == 0) spref[KW] = n_o;
  __syncthreads();
  return n_o;
}

template <int NT>
__device__ int outlier_scan(const uint32_t* __restrict__ mask, int64_t KW, uint32_t* smask,
                            int32_t* spref, int32_t* wsum) {
  for (int64_t w = threadIdx.x; w < KW; w += NT) smask[w] = mask[w];
  return outlier_scan_lds<NT>(KW, smask, spref, wsum);
}

// O[o] for o < cap (ascending), into `dst` (global or LDS)
template <int NT, typename I>
__device__ void outlier_list(const uint32_t* smask, const int32_t* spref, int64_t KW, int64_t cap,
                             I* dst) {
  for (int64_t w = threadIdx.x; w < KW; w += NT) {
    uint32_t m = smask[w];
    int64_t o = spref[w];
    while (m && o < cap) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      dst[o++] = (I)(w * 32 + b);
    }
  }
}

// Stage entry point only: mask -> O (first max_o entries) and counts.
__global__ __launch_bounds__(1024) void k_compact(const uint32_t* __restrict__ mask, int64_t KW,
                                                  int32_t* __restrict__ O,
                                                  int32_t* __restrict__ counts, int64_t max_o) {
  extern __shared__ __attribute__((aligned(16))) uint32_t sm[];
  __shared__ int32_t wsum[16];
  uint32_t* smask = sm;
  int32_t* spref = (int32_t*)(sm + KW);
  const int n_o = outlier_scan<1024>(mask, KW, smask, spref, wsum);
  outlier_list<1024>(smask, spref, KW, max_o, O);
  if (threadIdx.x == 0) {
    counts[0] = n_o;
    counts[1] = (int64_t)n_o > max_o ? 1 : 0;
    counts[2] = 0;
    counts[3] = 0;
  }
}

void launch_compact(const uint32_t* mask, int64_t K, int32_t* O, int32_t* counts, int64_t max_o,
                    hipStream_t st) {
  const int64_t KW = ceil_div(K, 32);
  const size_t lds = (size_t)(2 * KW + 1) * 4;
  (void)lds_limit<k_compact>((size_t)(2 * ceil_div(kMaxK, 32) + 1) * 4);
  k_compact<<<dim3(1), dim3(1024), lds, st>>>(mask, KW, O, counts, max_o);
}

// ---------------------------------------------------------------------------
// Step 2 preparation, one launch.  Every workgroup rebuilds the outlier set
// from the mask (outlier_scan) and, when it has at most ocap columns, the
// list O in LDS.
//   workgroup 0 also publishes O and counts (n_o, overflow);
//   workgroups [0, R = ceil(T/RPB)): RPB rows of X each, 256/RPB threads a
//     row: masked absmax -> sx, codes -> Xq (0 on outlier and pad columns),
//     X[:, O] -> Xo (0 on pad columns);
//   workgroups [R, R + ceil(N/16)): 16 output channels each:
//     Wo[j, o] = fp16(fl32(fl32(CB[j, O[o]] * SCB[j]) / 127)), 0 on pad
//     (skipped for outlier sets of at most wo_skip columns, which the
//     few-token product kernel extracts itself).
// A row workgroup issues its loads of X before rebuilding the outlier set
// (they do not depend on it), so the two latencies overlap.  O is
// ascending, so the gathers of consecutive o by consecutive lanes read
// increasing addresses of one row; stores of Xo/Wo rows are coalesced.
// Wide sets (at least one column in 64, at most 4096) stream whole CB rows
// through LDS instead of gathering, two rows in flight a workgroup; sets
// beyond ocap fall back to enumerating the mask per row.
// LDS: mask[KW], pref[KW + 1], O[ocap]; for the wide sets, two row buffers
// over them.
// ---------------------------------------------------------------------------
constexpr int kChansPerWoBlock = 16;
constexpr int64_t kFewChanGroups = 64;  // channel workgroups of a few-token call
constexpr int kMaskWords = 2;  // mask words a thread requests before the row
constexpr int kRowChunks = 4;  // 4 KB pieces of a streamed CB row (K <= 16384)
// Wide outlier sets of at most 256 * kWoRingCols columns: a thread keeps the
// column of each of its outputs o = tid + 256 m in registers.
constexpr int kWoRingCols = 16;
// LDS of the step-2 kernel: mask[KW], pref[KW + 1], O[ocap], and at least
// two CB rows rounded up to 4 KB plus a spare 1 KB where the wide-set Wo
// build can run (16-byte multiples K <= 16384)
constexpr size_t prep_lds_total(int64_t K, int64_t ocap) {
  const size_t a = prep_lds_bytes(K, ocap);
  const size_t b = K % 16 == 0 && K <= 256 * kRowChunks * 16
                       ? (size_t)(2 * ((K + 4095) / 4096) * 4096 + 1024)
                       : 0;
  return a > b ? a : b;
}
// Eight signed bytes from LDS addresses a[0..7], read and waited for in one
// asm block: the compiler's own wait before an LDS read, while loads into
// LDS are in flight, covers all of them (it cannot tell the row buffers
// apart) and would drain the loads of the rows after this one.
__device__ __forceinline__ void lds_bytes8(const uint32_t (&a)[8], int (&c)[8]) {
  asm volatile(
      "ds_read_i8 %0, %8\n\t"
      "ds_read_i8 %1, %9\n\t"
      "ds_read_i8 %2, %10\n\t"
      "ds_read_i8 %3, %11\n\t"
      "ds_read_i8 %4, %12\n\t"
      "ds_read_i8 %5, %13\n\t"
      "ds_read_i8 %6, %14\n\t"
      "ds_read_i8 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(c[4]), "=&v"(c[5]),
        "=&v"(c[6]), "=&v"(c[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
}
// wait until at most N of this wave's vector memory operations are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// One row per workgroup measured best across the first-FF shapes (2 and 4
// rows per workgroup: 13B-scale 12.2 / 10.9 us against 11.8 us, 175B-scale
// 51 / 60 us against 46 us, 32-token decode 10 / 16 us against 7 us).
constexpr int kRowsPerPrepBlock = 1;

// RPB rows of X per workgroup, 256 / RPB threads (whole waves) per row
// F16W: the outlier weights are copied from an fp16 weight W16 [N][K]
// instead of dequantized from CB (the fp16-weight variant of the layer).
// ZP: zero-point row codes (sx = range / 2 and the offset Z per row, to zp)
// instead of absmax ones, and the weight-side sum of each channel's outlier
// codes, osum[j] = sum_o CB[j, O_o] (for the product's offset correction).
template <bool VEC, int RPB, bool F16W, bool ZP>
__global__ __launch_bounds__(256) void k_prep(
    const _Float16* __restrict__ X, int64_t T, int64_t K, const uint32_t* __restrict__ mask,
    int32_t* __restrict__ O_out, int32_t* __restrict__ counts, int64_t max_o,
    int8_t* __restrict__ Xq, int64_t ldq, float* __restrict__ sx, _Float16* __restrict__ Xo,
    int64_t ldo, int64_t nrowblk, const int8_t* __restrict__ CB, const float* __restrict__ SCB,
    int64_t N, _Float16* __restrict__ Wo, int64_t ocap, int64_t wo_skip,
    const _Float16* __restrict__ W16, int32_t* __restrict__ zp, int32_t* __restrict__ osum,
    int64_t nwoblk) {
  // The body uses amdgcn-only types (buffer resources); the host pass only
  // needs the kernel's signature to emit its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int TPR = 256 / RPB;                        // threads per row
  constexpr int kCachedChunks = RPB == 1 ? 4 : RPB == 2 ? 6 : 10;  // chunks a thread keeps
  extern __shared__ __attribute__((aligned(16))) uint32_t sm[];
  __shared__ int32_t wsum[4];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int rt = tid % TPR;  // thread within its row
  const int64_t KW = ceil_div(K, 32);
  uint32_t* smask = sm;
  int32_t* spref = (int32_t*)(sm + KW);
  int32_t* sO = spref + KW + 1;

  // The mask words are requested first and the row's X chunks right after:
  // loads complete in order, so the scan waits only for the mask while the
  // X loads are still in flight.
  // (Buffer loads: out-of-range offsets read 0 and touch no memory, so every
  // workgroup runs the same straight-line loads -- the channel workgroups
  // with an empty row range -- and the compiler can wait for the mask alone.)
  const __amdgpu_buffer_rsrc_t rmask = make_rsrc(mask, (uint32_t)(KW * 4));
  uint32_t mw[kMaskWords];
#pragma unroll
  for (int u = 0; u < kMaskWords; ++u)
    mw[u] = __builtin_amdgcn_raw_buffer_load_b32(rmask, (tid + 256 * u) * 4, 0, 0);
  __builtin_amdgcn_sched_barrier(0);  // keep the mask loads ahead of the row's
  const bool row_block = (int64_t)blockIdx.x < nrowblk;
  // the row of this thread's wave (wave-uniform: a row spans whole waves)
  const int64_t i = (int64_t)blockIdx.x * RPB + __builtin_amdgcn_readfirstlane(tid / TPR);
  const bool row_ok = row_block && i < T;
  const _Float16* row = X + (row_ok ? i * K : 0);
  const int64_t nc = K / 8;
  v8h cache[kCachedChunks];
  if (VEC) {
    // chunks rt + TPR*u stay in registers between the two passes; chunks
    // beyond kCachedChunks per thread are read again (an L2 hit)
    const __amdgpu_buffer_rsrc_t rrow = make_rsrc(row, row_ok ? (uint32_t)(nc * 16) : 0u);
#pragma unroll
    for (int u = 0; u < kCachedChunks; ++u)
      cache[u] = __builtin_bit_cast(
          v8h, __builtin_amdgcn_raw_buffer_load_b128(rrow, (rt + TPR * u) * 16, 0, 0));
  }
  // unconditional stores (a conditional one lets the compiler sink its load
  // behind the row's): words past the mask are 0 and land in smask[KW], the
  // first prefix slot, which the scan writes after its first barrier
#pragma unroll
  for (int u = 0; u < kMaskWords; ++u) {
    const int64_t w = tid + 256 * u;
    smask[w < KW ? w : KW] = mw[u];
  }
  for (int64_t w = tid + 256 * kMaskWords; w < KW; w += 256) smask[w] = mask[w];
  const int n_o = outlier_scan_lds<256>(KW, smask, spref, wsum);
  const int64_t n_use = (int64_t)n_o < max_o ? n_o : max_o;
  const int64_t n_pad = round_up(n_use, 32);
  const bool listed = n_use <= ocap;
  // Wide outlier sets (at least one column in 64, at most 256 * kWoRingCols
  // of them) touch nearly every cache line of a CB row: the channel
  // workgroups then stream whole rows instead of gathering -- see below.
  const bool wo_ring = !F16W && !ZP && !row_block && n_use * 64 >= K && K % 16 == 0 &&
                       K <= 256 * kRowChunks * 16 && (((uintptr_t)CB) & 15) == 0 && listed &&
                       n_use <= 256 * kWoRingCols;
  if (listed) outlier_list<256>(smask, spref, KW, n_use, sO);
  if (blockIdx.x == 0 && counts) {
    outlier_list<256>(smask, spref, KW, max_o, O_out);
    if (tid == 0) {
      counts[0] = n_o;
      counts[1] = (int64_t)n_o > max_o ? 1 : 0;
      counts[2] = 0;
      counts[3] = 0;
    }
  }
  __syncthreads();

  if (row_block) {
    // ---- RPB rows of X, TPR threads each
    // max over the TPR threads of a row (every thread of the block calls it)
    auto row_max = [&](float v) {
      v = wave_max(v);
      if constexpr (TPR > 64) {
        constexpr int WPR = TPR / 64;
        const int w = tid >> 6;
        if ((tid & 63) == 0) red[w] = v;
        __syncthreads();
        const int w0 = w - w % WPR;
        v = red[w0];
#pragma unroll
        for (int q = 1; q < WPR; ++q) v = fmaxf(v, red[w0 + q]);
      }
      return v;
    };
    int8_t* qrow = Xq + (row_ok ? i : 0) * ldq;
    float m = 0.0f;
    if (VEC && ZP) {
      // zero-point: the kept values' range, with 0 in it (outlier columns
      // zeroed first change neither end), then codes with outliers at 0
      auto chunk_bits = [&](int64_t c) { return smask[c >> 2] >> (8 * (c & 3)); };
      float lo = 0.0f, hi = 0.0f;
#pragma unroll
      for (int u = 0; u < kCachedChunks; ++u) {
        const int64_t c = rt + TPR * u;
        if (c < nc) {
          cache[u] = zero_masked8(cache[u], chunk_bits(c));
          minmax8(cache[u], lo, hi);
        }
      }
      if (row_ok)
        for (int64_t c = rt + TPR * kCachedChunks; c < nc; c += TPR)
          minmax8(zero_masked8(*(const v8h*)(row + c * 8), chunk_bits(c)), lo, hi);
      const float hi_r = row_max(hi);
      __syncthreads();  // row_max's scratch is reused
      const float lo_r = -row_max(-lo);
      if (!row_ok) return;
      const ZpRow z = zp_row(lo_r, hi_r);
      if (rt == 0) {
        sx[i] = z.sx;
        zp[i] = z.Z;
      }
#pragma unroll
      for (int u = 0; u < kCachedChunks; ++u) {
        const int64_t c = rt + TPR * u;
        if (c < nc) *(v2u*)(qrow + c * 8) = zp_codes8(cache[u], chunk_bits(c), z);
      }
      for (int64_t c = rt + TPR * kCachedChunks; c < nc; c += TPR)
        *(v2u*)(qrow + c * 8) = zp_codes8(*(const v8h*)(row + c * 8), chunk_bits(c), z);
      for (int64_t k = K + rt; k < ldq; k += TPR) qrow[k] = 0;
    } else if (ZP) {
      float lo = 0.0f, hi = 0.0f;
      if (row_ok)
        for (int64_t k = rt; k < K; k += TPR)
          if (!((smask[k >> 5] >> (k & 31)) & 1u)) {
            const float x = h2f(row[k]);
            lo = fminf(lo, x);
            hi = fmaxf(hi, x);
          }
      const float hi_r = row_max(hi);
      __syncthreads();
      const float lo_r = -row_max(-lo);
      if (!row_ok) return;
      const ZpRow z = zp_row(lo_r, hi_r);
      if (rt == 0) {
        sx[i] = z.sx;
        zp[i] = z.Z;
      }
      for (int64_t k = rt; k < ldq; k += TPR) {
        int8_t q = 0;
        if (k < K && !((smask[k >> 5] >> (k & 31)) & 1u)) q = (int8_t)zp_code(h2f(row[k]), z);
        qrow[k] = q;
      }
    } else if (VEC) {
      // outlier columns are zeroed in the chunk first (rare); then the row
      // absmax and the codes need no per-element test
      auto chunk_bits = [&](int64_t c) { return smask[c >> 2] >> (8 * (c & 3)); };
#pragma unroll
      for (int u = 0; u < kCachedChunks; ++u) {
        const int64_t c = rt + TPR * u;
        if (c < nc) {
          cache[u] = zero_masked8(cache[u], chunk_bits(c));
          m = fmaxf(m, absmax8(cache[u]));
        }
      }
      if (row_ok)
        for (int64_t c = rt + TPR * kCachedChunks; c < nc; c += TPR)
          m = fmaxf(m, absmax8(zero_masked8(*(const v8h*)(row + c * 8), chunk_bits(c))));
      const float s = row_max(m);
      if (!row_ok) return;
      const float rs = code_recip(s);
      if (rt == 0) sx[i] = s;
#pragma unroll
      for (int u = 0; u < kCachedChunks; ++u) {
        const int64_t c = rt + TPR * u;
        if (c < nc) *(v2u*)(qrow + c * 8) = absmax_codes8(cache[u], s, rs);
      }
      for (int64_t c = rt + TPR * kCachedChunks; c < nc; c += TPR)
        *(v2u*)(qrow + c * 8) =
            absmax_codes8(zero_masked8(*(const v8h*)(row + c * 8), chunk_bits(c)), s, rs);
      for (int64_t k = K + rt; k < ldq; k += TPR) qrow[k] = 0;
    } else {
      if (row_ok)
        for (int64_t k = rt; k < K; k += TPR)
          if (!((smask[k >> 5] >> (k & 31)) & 1u)) m = fmaxf(m, fabsf(h2f(row[k])));
      const float s = row_max(m);
      if (!row_ok) return;
      const float rs = code_recip(s);
      if (rt == 0) sx[i] = s;
      for (int64_t k = rt; k < ldq; k += TPR) {
        int8_t q = 0;
        if (k < K && !((smask[k >> 5] >> (k & 31)) & 1u))
          q = (int8_t)absmax_code(h2f(row[k]), s, rs);
        qrow[k] = q;
      }
    }
    // X[i, O] -> Xo[i, :]
    _Float16* xorow = Xo + i * ldo;
    if (listed) {
      for (int64_t o0 = 0; o0 < n_pad; o0 += 4 * TPR) {
        _Float16 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t o = o0 + u * TPR + rt;
          v[u] = o < n_use ? row[sO[o]] : (_Float16)0.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t o = o0 + u * TPR + rt;
          if (o < n_pad) xorow[o] = v[u];
        }
      }
    } else {
      for (int64_t w = rt; w < KW; w += TPR) {
        uint32_t mb = smask[w];
        int64_t o = spref[w];
        while (mb && o < n_use) {
          const int b = __ffs(mb) - 1;
          mb &= mb - 1;
          xorow[o++] = row[w * 32 + b];
        }
      }
      for (int64_t o = n_use + rt; o < n_pad; o += TPR) xorow[o] = (_Float16)0.0f;
    }
    return;
  }

  // ---- dequantized outlier weight rows, blocks of 16 channels: block
  // blockIdx.x - nrowblk, then every (channel workgroups)-th one after it
  if (n_pad == 0 || n_use <= wo_skip) return;
  if (wo_ring) {
    // Rows streamed whole through two LDS row buffers (the mask, prefix and
    // list are read before them and not after): row r + 2 is loaded straight
    // into LDS, one 1 KB piece a wave and load, while row r is picked; each
    // thread writes its outputs o = tid + 256 m of the row (coalesced) from
    // the columns it holds.  Rows past the block load nothing (an empty
    // buffer range reads 0), and pieces past K go to a spare 1 KB, so every
    // row issues 4 loads and every pick 16 stores: the wait for row r counts
    // the 20 issued after its loads.  (Its own loop: the other paths' loop
    // invariants are not held in registers through it.)
    uint32_t wcol[kWoRingCols / 2];  // two 16-bit columns a register (K <= 16384)
#pragma unroll
    for (int m = 0; m < kWoRingCols; m += 2) {
      const int64_t o = tid + 256 * m;
      const uint32_t c0 = o < n_use ? (uint32_t)sO[o] : 0u;
      const uint32_t c1 = o + 256 < n_use ? (uint32_t)sO[o + 256] : 0u;
      wcol[m / 2] = c0 | (c1 << 16);
    }
    __syncthreads();  // the row buffers overlay the list
    const int64_t rbytes = round_up(K, (int64_t)4096);
    char* lbase = (char*)sm;
    char* spare = lbase + 2 * rbytes;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int64_t blk = (int64_t)blockIdx.x - nrowblk; blk < nwoblk;
         blk += (int64_t)gridDim.x - nrowblk) {
      const int64_t j0 = blk * kChansPerWoBlock;
      const int64_t nch = min((int64_t)kChansPerWoBlock, N - j0);
      auto load_row = [&](int64_t buf, int64_t r) {
        const bool in = r < nch;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(CB + (in ? (j0 + r) * K : 0), in ? (uint32_t)K : 0u);
        int t = tid;
        asm volatile("" : "+v"(t));
#pragma unroll
        for (int u = 0; u < kRowChunks; ++u) {
          char* dst = 4096 * u < K ? lbase + buf * rbytes + 4096 * u + 1024 * wave : spare;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (__attribute__((address_space(3))) void*)dst, 16, (uint32_t)(t * 16 + 4096 * u),
              0, 0, 0);
        }
      };
      // (stores through a buffer range of the row's n_pad outputs: those
      // past it, and all of a row outside the block, are dropped)
      auto take_row = [&](int64_t buf, int64_t r) {
        const bool in = r >= 0 && r < nch;
        const int64_t j = j0 + (in ? r : 0);
        const float sj = SCB[j];
        const __amdgpu_buffer_rsrc_t rw =
            make_rsrc(Wo + j * ldo, in ? (uint32_t)(n_pad * 2) : 0u);
        const char* srow = lbase + buf * rbytes;
        // (the thread index and packed columns made opaque here: the 16
        // addresses, offsets and predicates derived from them are not
        // hoisted out of the row loop into registers of their own)
        int t = tid;
        asm volatile("" : "+v"(t));
#pragma unroll
        for (int m = 0; m < kWoRingCols / 2; ++m) asm volatile("" : "+v"(wcol[m]));
        const uint32_t lrow =
            (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)srow;
        // two batches of 8 outputs (LDS reads, then dequantize and store)
#pragma unroll
        for (int m0 = 0; m0 < kWoRingCols; m0 += 8) {
          uint32_t ad[8];
#pragma unroll
          for (int m = 0; m < 8; ++m) ad[m] = lrow + ((wcol[(m0 + m) / 2] >> (16 * (m & 1))) & 0xffffu);
          int code[8];
          lds_bytes8(ad, code);
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const int o = t + 256 * (m0 + m);
            const unsigned short h =
                __builtin_bit_cast(unsigned short, dequant_weight(code[m], sj));
            __builtin_amdgcn_raw_buffer_store_b16(o < n_use ? h : (unsigned short)0, rw, o * 2,
                                                  0, 0);
          }
        }
      };
      load_row(0, 0);
      take_row(1, -1);
      load_row(1, 1);
      // (plain barriers: a workgroup fence would wait for every load into
      // LDS in flight, the next row's too; the reads of a row are waited for
      // where they are issued)
      for (int64_t r = 0; r < nch; ++r) {
        wait_vm<4 + 16>();             // this wave's pieces of row r are in LDS
        __builtin_amdgcn_s_barrier();  // and every wave's
        take_row(r & 1, r);
        __builtin_amdgcn_s_barrier();  // the buffer is refilled next
        load_row(r & 1, r + 2);
      }
    }
    wait_vm<0>();  // no load into LDS outstanding when the workgroup ends
    return;
  }
  for (int64_t blk = (int64_t)blockIdx.x - nrowblk; blk < nwoblk;
       blk += (int64_t)gridDim.x - nrowblk) {
  const int64_t j0 = blk * kChansPerWoBlock;
  const int64_t nch = min((int64_t)kChansPerWoBlock, N - j0);
  if (listed) {
    // per wave: items (channel r, chunk u of 64 outputs), wave-uniform, so
    // the channel's row address and scale stay scalar; a lane gathers
    // output o = 64u + lane; kGather items in flight
    constexpr int kGather = 4;
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t nu = ceil_div(n_pad, 64);
    const int64_t nr = ceil_div(nch - wave, 4);  // channels wave, wave+4, ...
    const int64_t items = nr * nu;
    int64_t r0 = 0, u0 = 0;  // (channel step, chunk) of the batch's first item
    int zrun = 0;            // ZP: the current channel's outlier code sum
    for (int64_t q0 = 0; q0 < items; q0 += kGather) {
      int64_t rg[kGather], ug[kGather];
      int64_t rr = r0, uu = u0;
#pragma unroll
      for (int g = 0; g < kGather; ++g) {
        rg[g] = rr;
        ug[g] = uu;
        if (++uu == nu) {
          uu = 0;
          ++rr;
        }
      }
      r0 = rr;
      u0 = uu;
      if constexpr (F16W) {
        _Float16 h[kGather];
#pragma unroll
        for (int g = 0; g < kGather; ++g) {
          const int64_t o = ug[g] * 64 + lane;
          h[g] = (q0 + g < items && o < n_use) ? W16[(j0 + wave + 4 * rg[g]) * K + sO[o]]
                                               : (_Float16)0.0f;
        }
#pragma unroll
        for (int g = 0; g < kGather; ++g) {
          const int64_t o = ug[g] * 64 + lane;
          if (q0 + g < items && o < n_pad) Wo[(j0 + wave + 4 * rg[g]) * ldo + o] = h[g];
        }
      } else {
        int8_t c[kGather];
#pragma unroll
        for (int g = 0; g < kGather; ++g) {
          const int64_t o = ug[g] * 64 + lane;
          c[g] = (q0 + g < items && o < n_use) ? CB[(j0 + wave + 4 * rg[g]) * K + sO[o]]
                                               : (int8_t)0;
        }
        if constexpr (ZP) {
          // a channel's chunks are consecutive items of this wave
#pragma unroll
          for (int g = 0; g < kGather; ++g) {
            const int cs = wave_sum((int)c[g]);
            if (q0 + g < items) {
              zrun += cs;
              if (ug[g] == nu - 1) {
                if (lane == 0) osum[j0 + wave + 4 * rg[g]] = zrun;
                zrun = 0;
              }
            }
          }
        }
#pragma unroll
        for (int g = 0; g < kGather; ++g) {
          const int64_t o = ug[g] * 64 + lane;
          if (q0 + g < items && o < n_pad) {
            const int64_t j = j0 + wave + 4 * rg[g];
            Wo[j * ldo + o] = dequant_weight(c[g], SCB[j]);
          }
        }
      }
    }
  } else {
    const int wave = tid >> 6, lane = tid & 63;
    for (int64_t r = wave; r < nch; r += 4) {
      const int64_t j = j0 + r;
      const int8_t* cbrow = CB + j * K;
      const float sj = SCB[j];
      _Float16* worow = Wo + j * ldo;
      int cs = 0;  // ZP: this lane's part of the channel's outlier code sum
      for (int64_t w = lane; w < KW; w += 64) {
        uint32_t mb = smask[w];
        int64_t o = spref[w];
        while (mb && o < n_use) {
          const int b = __ffs(mb) - 1;
          mb &= mb - 1;
          if constexpr (F16W) {
            worow[o++] = W16[j * K + w * 32 + b];
          } else {
            const int c = cbrow[w * 32 + b];
            if constexpr (ZP) cs += c;
            worow[o++] = dequant_weight(c, sj);
          }
        }
      }
      if constexpr (ZP) {
        cs = wave_sum(cs);
        if (lane == 0) osum[j] = cs;
      }
      for (int64_t o = n_use + lane; o < n_pad; o += 64) worow[o] = (_Float16)0.0f;
    }
  }
  }  // channel blocks
#endif  // __HIP_DEVICE_COMPILE__
}

// rsum[j] = sum_k CB[j, k]: one wave per row, 16-byte loads when aligned
__global__ __launch_bounds__(256) void k_rowsum(const int8_t* __restrict__ CB, int64_t N,
                                                 int64_t K, int32_t* __restrict__ rsum) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= N) return;
  const int8_t* row = CB + j * K;
  int s = 0;
  if ((K % 16) == 0 && (((uintptr_t)CB) & 15) == 0) {
    for (int64_t c = lane; c < K / 16; c += 64) {
      const v4i v = *(const v4i*)(row + 16 * c);
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int b = 0; b < 4; ++b) s += (int)(int8_t)(v[w] >> (8 * b));
    }
  } else {
    for (int64_t k = lane; k < K; k += 64) s += row[k];
  }
  s = wave_sum(s);
  if (lane == 0) rsum[j] = s;
}

void launch_rowsum(const int8_t* CB, int64_t N, int64_t K, int32_t* rsum, hipStream_t st) {
  if (N <= 0) return;
  k_rowsum<<<dim3((unsigned)ceil_div(N, 4)), dim3(256), 0, st>>>(CB, N, K, rsum);
}

template <bool VEC, int RPB, bool F16W, bool ZP>
void launch_prep_t(const PrepArgs& p, dim3 g, size_t lds, int64_t nrowblk, hipStream_t st) {
  (void)lds_limit<k_prep<VEC, RPB, F16W, ZP>>(prep_lds_total(kMaxK, kMaxOcap));
  k_prep<VEC, RPB, F16W, ZP><<<g, dim3(256), lds, st>>>(
      p.X, p.T, p.K, p.mask, p.O_out, p.counts, p.max_o, p.Xq, p.ldq, p.sx, p.Xo, p.ldo, nrowblk,
      p.CB, p.SCB, p.N, p.Wo, p.ocap, p.wo_skip, p.W16, p.zp, p.osum,
      p.Wo ? ceil_div(p.N, kChansPerWoBlock) : 0);
}

void launch_prep(const PrepArgs& p, hipStream_t st) {
  constexpr int R = kRowsPerPrepBlock;
  const int64_t nrowblk = p.Xq ? ceil_div(p.T, R) : 0;
  int64_t nwoblk = p.Wo ? ceil_div(p.N, kChansPerWoBlock) : 0;
  // few tokens: the channel blocks go to a few workgroups, which usually
  // find nothing to do (the product picks small outlier sets out of CB);
  // launching one per block cost a few microseconds of dispatch
  // (only where the product can take the outliers itself: the fp16-weight
  // and zero-point layers always need Wo, and osum, from all blocks)
  if (p.T <= kFewT && p.wo_skip >= 0 && nwoblk > kFewChanGroups) nwoblk = kFewChanGroups;
  // (the row buffers of the wide-set Wo build: absmax layer only)
  const size_t lds =
      p.W16 || p.zp ? prep_lds_bytes(p.K, p.ocap) : prep_lds_total(p.K, p.ocap);
  const dim3 g((unsigned)(nrowblk + nwoblk > 0 ? nrowblk + nwoblk : 1));
  if (p.W16) {
    if (p.vec)
      launch_prep_t<true, R, true, false>(p, g, lds, nrowblk, st);
    else
      launch_prep_t<false, R, true, false>(p, g, lds, nrowblk, st);
  } else if (p.zp) {
    if (p.vec)
      launch_prep_t<true, R, false, true>(p, g, lds, nrowblk, st);
    else
      launch_prep_t<false, R, false, true>(p, g, lds, nrowblk, st);
  } else if (p.vec) {
    launch_prep_t<true, R, false, false>(p, g, lds, nrowblk, st);
  } else {
    launch_prep_t<false, R, false, false>(p, g, lds, nrowblk, st);
  }
}

// Y[i, j] = bias[j] (or 0): the layer with K == 0 (no columns, no outliers).
__global__ void k_fill_bias(_Float16* Y, int64_t T, int64_t N, const _Float16* bias,
                            int32_t* counts) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < T * N) Y[idx] = bias ? bias[idx % N] : (_Float16)0.0f;
  if (idx < 4) counts[idx] = 0;
}

void launch_fill_bias(_Float16* Y, int64_t T, int64_t N, const _Float16* bias, int32_t* counts,
                      hipStream_t st) {
  k_fill_bias<<<dim3((unsigned)ceil_div(T * N, 256)), dim3(256), 0, st>>>(Y, T, N, bias, counts);
}

// ---------------------------------------------------------------------------
// Steps 1-2 for up to TR rows of X (one- to eight-token calls) in one launch:
// workgroup i takes row i.  Thread t holds chunks t + NT u (8 columns each);
// the column flags need every row, so each workgroup reads all T rows
// (after the first, from L2) and ORs their flags, which for fp16 values is
// an integer test: |x| >= thr exactly when the magnitude bits of x reach
// those of the smallest fp16 value >= thr (`t16`, from the host), i.e. when
// (bits & 0x7fff) + (0x8000 - t16) carries into bit 15 -- two operations a
// pair of values, no conversion.  Every workgroup then has the same flags
// and builds the same ascending list O (an exclusive scan of the per-chunk
// counts in column order, one block-wide scan per chunk round); workgroup 0
// publishes O and the counts, workgroup i writes X[i, O], the absmax of row
// i over the other columns (a block max), its codes and sx[i] -- the values
// k_detect and k_prep produce.  (One workgroup for all rows spent its time
// in the codes of 8 x 12288 values: 24 us; one wave for one row, 21 us: its
// dependent chains had nothing to hide behind.)
// ---------------------------------------------------------------------------
template <int TR>
__global__ __launch_bounds__(512) void k_rows(
    const _Float16* __restrict__ X, int64_t T, int64_t K, uint32_t t16, int32_t* __restrict__ O,
    int32_t* __restrict__ counts, int64_t max_o, int8_t* __restrict__ Xq, int64_t ldq,
    float* __restrict__ sx, _Float16* __restrict__ Xo_, int64_t ldo) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NT = 512, NW = NT / 64, CH = (int)(kRow1MaxK / 8 / NT);
  __shared__ float red[NW];
  __shared__ int32_t wtot[CH][NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const int64_t nc = K / 8;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)(T * K * 2));
  // chunks past a row, and rows past T, read 0 (no flag)
  auto load = [&](int64_t i, int u) {
    const int64_t c = tid + NT * u;
    return __builtin_bit_cast(
        v4u, __builtin_amdgcn_raw_buffer_load_b128(
                 rx, (i < T && c < nc) ? (uint32_t)(i * K * 2 + c * 16) : 0x80000000u, 0, 0));
  };
  v4u own[CH], cv[TR][CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) own[u] = load(row, u);
  if constexpr (TR > 1) {
#pragma unroll
    for (int i = 0; i < TR; ++i)
#pragma unroll
      for (int u = 0; u < CH; ++u) cv[i][u] = load(i, u);
  }
  const uint32_t addc = (0x8000u - t16) * 0x10001u;
  auto carry = [&](const v4u& w, v4u& acc) {
#pragma unroll
    for (int d = 0; d < 4; ++d) acc[d] |= (w[d] & 0x7fff7fffu) + addc;
  };

  // flags of this thread's columns (any row); per round, the outlier count
  // of each wave (for the scan)
  uint32_t f[CH];
  int incl[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    v4u acc = v4u{0u, 0u, 0u, 0u};
    if constexpr (TR > 1) {
#pragma unroll
      for (int i = 0; i < TR; ++i) carry(cv[i][u], acc);
    } else {
      carry(own[u], acc);
    }
    uint32_t fu = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      fu |= ((acc[d] >> 15) & 1u) << (2 * d) | ((acc[d] >> 31) & 1u) << (2 * d + 1);
    f[u] = fu;
    const int cnt = __popc(fu);
    incl[u] = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl[u], o, 64);
      if (lane >= o) incl[u] += t;
    }
    if (lane == 63) wtot[u][wave] = incl[u];
  }
  __syncthreads();

  // O (first max_o entries, workgroup 0) and X[row, O]: columns in order are
  // round-major
  uint16_t* Xo = reinterpret_cast<uint16_t*>(Xo_) + row * ldo;
  int n_o = 0;
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    int before = 0, total = 0;  // outliers of this round in lower waves, in all
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int t = wtot[u][w];
      before += w < wave ? t : 0;
      total += t;
    }
    if (f[u]) {
      int pos = n_o + before + incl[u] - __popc(f[u]);
      for (uint32_t ff = f[u]; ff; ff &= ff - 1, ++pos) {
        const int e = __builtin_ctz(ff);
        if (pos < max_o) {
          if (row == 0) O[pos] = (int32_t)((tid + NT * u) * 8 + e);
          const uint32_t wd = own[u][e >> 1];
          Xo[pos] = (uint16_t)(wd >> (16 * (e & 1)));
        }
      }
    }
    n_o += total;
  }
  const int64_t n_use = n_o < max_o ? n_o : max_o;
  for (int64_t o = n_use + tid; o < round_up(n_use, 32); o += NT) Xo[o] = 0;

  // the row's absmax over the other columns, its codes (zeros on the
  // outlier columns and past K)
  float m = 0.0f;
  v8h xv[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    xv[u] = zero_masked8(__builtin_bit_cast(v8h, own[u]), f[u]);
    m = fmaxf(m, absmax8(xv[u]));
  }
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float sr = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) sr = fmaxf(sr, red[w]);
  const float rs = code_recip(sr);
  int8_t* q = Xq + row * ldq;
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int64_t c = tid + NT * u;
    if (c < nc) *(v2u*)(q + c * 8) = absmax_codes8(xv[u], sr, rs);
  }
  for (int64_t k = K + 8 * tid; k < ldq; k += 8 * NT) *(v2u*)(q + k) = v2u{0u, 0u};
  if (tid == 0) {
    sx[row] = sr;
    if (row == 0) {
      counts[0] = n_o;
      counts[1] = n_o > max_o ? 1 : 0;
      counts[2] = 0;
      counts[3] = 0;
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// The bits of the smallest fp16 value >= thr (thr > 0); above the largest
// finite fp16 value, the bits of infinity (no finite value reaches it).
static uint32_t fp16_ceil_bits(float thr) {
  if (!(thr <= 65504.0f)) return 0x7C00u;
  const _Float16 h = (_Float16)thr;  // round to nearest even
  uint16_t b;
  memcpy(&b, &h, 2);
  if ((float)h < thr) b = (uint16_t)(b + 1);  // the next fp16 value up
  return b;
}

void launch_rows(const _Float16* X, int64_t T, int64_t K, float thr, int32_t* O, int32_t* counts,
                 int64_t max_o, int8_t* Xq, int64_t ldq, float* sx, _Float16* Xo, int64_t ldo,
                 hipStream_t st) {
  const uint32_t t16 = fp16_ceil_bits(thr);
  if (T <= 1)
    k_rows<1><<<dim3(1), dim3(512), 0, st>>>(X, T, K, t16, O, counts, max_o, Xq, ldq, sx, Xo, ldo);
  else
    k_rows<kRowsMaxT><<<dim3((unsigned)T), dim3(512), 0, st>>>(X, T, K, t16, O, counts, max_o,
                                                               Xq, ldq, sx, Xo, ldo);
}

}  // namespace i8mm
