// Bandwidth-bound kernels of the LLM.int8() layer on gfx950:
//   k_wquant           weight -> CB/SCB (absmax per output channel)
//   k_detect_partial   per-row-block column flags |x| >= threshold
//   k_detect_compact   OR of the row blocks + ordered compaction into O
//   k_prep             rebuilds the outlier set, masked row absmax, int8
//                      codes, X[:,O] gather, dequantized weight rows
//                      CB[:,O]*SCB/127
//
// The method: Hugging Face LLM.int8() summary (agentlenshq.com), section
// "LLM.int8() の核心アイデア" steps 1-2; absmax rule from its section
// "量子化の仕組み"; CB/SCB storage from "transformers への統合".
#include "common.h"
#include "kernels.h"

namespace i8mm {

// ---------------------------------------------------------------------------
// Weight quantization: one workgroup per output channel j (row of W[N,K]).
// Pass 1 takes the row absmax (exact: the max of fp16 magnitudes), pass 2
// re-reads the row (an L2 hit) and writes the codes.
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(256) void k_wquant(const _Float16* __restrict__ W, int64_t K,
                                                int8_t* __restrict__ CB, float* __restrict__ SCB) {
  __shared__ float red[4];
  const int64_t j = blockIdx.x;
  const _Float16* row = W + j * K;
  int8_t* out = CB + j * K;
  float m = 0.0f;
  if (VEC) {
    const int64_t nc = K / 8;
    for (int64_t c = threadIdx.x; c < nc; c += 256) {
      v8h v = *(const v8h*)(row + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(h2f(v[e])));
    }
  } else {
    for (int64_t k = threadIdx.x; k < K; k += 256) m = fmaxf(m, fabsf(h2f(row[k])));
  }
  const float s = block_max<256>(m, red);
  const float r = 1.0f / s;
  if (threadIdx.x == 0) SCB[j] = s;
  if (VEC) {
    const int64_t nc = K / 8;
    for (int64_t c = threadIdx.x; c < nc; c += 256) {
      v8h v = *(const v8h*)(row + c * 8);
      v2u packed = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t q = (uint8_t)absmax_code(h2f(v[e]), s, r);
        packed[e / 4] |= q << (8 * (e % 4));
      }
      *(v2u*)(out + c * 8) = packed;
    }
  } else {
    for (int64_t k = threadIdx.x; k < K; k += 256) out[k] = absmax_code(h2f(row[k]), s, r);
  }
}

void launch_wquant(const _Float16* W, int64_t N, int64_t K, int8_t* CB, float* SCB, bool vec,
                   hipStream_t st) {
  if (vec)
    k_wquant<true><<<dim3((unsigned)N), dim3(256), 0, st>>>(W, K, CB, SCB);
  else
    k_wquant<false><<<dim3((unsigned)N), dim3(256), 0, st>>>(W, K, CB, SCB);
}

// ---------------------------------------------------------------------------
// Outlier detection, phase 1.  Grid (column slabs of 512, row blocks).  A
// lane owns 8 consecutive columns (one 16-byte load per row); the 4 waves of
// a workgroup split the rows of the row block.  Each workgroup writes the
// 512 flag bits of its slab for its row block with plain stores, so nothing
// needs to be zeroed beforehand.
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(256) void k_detect_partial(const _Float16* __restrict__ X, int64_t T,
                                                        int64_t K, int64_t rows_per_block, float thr,
                                                        uint32_t* __restrict__ partial, int64_t KW) {
  __shared__ uint32_t fl[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * 512 + lane * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(T, r0 + rows_per_block);
  uint32_t f = 0;
  if (VEC) {
    if (c0 < K) {
      const _Float16* p = X + c0;
#pragma unroll 16
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
    uint32_t g = fl[0][lane] | fl[1][lane] | fl[2][lane] | fl[3][lane];
    uint32_t word = g << (8 * (lane & 3));
    word |= __shfl_xor(word, 1, 64);
    word |= __shfl_xor(word, 2, 64);
    const int64_t wi = ((int64_t)blockIdx.x * 512 + lane * 8) / 32;
    if ((lane & 3) == 0 && wi < KW) partial[(int64_t)blockIdx.y * KW + wi] = word;
  }
}

// ---------------------------------------------------------------------------
// Outlier detection, phase 2: one workgroup of 1024 threads (16 waves).
// (a) mask word w = OR over the row blocks of partial[rb][w]: a wave takes 64
//     consecutive words (one per lane, coalesced) and every 16th row block;
//     the 16 waves' results meet in LDS.
// (b) an exclusive scan of the per-word popcounts, in ascending word order,
//     gives every set bit its rank, so O comes out ascending and unique.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_detect_compact(const uint32_t* __restrict__ partial,
                                                         int64_t nrb, int64_t KW,
                                                         uint32_t* __restrict__ mask,
                                                         int32_t* __restrict__ O,
                                                         int32_t* __restrict__ counts,
                                                         int64_t max_o) {
  extern __shared__ uint32_t smask[];  // KW words
  __shared__ uint32_t ors[16][64];
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int64_t g = 0; g < KW; g += 64) {
    const int64_t w = g + lane;
    uint32_t m = 0;
    if (w < KW) {
#pragma unroll 4
      for (int64_t r = wv; r < nrb; r += 16) m |= partial[r * KW + w];
    }
    ors[wv][lane] = m;
    __syncthreads();
    if (wv == 0 && w < KW) {
      uint32_t t = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) t |= ors[i][lane];
      mask[w] = t;
      smask[w] = t;
    }
    __syncthreads();
  }
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int64_t base = 0; base < KW; base += 1024) {
    const int64_t w = base + tid;
    uint32_t m = (w < KW) ? smask[w] : 0u;
    const int c = __popc(m);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int s = wsum[i];
      before += (i < wv) ? s : 0;
      total += s;
    }
    int pos = carry_s + before + incl - c;
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      if (pos < max_o) O[pos] = (int32_t)(w * 32 + b);
      ++pos;
    }
    __syncthreads();
    if (tid == 0) carry_s += total;
    __syncthreads();
  }
  if (tid == 0) {
    counts[0] = carry_s;
    counts[1] = (int64_t)carry_s > max_o ? 1 : 0;
    counts[2] = 0;
    counts[3] = 0;
  }
}

void launch_detect_partial(const _Float16* X, int64_t T, int64_t K, float thr, uint32_t* partial,
                           int64_t rows_per_block, int64_t nrb, bool vec, hipStream_t st) {
  const int64_t KW = ceil_div(K, 32);
  dim3 g((unsigned)ceil_div(K, 512), (unsigned)nrb);
  if (vec)
    k_detect_partial<true><<<g, dim3(256), 0, st>>>(X, T, K, rows_per_block, thr, partial, KW);
  else
    k_detect_partial<false><<<g, dim3(256), 0, st>>>(X, T, K, rows_per_block, thr, partial, KW);
}

void launch_detect_compact(const uint32_t* partial, int64_t nrb, int64_t K, uint32_t* mask,
                           int32_t* O, int32_t* counts, int64_t max_o, hipStream_t st) {
  const int64_t KW = ceil_div(K, 32);
  k_detect_compact<<<dim3(1), dim3(1024), (size_t)KW * 4, st>>>(partial, nrb, KW, mask, O,
                                                                 counts, max_o);
}

// ---------------------------------------------------------------------------
// Step 2 preparation, one launch.  Every workgroup first rebuilds the outlier
// set from the detection pass's per-row-block flags: mask word w = OR over
// the row blocks, and pref[w] = number of outlier columns in words < w (an
// exclusive scan of popcounts in ascending word order), so the o-th outlier
// column is the q-th set bit of the word with pref[w] <= o < pref[w+1].
// Enumerating words in order therefore yields (o, column) pairs ascending
// and without duplicates -- no sorted list is needed.
//   workgroup 0 also publishes mask, O and counts (n_o, overflow);
//   workgroups [0, nrowblk): 4 rows of X each, one row per wave: masked
//     absmax -> sx, codes -> Xq (0 on outlier and pad columns), X[:, O] ->
//     Xo (0 on pad columns);
//   workgroups [nrowblk, nrowblk + nwoblk): 16 output channels each:
//     Wo[j, o] = fp16(fl32(fl32(CB[j, O[o]] * SCB[j]) / 127)), 0 on pad
//     columns (skipped when the outlier set has at most small_tail columns).
// LDS: mask[KW], pref[KW + 1], then (channel workgroups) the O list of up to
// ocap entries and, when allowed (16-byte aligned CB rows, K <= 16384), one
// staged CB row per wave.
// ---------------------------------------------------------------------------
constexpr int kRowsPerPrepBlock = 4;
constexpr int kChansPerWoBlock = 16;
constexpr int kMaxCachedChunks = 24;  // 16-byte chunks of a row a lane keeps in registers

template <bool VEC>
__global__ __launch_bounds__(256) void k_prep(
    const _Float16* __restrict__ X, int64_t T, int64_t K, const uint32_t* __restrict__ partial,
    int64_t nrb, uint32_t* __restrict__ mask_out, int32_t* __restrict__ O_out,
    int32_t* __restrict__ counts, int64_t max_o, int8_t* __restrict__ Xq, int64_t ldq,
    float* __restrict__ sx, _Float16* __restrict__ Xo, int64_t ldo, int64_t nrowblk,
    const int8_t* __restrict__ CB, const float* __restrict__ SCB, int64_t N,
    _Float16* __restrict__ Wo, int64_t small_tail, int64_t ocap, int stage_rows) {
  extern __shared__ __attribute__((aligned(16))) uint32_t sm[];
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t KW = ceil_div(K, 32);
  uint32_t* smask = sm;
  int32_t* spref = (int32_t*)(sm + KW);

  // ---- the outlier set: mask words and exclusive prefix of their popcounts
  // (1) OR the row blocks' words into LDS: coalesced, independent loads,
  //     8 in flight per thread
  for (int64_t w = tid; w < KW; w += 256) smask[w] = 0u;
  __syncthreads();
  const int64_t tot = nrb * KW;
  for (int64_t b0 = 0; b0 < tot; b0 += 256 * 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t idx = b0 + u * 256 + tid;
      v[u] = idx < tot ? partial[idx] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t idx = b0 + u * 256 + tid;
      if (v[u]) atomicOr(&smask[idx % KW], v[u]);
    }
  }
  __syncthreads();
  // (2) block-wide exclusive scan of the popcounts; each thread owns a
  //     contiguous run of words
  const int64_t per = ceil_div(KW, 256);
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
  int base = 0;
  for (int i = 0; i < wave; ++i) base += wsum[i];
  const int n_o = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  int acc = base + incl - run;
  for (int64_t w = w0; w < w1; ++w) {
    spref[w] = acc;
    acc += __popc(smask[w]);
  }
  if (tid == 0) spref[KW] = n_o;
  __syncthreads();
  const int64_t n_use = (int64_t)n_o < max_o ? n_o : max_o;
  const int64_t n_pad = round_up(n_use, 32);

  if (blockIdx.x == 0 && counts) {
    for (int64_t w = tid; w < KW; w += 256) {
      uint32_t m = smask[w];
      if (mask_out) mask_out[w] = m;
      int64_t o = spref[w];
      while (m) {
        const int b = __ffs(m) - 1;
        m &= m - 1;
        if (o < max_o) O_out[o] = (int32_t)(w * 32 + b);
        ++o;
      }
    }
    if (tid == 0) {
      counts[0] = n_o;
      counts[1] = (int64_t)n_o > max_o ? 1 : 0;
      counts[2] = 0;
      counts[3] = 0;
    }
  }

  if ((int64_t)blockIdx.x < nrowblk) {
    // ---- rows: one per wave, no barrier below this point
    const int64_t i = (int64_t)blockIdx.x * kRowsPerPrepBlock + wave;
    if (i >= T) return;
    const _Float16* row = X + i * K;
    int8_t* qrow = Xq + i * ldq;
    float m = 0.0f;
    if (VEC) {
      const int64_t nc = K / 8;
      // chunks lane + 64u stay in registers between the two passes; chunks
      // beyond kMaxCachedChunks per lane are read again (an L2 hit)
      v8h cache[kMaxCachedChunks];
#pragma unroll
      for (int u = 0; u < kMaxCachedChunks; ++u) {
        const int64_t c = lane + 64 * u;
        if (c < nc) cache[u] = *(const v8h*)(row + c * 8);
      }
      auto absmax_chunk = [&](int64_t c, v8h v) {
        const uint32_t bits = smask[c >> 2] >> (8 * (c & 3));
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!((bits >> e) & 1u)) m = fmaxf(m, fabsf(h2f(v[e])));
      };
#pragma unroll
      for (int u = 0; u < kMaxCachedChunks; ++u) {
        const int64_t c = lane + 64 * u;
        if (c < nc) absmax_chunk(c, cache[u]);
      }
      for (int64_t c = lane + 64 * kMaxCachedChunks; c < nc; c += 64)
        absmax_chunk(c, *(const v8h*)(row + c * 8));
      const float s = wave_max(m);
      const float rs = 1.0f / s;
      if (lane == 0) sx[i] = s;
      auto quant_chunk = [&](int64_t c, v8h v) {
        const uint32_t bits = smask[c >> 2] >> (8 * (c & 3));
        v2u packed = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t q =
              ((bits >> e) & 1u) ? 0u : (uint32_t)(uint8_t)absmax_code(h2f(v[e]), s, rs);
          packed[e / 4] |= q << (8 * (e % 4));
        }
        *(v2u*)(qrow + c * 8) = packed;
      };
#pragma unroll
      for (int u = 0; u < kMaxCachedChunks; ++u) {
        const int64_t c = lane + 64 * u;
        if (c < nc) quant_chunk(c, cache[u]);
      }
      for (int64_t c = lane + 64 * kMaxCachedChunks; c < nc; c += 64)
        quant_chunk(c, *(const v8h*)(row + c * 8));
      for (int64_t k = K + lane; k < ldq; k += 64) qrow[k] = 0;
    } else {
      for (int64_t k = lane; k < K; k += 64)
        if (!((smask[k >> 5] >> (k & 31)) & 1u)) m = fmaxf(m, fabsf(h2f(row[k])));
      const float s = wave_max(m);
      const float rs = 1.0f / s;
      if (lane == 0) sx[i] = s;
      for (int64_t k = lane; k < ldq; k += 64) {
        int8_t q = 0;
        if (k < K && !((smask[k >> 5] >> (k & 31)) & 1u)) q = absmax_code(h2f(row[k]), s, rs);
        qrow[k] = q;
      }
    }
    // X[i, O] -> Xo[i, :]
    _Float16* xorow = Xo + i * ldo;
    for (int64_t w = lane; w < KW; w += 64) {
      uint32_t mb = smask[w];
      int64_t o = spref[w];
      while (mb) {
        const int b = __ffs(mb) - 1;
        mb &= mb - 1;
        if (o < n_use) xorow[o] = row[w * 32 + b];
        ++o;
      }
    }
    for (int64_t o = n_use + lane; o < n_pad; o += 64) xorow[o] = (_Float16)0.0f;
    return;
  }

  // ---- dequantized outlier weight rows
  if (n_use <= small_tail) return;  // the product kernel builds its own
  const int64_t j0 = ((int64_t)blockIdx.x - nrowblk) * kChansPerWoBlock;
  if (n_use <= ocap) {
    // the O list in LDS, then per channel a gather from the CB row (staged
    // in LDS when wide, so the reads of CB stay coalesced)
    int32_t* sO = (int32_t*)(spref + KW + 1);
    for (int64_t w = tid; w < KW; w += 256) {
      uint32_t mb = smask[w];
      int64_t o = spref[w];
      while (mb) {
        const int b = __ffs(mb) - 1;
        mb &= mb - 1;
        if (o < n_use) sO[o] = (int32_t)(w * 32 + b);
        ++o;
      }
    }
    __syncthreads();
    // a wide outlier set reads each CB row once, coalesced, into LDS
    const bool stage = stage_rows && n_use > 64;
    int8_t* srow = (int8_t*)sm + round_up((2 * KW + 1 + ocap) * 4, 16) + wave * K;
    for (int r = 0; r < kChansPerWoBlock / 4; ++r) {
      const int64_t j = j0 + wave * (kChansPerWoBlock / 4) + r;
      if (j >= N) break;  // uniform across the wave
      const int8_t* cbrow = CB + j * K;
      const float sj = SCB[j];
      if (stage) {  // K % 16 == 0, 16-byte aligned rows, K <= 16384: <= 16 chunks a lane
        v4i t[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int64_t c = lane + 64 * u;
          if (c < K / 16) t[u] = *(const v4i*)(cbrow + c * 16);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int64_t c = lane + 64 * u;
          if (c < K / 16) *(v4i*)(srow + c * 16) = t[u];
        }
      }
      _Float16* worow = Wo + j * ldo;
      for (int64_t o = lane; o < n_pad; o += 64) {
        _Float16 v = (_Float16)0.0f;
        if (o < n_use) {
          const int8_t c = stage ? srow[sO[o]] : cbrow[sO[o]];
          v = dequant_weight(c, sj);
        }
        worow[o] = v;
      }
    }
  } else {
    // very large outlier sets: enumerate (o, column) word by word per channel
    for (int r = 0; r < kChansPerWoBlock / 4; ++r) {
      const int64_t j = j0 + wave * (kChansPerWoBlock / 4) + r;
      if (j >= N) break;
      const int8_t* cbrow = CB + j * K;
      const float sj = SCB[j];
      _Float16* worow = Wo + j * ldo;
      for (int64_t w = lane; w < KW; w += 64) {
        uint32_t mb = smask[w];
        int64_t o = spref[w];
        while (mb) {
          const int b = __ffs(mb) - 1;
          mb &= mb - 1;
          if (o < n_use) worow[o] = dequant_weight(cbrow[w * 32 + b], sj);
          ++o;
        }
      }
      for (int64_t o = n_use + lane; o < n_pad; o += 64) worow[o] = (_Float16)0.0f;
    }
  }
}

size_t prep_lds_bytes(int64_t K, int64_t ocap, bool stage_rows) {
  const int64_t KW = ceil_div(K, 32);
  return (size_t)(round_up((2 * KW + 1 + ocap) * 4, 16) + (stage_rows ? 4 * K : 0));
}

void launch_prep(const PrepArgs& p, hipStream_t st) {
  const int64_t nrowblk = p.Xq ? ceil_div(p.T, kRowsPerPrepBlock) : 0;
  const int64_t nwoblk = p.Wo ? ceil_div(p.N, kChansPerWoBlock) : 0;
  const int64_t ocap = p.Wo ? p.ocap : 0;
  const bool stage_rows = p.Wo && p.stage_rows;
  const size_t lds = prep_lds_bytes(p.K, ocap, stage_rows);
  dim3 g((unsigned)(nrowblk + nwoblk > 0 ? nrowblk + nwoblk : 1));
  auto go = [&](auto kern) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
    kern<<<g, dim3(256), lds, st>>>(p.X, p.T, p.K, p.partial, p.nrb, p.mask_out, p.O_out,
                                    p.counts, p.max_o, p.Xq, p.ldq, p.sx, p.Xo, p.ldo, nrowblk,
                                    p.CB, p.SCB, p.N, p.Wo, p.small_tail, ocap,
                                    stage_rows ? 1 : 0);
  };
  if (p.vec)
    go(k_prep<true>);
  else
    go(k_prep<false>);
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

}  // namespace i8mm
