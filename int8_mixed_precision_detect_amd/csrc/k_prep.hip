// Bandwidth-bound kernels of the LLM.int8() layer on gfx950:
//   k_wquant           weight -> CB/SCB (absmax per output channel)
//   k_detect_partial   per-row-block column flags |x| >= threshold
//   k_detect_compact   OR of the row blocks + ordered compaction into O
//   k_rowquant         masked row absmax, int8 codes, X[:,O] gather, and the
//                      dequantized outlier weight rows CB[:,O]*SCB/127
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
  if (threadIdx.x == 0) SCB[j] = s;
  if (VEC) {
    const int64_t nc = K / 8;
    for (int64_t c = threadIdx.x; c < nc; c += 256) {
      v8h v = *(const v8h*)(row + c * 8);
      v2u packed = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t q = (uint8_t)absmax_code(h2f(v[e]), s);
        packed[e / 4] |= q << (8 * (e % 4));
      }
      *(v2u*)(out + c * 8) = packed;
    }
  } else {
    for (int64_t k = threadIdx.x; k < K; k += 256) out[k] = absmax_code(h2f(row[k]), s);
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
#pragma unroll 8
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

void launch_detect(const _Float16* X, int64_t T, int64_t K, float thr, uint32_t* partial,
                   int64_t rows_per_block, int64_t nrb, uint32_t* mask, int32_t* O,
                   int32_t* counts, int64_t max_o, bool vec, hipStream_t st) {
  const int64_t KW = ceil_div(K, 32);
  dim3 g((unsigned)ceil_div(K, 512), (unsigned)nrb);
  if (vec)
    k_detect_partial<true><<<g, dim3(256), 0, st>>>(X, T, K, rows_per_block, thr, partial, KW);
  else
    k_detect_partial<false><<<g, dim3(256), 0, st>>>(X, T, K, rows_per_block, thr, partial, KW);
  k_detect_compact<<<dim3(1), dim3(1024), (size_t)KW * 4, st>>>(partial, nrb, KW, mask, O,
                                                                 counts, max_o);
}

// ---------------------------------------------------------------------------
// Step 2 preparation.  Workgroups [0, nrow) quantize one row of X each:
// masked absmax -> sx[i], codes -> Xq[i, :] (0 on outlier and pad columns),
// X[i, O] -> Xo[i, :] (0 on pad columns).  Workgroups [nrow, nrow + ceil(N/8))
// build 8 rows each of Wo = fp16(fl32(fl32(CB[j, O] * SCB[j]) / 127)).
// The outlier bit mask lives in LDS (copied from `mask`, or rebuilt from O).
// ---------------------------------------------------------------------------
template <bool VEC>
__global__ __launch_bounds__(256) void k_rowquant(
    const _Float16* __restrict__ X, int64_t T, int64_t K, const int32_t* __restrict__ O,
    const int32_t* __restrict__ counts, const uint32_t* __restrict__ mask, int64_t max_o,
    int8_t* __restrict__ Xq, int64_t ldq, float* __restrict__ sx, _Float16* __restrict__ Xo,
    int64_t ldo, int64_t nrow, const int8_t* __restrict__ CB, const float* __restrict__ SCB,
    int64_t N, _Float16* __restrict__ Wo) {
  extern __shared__ uint32_t smask[];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int64_t n_o = counts[0];
  const int64_t n_use = n_o < max_o ? n_o : max_o;
  const int64_t n_pad = round_up(n_use, 32);

  if ((int64_t)blockIdx.x >= nrow) {
    // dequantized outlier weight rows
    const int64_t j = ((int64_t)blockIdx.x - nrow) * 8 + (tid >> 5);
    if (j >= N) return;
    const float s = SCB[j];
    const int8_t* cbrow = CB + j * K;
    for (int64_t o = tid & 31; o < n_pad; o += 32) {
      _Float16 v = (_Float16)0.0f;
      if (o < n_use) {
        const float p = (float)cbrow[O[o]] * s;  // exact: <= 8 x 11 significant bits
        v = (_Float16)(p / 127.0f);               // fp32 division, then RNE to fp16
      }
      Wo[j * ldo + o] = v;
    }
    return;
  }

  const int64_t KW = ceil_div(K, 32);
  if (mask) {
    for (int64_t w = tid; w < KW; w += 256) smask[w] = mask[w];
  } else {
    for (int64_t w = tid; w < KW; w += 256) smask[w] = 0u;
    __syncthreads();
    for (int64_t o = tid; o < n_use; o += 256) {
      const int32_t k = O[o];
      atomicOr(&smask[k >> 5], 1u << (k & 31));
    }
  }
  __syncthreads();

  const int64_t i = blockIdx.x;
  const _Float16* row = X + i * K;
  int8_t* qrow = Xq + i * ldq;
  float m = 0.0f;
  if (VEC) {
    for (int64_t c = tid; c < K / 8; c += 256) {
      v8h v = *(const v8h*)(row + c * 8);
      const uint32_t bits = smask[c >> 2] >> (8 * (c & 3));
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!((bits >> e) & 1u)) m = fmaxf(m, fabsf(h2f(v[e])));
    }
  } else {
    for (int64_t k = tid; k < K; k += 256)
      if (!((smask[k >> 5] >> (k & 31)) & 1u)) m = fmaxf(m, fabsf(h2f(row[k])));
  }
  const float s = block_max<256>(m, red);
  if (tid == 0) sx[i] = s;
  if (VEC) {
    for (int64_t c = tid; c < K / 8; c += 256) {
      v8h v = *(const v8h*)(row + c * 8);
      const uint32_t bits = smask[c >> 2] >> (8 * (c & 3));
      v2u packed = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t q = ((bits >> e) & 1u) ? 0u : (uint32_t)(uint8_t)absmax_code(h2f(v[e]), s);
        packed[e / 4] |= q << (8 * (e % 4));
      }
      *(v2u*)(qrow + c * 8) = packed;
    }
    for (int64_t k = K + tid; k < ldq; k += 256) qrow[k] = 0;
  } else {
    for (int64_t k = tid; k < ldq; k += 256) {
      int8_t q = 0;
      if (k < K && !((smask[k >> 5] >> (k & 31)) & 1u)) q = absmax_code(h2f(row[k]), s);
      qrow[k] = q;
    }
  }
  for (int64_t o = tid; o < n_pad; o += 256)
    Xo[i * ldo + o] = (o < n_use) ? row[O[o]] : (_Float16)0.0f;
}

void launch_rowquant(const _Float16* X, int64_t T, int64_t K, const int32_t* O,
                     const int32_t* counts, const uint32_t* mask, int64_t max_o, int8_t* Xq,
                     int64_t ldq, float* sx, _Float16* Xo, int64_t ldo, const int8_t* CB,
                     const float* SCB, int64_t N, _Float16* Wo, bool vec, hipStream_t st) {
  const int64_t nrow = (Xq != nullptr) ? T : 0;
  const int64_t nwo = (Wo != nullptr) ? ceil_div(N, 8) : 0;
  const size_t lds = (size_t)ceil_div(K, 32) * 4;
  dim3 g((unsigned)(nrow + nwo));
  if (vec)
    k_rowquant<true><<<g, dim3(256), lds, st>>>(X, T, K, O, counts, mask, max_o, Xq, ldq, sx, Xo,
                                                ldo, nrow, CB, SCB, N, Wo);
  else
    k_rowquant<false><<<g, dim3(256), lds, st>>>(X, T, K, O, counts, mask, max_o, Xq, ldq, sx, Xo,
                                                 ldo, nrow, CB, SCB, N, Wo);
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
