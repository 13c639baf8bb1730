// Host side of the libi8mm C ABI: argument checks, workspace carving and
// kernel sequencing on the caller's stream.  See include/i8mm.h for the
// contract of every entry point.
#include <math.h>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/i8mm.h"
#include "common.h"
#include "kernels.h"

using namespace i8mm;

namespace {

constexpr int64_t kAlign = 256;
constexpr size_t kMaskRegion = (size_t)(kMaxK / 32) * 4;  // bytes: the mask of the largest K
constexpr int64_t kMaxDim = (int64_t)1 << 31;  // sizes must fit int32 indexing of O

inline bool aligned(const void* p, uintptr_t a) { return (((uintptr_t)p) & (a - 1)) == 0; }

// O-list capacity (entries) the step-2 workgroups keep in LDS; larger
// outlier sets are enumerated from the mask instead.
constexpr int64_t kOcap = kMaxOcap;

i8mm_status layout_of(int64_t T, int64_t N, int64_t K, int64_t max_o, i8mm_ws_layout* L) {
  if (T < 0 || N < 0 || K < 0 || max_o < 0 || max_o > K) return I8MM_ERR_INVALID_ARG;
  if (T >= kMaxDim || N >= kMaxDim || K > kMaxK) return I8MM_ERR_UNSUPPORTED;
  const int64_t KW = ceil_div(K, 32);
  L->ldq = round_up(K, 64);
  L->ldo = round_up(max_o, 32);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (size_t)round_up((int64_t)(off + bytes), kAlign);
    return o;
  };
  L->counts = take(16);
  // the mask sits at the same place, with room for the largest K, whatever
  // the shape: forwards leave its words zero, so one initialized workspace
  // serves calls of any shape in turn
  L->mask = take(kMaskRegion);
  L->outliers = take((size_t)(max_o > 0 ? max_o : 1) * 4);
  (void)KW;
  L->sx = take((size_t)T * 4);
  L->xq = take((size_t)T * (size_t)L->ldq);
  L->xo = take((size_t)T * (size_t)L->ldo * 2);
  L->wo = take((size_t)N * (size_t)L->ldo * 2);
  L->zp = take((size_t)(T > 0 ? T : 1) * 4);
  L->osum = take((size_t)(N > 0 ? N : 1) * 4);
  // partial tiles of the product's plan (both layer variants share it)
  const GemmPlan gp = plan_gemm_i8(T, N, K);
  L->part = take((size_t)gp.part_elems * 4);
  L->splits = gp.splits;
  L->total = off;
  return I8MM_OK;
}

i8mm_status hip_status() {
  return hipGetLastError() == hipSuccess ? I8MM_OK : I8MM_ERR_HIP;
}

// ---- instrumentation state ----
constexpr int kProfCap = 4096;
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
int g_prof_n = 0;
std::vector<hipEvent_t> g_prof_ev;  // kProfCap * 4 events, created on first enable

// forwards of one to eight tokens with steps 1-2 in one launch of one workgroup (see
// i8mm_set_row_prep); a test and tuning control
std::atomic<bool> g_row_prep{true};

}  // namespace

extern "C" {

const char* i8mm_status_string(i8mm_status s) {
  switch (s) {
    case I8MM_OK: return "I8MM_OK";
    case I8MM_ERR_INVALID_ARG: return "I8MM_ERR_INVALID_ARG";
    case I8MM_ERR_WORKSPACE: return "I8MM_ERR_WORKSPACE";
    case I8MM_ERR_UNSUPPORTED: return "I8MM_ERR_UNSUPPORTED";
    case I8MM_ERR_HIP: return "I8MM_ERR_HIP";
    case I8MM_ERR_OUTLIER_OVERFLOW: return "I8MM_ERR_OUTLIER_OVERFLOW";
  }
  return "I8MM_UNKNOWN_STATUS";
}

int i8mm_abi_version(void) { return I8MM_ABI_VERSION; }

i8mm_status i8mm_set_split_override(int64_t splits) {
  if (splits < 0) return I8MM_ERR_INVALID_ARG;
  set_split_override(splits);
  return I8MM_OK;
}

i8mm_status i8mm_set_row_prep(int enable) {
  if (enable != 0 && enable != 1) return I8MM_ERR_INVALID_ARG;
  g_row_prep.store(enable == 1);
  return I8MM_OK;
}

i8mm_status i8mm_set_tile_override(int64_t cfg) {
  if (cfg < -1 || cfg > 3) return I8MM_ERR_INVALID_ARG;
  set_tile_override(cfg);
  return I8MM_OK;
}

i8mm_status int8_quantize_weight(const void* W, int64_t N, int64_t K, int8_t* CB, float* SCB,
                                 hipStream_t stream) {
  if (N < 0 || K < 0) return I8MM_ERR_INVALID_ARG;
  if (N >= kMaxDim || K >= kMaxDim) return I8MM_ERR_UNSUPPORTED;
  if (N == 0) return I8MM_OK;
  if (!SCB || !aligned(SCB, 4)) return I8MM_ERR_INVALID_ARG;
  if (K > 0 && (!W || !CB || !aligned(W, 2))) return I8MM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const bool vec = (K % 8 == 0) && aligned(W, 16) && aligned(CB, 8);
  launch_wquant((const _Float16*)W, N, K, CB, SCB, vec, stream);
  return hip_status();
}

i8mm_status int8_linear_workspace_layout(int64_t T, int64_t N, int64_t K, int64_t max_outliers,
                                         i8mm_ws_layout* out) {
  if (!out) return I8MM_ERR_INVALID_ARG;
  return layout_of(T, N, K, max_outliers, out);
}

i8mm_status int8_linear_workspace_init(void* ws, int64_t T, int64_t N, int64_t K,
                                       int64_t max_outliers, hipStream_t stream) {
  i8mm_ws_layout L;
  const i8mm_status ls = layout_of(T, N, K, max_outliers, &L);
  if (ls != I8MM_OK) return ls;
  if (!ws || !aligned(ws, kAlign)) return I8MM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  // counts and the whole mask region: the head of the workspace
  launch_zero_words((uint32_t*)ws, (int64_t)((L.mask + kMaskRegion) / 4), stream);
  return hip_status();
}

size_t int8_linear_workspace_size(int64_t T, int64_t N, int64_t K, int64_t max_outliers) {
  i8mm_ws_layout L;
  if (layout_of(T, N, K, max_outliers, &L) != I8MM_OK) return 0;
  return L.total;
}

namespace {
// The forward.  W16 != null: the fp16-weight variant -- W16 is quantized
// into CB/SCB first (they are outputs then) and Wo is copied from W16.
// rsum != null: the zero-point layer (rsum = CB's row sums).
i8mm_status forward_impl(const void* X, int64_t T, int64_t K, const int8_t* CB, const float* SCB,
                         int64_t N, const void* bias, float threshold, void* Y, void* ws,
                         size_t ws_bytes, int64_t max_outliers, hipStream_t stream,
                         const _Float16* W16, const int32_t* rsum = nullptr,
                         int32_t* counts_ext = nullptr, bool zero_mask = false) {
  if (isnan(threshold) || !(threshold > 0.0f)) return I8MM_ERR_INVALID_ARG;
  i8mm_ws_layout L;
  const i8mm_status ls = layout_of(T, N, K, max_outliers, &L);
  if (ls != I8MM_OK) return ls;
  if (T == 0 || N == 0) return I8MM_OK;
  if (!Y || !ws || !aligned(Y, 2) || !aligned(ws, kAlign)) return I8MM_ERR_INVALID_ARG;
  if (bias && !aligned(bias, 2)) return I8MM_ERR_INVALID_ARG;
  if (K > 0 && (!X || !CB || !SCB || !aligned(X, 2) || !aligned(SCB, 4)))
    return I8MM_ERR_INVALID_ARG;
  if (W16 && K > 0 && !aligned(W16, 2)) return I8MM_ERR_INVALID_ARG;
  if (ws_bytes < L.total) return I8MM_ERR_WORKSPACE;
  (void)hipGetLastError();

  char* w = (char*)ws;
  int32_t* counts = counts_ext ? counts_ext : (int32_t*)(w + L.counts);
  hipEvent_t* ev = nullptr;
  if (K > 0 && g_prof_on.load(std::memory_order_relaxed)) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_on && g_prof_n < kProfCap) ev = &g_prof_ev[(size_t)(g_prof_n++) * 4];
  }
  if (ev) (void)hipEventRecord(ev[0], stream);
  if (W16) {
    // (in the profile, the per-call weight quantization counts as detection)
    const bool wvec = (K % 8 == 0) && aligned(W16, 16) && aligned(CB, 8);
    launch_wquant(W16, N, K, (int8_t*)CB, (float*)SCB, wvec, stream);
  }
  if (K == 0) {
    launch_fill_bias((_Float16*)Y, T, N, (const _Float16*)bias, counts, stream);
    return hip_status();
  }

  int32_t* O = (int32_t*)(w + L.outliers);
  uint32_t* mask = (uint32_t*)(w + L.mask);
  const bool xvec = (K % 8 == 0) && aligned(X, 16);

  int8_t* Xq = (int8_t*)(w + L.xq);
  float* sx = (float*)(w + L.sx);
  _Float16* Xo = (_Float16*)(w + L.xo);
  _Float16* Wo = (_Float16*)(w + L.wo);
  PrepArgs pa{};
  pa.X = (const _Float16*)X;
  pa.T = T;
  pa.K = K;
  pa.mask = mask;
  pa.O_out = O;
  pa.counts = counts;
  pa.max_o = max_outliers;
  pa.Xq = Xq;
  pa.ldq = L.ldq;
  pa.sx = sx;
  pa.Xo = Xo;
  pa.ldo = L.ldo;
  pa.CB = CB;
  pa.SCB = SCB;
  pa.N = N;
  pa.Wo = Wo;
  pa.ocap = max_outliers < kOcap ? max_outliers : kOcap;
  pa.vec = xvec;
  pa.W16 = W16;
  int32_t* zp = (int32_t*)(w + L.zp);
  int32_t* osum = (int32_t*)(w + L.osum);
  if (rsum) {
    pa.zp = zp;
    pa.osum = osum;
  }

  GemmArgs a{};
  a.A = CB;
  a.lda = K;
  a.B = Xq;
  a.ldb = L.ldq;
  a.N = N;
  a.T = T;
  a.K = K;
  a.sx = sx;
  a.SCB = SCB;
  a.Wo = Wo;
  a.Xo = Xo;
  a.ldo = L.ldo;
  a.counts = counts;
  a.O = O;
  a.max_o = max_outliers;
  a.bias = (const _Float16*)bias;
  a.Y = (_Float16*)Y;
  const GemmPlan gp = plan_gemm_i8(T, N, K);
  a.cfg = gp.cfg;
  a.splits = gp.splits;
  a.part = gp.part_elems > 0 ? (int32_t*)(w + L.part) : nullptr;
  if (rsum) {
    a.zp = zp;
    a.rsum = rsum;
    a.osum = osum;
  }
  // aligned operands: the tiled kernel (for few tokens it extracts small
  // outlier weight sets itself); otherwise the generic one
  const bool fast = gemm_i8_supported(a);
  // Wo (and, zero-point, the outlier code sums) built by step 2: the
  // few-token tiles then do not rebuild Wo from CB
  a.wo_ready = W16 != nullptr || rsum != nullptr;
  // One to eight tokens, absmax layer: steps 1-2 are done by one workgroup
  // holding the rows, in one launch (k_rows: no mask, no detection launch),
  // and the product takes the outlier weights of any set out of CB itself.
  // (In the stage profile, the detection stage covers both steps.)
  if (T <= kRowsMaxT && xvec && K <= kRow1MaxK && fast && !a.wo_ready &&
      g_row_prep.load(std::memory_order_relaxed)) {
    launch_rows((const _Float16*)X, T, K, threshold, O, counts, max_outliers, Xq, L.ldq, sx, Xo,
                L.ldo, stream);
    if (ev) (void)hipEventRecord(ev[1], stream);
    if (ev) (void)hipEventRecord(ev[2], stream);
    a.wo_gather = true;
    const hipError_t ge = launch_gemm_i8_fused(a, stream);
    if (ge != hipSuccess) return I8MM_ERR_HIP;
    if (ev) (void)hipEventRecord(ev[3], stream);
    return hip_status();
  }
  // (the mask is zero: the last forward on this workspace, or its
  // initialization, left it so.  The allocation-free forward's array has no
  // initialization call, and a call that stopped between detection and the
  // product would leave bits set: it clears the mask every call, a fill
  // kernel.)
  if (zero_mask) launch_zero_words(mask, ceil_div(K, 32), stream);
  launch_detect((const _Float16*)X, T, K, threshold, mask, false, xvec, stream);
  if (ev) (void)hipEventRecord(ev[1], stream);
  a.clear_mask = mask;
  a.clear_words = ceil_div(K, 32);
  pa.wo_skip = fast && T <= kFewT && !a.wo_ready ? kFewOcap : -1;
  launch_prep(pa, stream);
  if (ev) (void)hipEventRecord(ev[2], stream);

  const hipError_t ge = fast ? launch_gemm_i8_fused(a, stream) : launch_gemm_fused(a, stream);
  if (ge != hipSuccess) return I8MM_ERR_HIP;
  if (ev) (void)hipEventRecord(ev[3], stream);
  return hip_status();
}
}  // namespace

i8mm_status int8_linear_forward(const void* X, int64_t T, int64_t K, const int8_t* CB,
                                const float* SCB, int64_t N, const void* bias, float threshold,
                                void* Y, void* ws, size_t ws_bytes, int64_t max_outliers,
                                hipStream_t stream) {
  return forward_impl(X, T, K, CB, SCB, N, bias, threshold, Y, ws, ws_bytes, max_outliers,
                      stream, nullptr);
}

}  // extern "C"

// ---- the allocation-free forward ----
// Its workspace: one array per device, held from the code object's load
// until the process ends.  Host code never uses this name as an address;
// it takes the device address from hipGetSymbolAddress (per device).
static __device__ __align__(256) unsigned char scratch[I8MM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, resolved on the first
// call made with that device current.
i8mm_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return I8MM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return I8MM_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return I8MM_ERR_HIP;
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return I8MM_OK;
}
}  // namespace

extern "C" {

i8mm_status int8_linear_forward_noalloc(const void* X, int64_t T, int64_t K, const int8_t* CB,
                                        const float* SCB, int64_t N, const void* bias,
                                        float threshold, void* Y, int64_t max_outliers,
                                        int32_t* status, hipStream_t stream) {
  i8mm_ws_layout L;
  const i8mm_status ls = layout_of(T, N, K, max_outliers, &L);
  if (ls != I8MM_OK) return ls;
  if (L.total > (size_t)I8MM_NOALLOC_SCRATCH_BYTES) return I8MM_ERR_WORKSPACE;
  if (status && !aligned(status, 4)) return I8MM_ERR_INVALID_ARG;
  if (T == 0 || N == 0) return I8MM_OK;
  void* ws = nullptr;
  const i8mm_status ss = scratch_of_current_device(&ws);
  if (ss != I8MM_OK) return ss;
  return forward_impl(X, T, K, CB, SCB, N, bias, threshold, Y, ws, L.total, max_outliers, stream,
                      nullptr, nullptr, status, true);
}

i8mm_status int8_weight_rowsum(const int8_t* CB, int64_t N, int64_t K, int32_t* rsum,
                               hipStream_t stream) {
  if (N < 0 || K < 0) return I8MM_ERR_INVALID_ARG;
  if (N == 0) return I8MM_OK;
  if (!rsum || !aligned(rsum, 4) || (K > 0 && !CB)) return I8MM_ERR_INVALID_ARG;
  if (N >= kMaxDim || K >= kMaxDim) return I8MM_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  launch_rowsum(CB, N, K, rsum, stream);
  return hip_status();
}

i8mm_status int8_linear_forward_zeropoint(const void* X, int64_t T, int64_t K, const int8_t* CB,
                                          const float* SCB, const int32_t* rsum, int64_t N,
                                          const void* bias, float threshold, void* Y, void* ws,
                                          size_t ws_bytes, int64_t max_outliers,
                                          hipStream_t stream) {
  if (T > 0 && N > 0 && K > 0 && (!rsum || !aligned(rsum, 4))) return I8MM_ERR_INVALID_ARG;
  return forward_impl(X, T, K, CB, SCB, N, bias, threshold, Y, ws, ws_bytes, max_outliers, stream,
                      nullptr, K > 0 ? rsum : nullptr);
}

i8mm_status int8_linear_forward_fp16w(const void* X, int64_t T, int64_t K, const void* W,
                                      int64_t N, const void* bias, float threshold, int8_t* CB,
                                      float* SCB, void* Y, void* ws, size_t ws_bytes,
                                      int64_t max_outliers, hipStream_t stream) {
  if (T > 0 && N > 0 && K > 0 && !W) return I8MM_ERR_INVALID_ARG;
  return forward_impl(X, T, K, CB, SCB, N, bias, threshold, Y, ws, ws_bytes, max_outliers,
                      stream, K > 0 ? (const _Float16*)W : nullptr);
}

i8mm_status int8_linear_status(const void* ws, int32_t* n_outliers, hipStream_t stream) {
  if (!ws || !aligned(ws, kAlign)) return I8MM_ERR_INVALID_ARG;
  int32_t c[4] = {0, 0, 0, 0};
  if (hipMemcpyAsync(c, ws, sizeof(c), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return I8MM_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return I8MM_ERR_HIP;
  if (n_outliers) *n_outliers = c[0];
  return c[1] ? I8MM_ERR_OUTLIER_OVERFLOW : I8MM_OK;
}

i8mm_status int8_find_outliers(const void* X, int64_t T, int64_t K, float threshold, int32_t* O,
                               int32_t* counts, uint32_t* mask, int64_t max_outliers,
                               hipStream_t stream) {
  if (isnan(threshold) || !(threshold > 0.0f)) return I8MM_ERR_INVALID_ARG;
  if (T <= 0 || K <= 0 || max_outliers < 0 || max_outliers > K) return I8MM_ERR_INVALID_ARG;
  if (T >= kMaxDim || K > kMaxK) return I8MM_ERR_UNSUPPORTED;
  if (!X || !O || !counts || !mask || !aligned(X, 2) || !aligned(O, 4) || !aligned(counts, 4) ||
      !aligned(mask, 4))
    return I8MM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const bool xvec = (K % 8 == 0) && aligned(X, 16);
  launch_detect((const _Float16*)X, T, K, threshold, mask, true, xvec, stream);
  launch_compact(mask, K, O, counts, max_outliers, stream);
  return hip_status();
}

i8mm_status int8_quantize_rows(const void* X, int64_t T, int64_t K, const uint32_t* mask,
                               int64_t max_outliers, int8_t* Xq, int64_t ldq, float* sx,
                               void* Xo, int64_t ldo, hipStream_t stream) {
  if (T <= 0 || K <= 0 || max_outliers < 0 || max_outliers > K) return I8MM_ERR_INVALID_ARG;
  if (T >= kMaxDim || K > kMaxK) return I8MM_ERR_UNSUPPORTED;
  if (ldq < K || ldq % 16 != 0 || ldo < round_up(max_outliers, 32) || ldo % 32 != 0)
    return I8MM_ERR_INVALID_ARG;
  if (!X || !mask || !Xq || !sx || !Xo || !aligned(X, 2) || !aligned(Xq, 16) || !aligned(sx, 4) ||
      !aligned(Xo, 2) || !aligned(mask, 4))
    return I8MM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  PrepArgs pa{};
  pa.X = (const _Float16*)X;
  pa.T = T;
  pa.K = K;
  pa.mask = mask;
  pa.max_o = max_outliers;
  pa.Xq = Xq;
  pa.ldq = ldq;
  pa.sx = sx;
  pa.Xo = (_Float16*)Xo;
  pa.ldo = ldo;
  pa.ocap = max_outliers < kOcap ? max_outliers : kOcap;
  pa.wo_skip = -1;
  pa.vec = (K % 8 == 0) && aligned(X, 16);
  launch_prep(pa, stream);
  return hip_status();
}

i8mm_status int8_outlier_weights(const int8_t* CB, const float* SCB, int64_t N, int64_t K,
                                 const uint32_t* mask, int64_t max_outliers, void* Wo,
                                 int64_t ldo, hipStream_t stream) {
  if (N <= 0 || K <= 0 || max_outliers < 0 || max_outliers > K) return I8MM_ERR_INVALID_ARG;
  if (N >= kMaxDim || K > kMaxK) return I8MM_ERR_UNSUPPORTED;
  if (ldo < round_up(max_outliers, 32) || ldo % 32 != 0) return I8MM_ERR_INVALID_ARG;
  if (!CB || !SCB || !mask || !Wo || !aligned(SCB, 4) || !aligned(Wo, 2) || !aligned(mask, 4))
    return I8MM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  PrepArgs pa{};
  pa.K = K;
  pa.mask = mask;
  pa.max_o = max_outliers;
  pa.CB = CB;
  pa.SCB = SCB;
  pa.N = N;
  pa.Wo = (_Float16*)Wo;
  pa.ldo = ldo;
  pa.ocap = max_outliers < kOcap ? max_outliers : kOcap;
  pa.wo_skip = -1;
  pa.vec = false;
  launch_prep(pa, stream);
  return hip_status();
}

i8mm_status int8_gemm_s32(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb, int32_t* C,
                          int64_t T, int64_t N, int64_t K, hipStream_t stream) {
  if (T < 0 || N < 0 || K < 0 || lda < K || ldb < K) return I8MM_ERR_INVALID_ARG;
  if (T >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return I8MM_ERR_UNSUPPORTED;
  if (T == 0 || N == 0) return I8MM_OK;
  if (!C || !aligned(C, 4) || (K > 0 && (!A || !B))) return I8MM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  GemmArgs a{};
  a.cfg = -1;  // the best unsplit tile configuration
  a.A = B;  // weight side (rows = output columns of C)
  a.lda = ldb;
  a.B = A;  // activation side (rows = rows of C)
  a.ldb = lda;
  a.N = N;
  a.T = T;
  a.K = K;
  a.C = C;
  const hipError_t ge = gemm_i8_supported(a) ? launch_gemm_i8_s32(a, stream)
                                             : launch_gemm_s32(a, stream);
  if (ge != hipSuccess) return I8MM_ERR_HIP;
  return hip_status();
}

i8mm_status i8mm_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on && g_prof_ev.empty()) {
    g_prof_ev.resize((size_t)kProfCap * 4);
    for (auto& e : g_prof_ev)
      if (hipEventCreate(&e) != hipSuccess) return I8MM_ERR_HIP;
  }
  g_prof_on = on != 0;
  g_prof_n = 0;
  return I8MM_OK;
}

i8mm_status i8mm_profile_read(double* ms_sum, int64_t* calls) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double acc[4] = {0, 0, 0, 0};
  for (int c = 0; c < g_prof_n; ++c) {
    hipEvent_t* ev = &g_prof_ev[(size_t)c * 4];
    if (hipEventSynchronize(ev[3]) != hipSuccess) return I8MM_ERR_HIP;
    float t;
    for (int s = 0; s < 3; ++s) {
      if (hipEventElapsedTime(&t, ev[s], ev[s + 1]) != hipSuccess) return I8MM_ERR_HIP;
      acc[s] += t;
    }
    if (hipEventElapsedTime(&t, ev[0], ev[3]) != hipSuccess) return I8MM_ERR_HIP;
    acc[3] += t;
  }
  for (int s = 0; s < 4; ++s) {
    if (ms_sum) ms_sum[s] = acc[s];
    if (calls) calls[s] = g_prof_n;
  }
  return I8MM_OK;
}

}  // extern "C"
