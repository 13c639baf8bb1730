/*
 * i8mm.h -- C ABI of libi8mm, an MI355X (gfx950) implementation of the
 * LLM.int8() mixed-precision linear layer  Y = X . W^T + b.
 *
 * The method, as the pages describe it:
 *   Hugging Face "LLM.int8() を Transformers と Accelerate に統合" summary
 *   (agentlenshq.com), section "LLM.int8() の核心アイデア", steps 1-3:
 *   (1) the hidden dims of X (columns) holding a value of magnitude above a
 *       threshold (~6) are outliers;
 *   (2) outlier columns are multiplied in fp16, the rest is quantized
 *       vector-wise (one absmax scale per row of X, one per output channel
 *       of W) and multiplied in int8;
 *   (3) the int8 result is dequantized and added to the fp16 result.
 *   Absmax quantization: section "量子化の仕組み" (divide by the absmax,
 *   multiply by 127, round; codes in [-127, 127]).  The weight is stored as
 *   int8 CB plus a scale SCB with W ~= CB * SCB / 127: section
 *   "transformers への統合".  The split also takes the matching weight dims:
 *   zenn.dev LLM.int8() summary, section "手法".
 *
 * Conventions that hold for every entry point:
 *   - All tensor arguments are DEVICE pointers (memory of the GPU that is
 *     current when the call is made), owned by the caller.  The library
 *     never allocates, frees or keeps them.
 *   - fp16 means IEEE binary16 (_Float16 / torch.float16); every tensor is
 *     row-major and dense unless a leading dimension (ld*) is given, in
 *     elements.
 *   - Every call only validates arguments on the host and enqueues kernels
 *     on `stream` (NULL = the default stream).  It does not synchronize,
 *     except int8_linear_status, which says so.  Results are ready when the
 *     stream has reached that point.
 *   - The return value reports host-detectable errors and launch failures
 *     (I8MM_ERR_HIP, from hipGetLastError after the launches).  Errors found
 *     on the device (more outliers than max_outliers) are reported through
 *     the workspace and read back with int8_linear_status.
 *   - Quantized codes use round-half-away-from-zero of the IEEE fp32
 *     quotient fl32(x * 127) / s; a zero scale gives code 0.  Codes are in
 *     [-127, 127]; -128 never appears.
 *   - Activations must be finite; non-finite inputs give undefined results.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef I8MM_H
#define I8MM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define I8MM_ABI_VERSION 9

typedef enum {
  I8MM_OK = 0,
  I8MM_ERR_INVALID_ARG = 1,     /* null pointer, negative size, bad threshold, misalignment */
  I8MM_ERR_WORKSPACE = 2,       /* ws_bytes smaller than the size query returns */
  I8MM_ERR_UNSUPPORTED = 3,     /* shape the library cannot handle (sizes above 2^31-1) */
  I8MM_ERR_HIP = 4,             /* a HIP runtime call or kernel launch failed */
  I8MM_ERR_OUTLIER_OVERFLOW = 5 /* device found more outlier columns than max_outliers */
} i8mm_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* i8mm_status_string(i8mm_status s);

/* I8MM_ABI_VERSION of the built library. */
int i8mm_abi_version(void);

/*
 * Tuning and test control, process-wide: the number of workgroups that share
 * each output tile of the int8 product at T > 32, each walking 1/splits of K
 * (split K; the partial int32 sums are added exactly, so Y does not depend on
 * it).  0 (the default) lets the library choose per shape -- it splits only
 * when the output tiles cannot fill the GPU, e.g. K-heavy down projections.
 * Values above 4, or above the 128-byte slices of K, are clamped.  Not
 * synchronized with calls in flight on other host threads.  splits < 0 ->
 * I8MM_ERR_INVALID_ARG.
 */
i8mm_status i8mm_set_split_override(int64_t splits);

/*
 * Tuning and test control, process-wide: the output tile of the int8
 * product at T > 32 -- 0: 320 channels x 256 tokens, 1: 256 x 256, 2: 192 x
 * 256, 3: 320 x 128.  -1 (the default) lets the library choose per shape.  The tile does
 * not change Y: every element is computed with the same operations in the
 * same order.  Not synchronized with calls in flight on other host threads;
 * size workspaces under the same setting.  cfg < -1 or cfg > 3 ->
 * I8MM_ERR_INVALID_ARG.
 */
i8mm_status i8mm_set_tile_override(int64_t cfg);

/*
 * Tuning and test control, process-wide: 1 (the default) takes steps 1-2
 * of a forward of one to eight tokens of the absmax layer (1 <= T <= 8, K a
 * multiple of 16 up to 16384, X 16-byte aligned; steps 1-2 of "LLM.int8()
 * の核心アイデア") from one launch of T workgroups, workgroup i holding row
 * i -- each reads all T rows for the column flags, so no mask and no
 * detection launch are needed -- and the product kernel takes the weights
 * of outlier sets of any width out of CB itself; 0 runs the detection and
 * step-2 launches of every other call.  The workspace holds the same values
 * either way (the mask is not used), and so does Y for outlier sets of up
 * to 128 columns (wider sets sum their fp16 products in another order).
 * Not synchronized with calls in flight on other host threads.  enable not
 * 0 or 1 -> I8MM_ERR_INVALID_ARG.
 */
i8mm_status i8mm_set_row_prep(int enable);

/*
 * Weight quantization (done once per weight, when it is moved to the GPU;
 * "transformers への統合" section of the Hugging Face summary).
 *
 *   SCB[j]   = max_k |W[j,k]|                      (fp32, exact)
 *   CB[j,k]  = rhaz(fl32(W[j,k] * 127) / SCB[j])   (0 when SCB[j] == 0)
 *
 * so that W ~= CB * SCB / 127 with |W - CB*SCB/127| <= SCB/254.
 *   W   : fp16 [N, K], nn.Linear layout (row j = output channel j)
 *   CB  : int8 [N, K] out
 *   SCB : fp32 [N]    out
 * N, K >= 0 (K == 0 gives SCB = 0).  W must be 2-byte aligned.
 */
i8mm_status int8_quantize_weight(const void* W, int64_t N, int64_t K,
                                 int8_t* CB, float* SCB, hipStream_t stream);

/*
 * Workspace of int8_linear_forward.  Every region starts on a 256-byte
 * boundary of `ws`; offsets are in bytes from `ws`.  counts and mask come
 * first and at the same offsets for every shape (the mask region has room
 * for the largest K), so one workspace, initialized once, serves forwards
 * of any shapes in turn as long as it is large enough for each.
 */
typedef struct {
  size_t counts;   /* int32[4]: n_o (true count), overflow flag, 0, 0          */
  size_t outliers; /* int32[max_outliers]: outlier columns O, ascending       */
  size_t mask;     /* uint32[ceil(K/32)] in use of 2^13 words: bit k set iff   */
                   /* column k is an outlier (left zero by every forward)      */
  size_t sx;       /* fp32[T]: row scales (absmax over non-outlier columns;    */
                   /* zero-point layer: half their range, see below)           */
  size_t xq;       /* int8[T][ldq]: quantized X, outlier and pad columns 0     */
  size_t xo;       /* fp16[T][ldo]: X[:, O], zero-padded to ldo                */
  size_t wo;       /* fp16[N][ldo]: fp16(CB[:, O] * SCB / 127), zero-padded    */
  size_t zp;       /* int32[T]: zero-point offsets Z of the rows (zero-point   */
                   /* layer only)                                              */
  size_t osum;     /* int32[N]: sum_o CB[j, O_o] (zero-point layer, n_o > 0)   */
  size_t part;     /* int32 partial accumulators of a K-split product: one    */
                   /* tile of the product per split (0 bytes when splits == 1) */
  int64_t ldq;     /* row pitch of xq in bytes (K rounded up to 64)            */
  int64_t ldo;     /* row pitch of xo and wo in elements (max_outliers up to 32) */
  int64_t splits;  /* workgroups that share each output tile of the product,  */
                   /* each walking 1/splits of K (1: no split)                 */
  size_t total;    /* bytes the workspace must hold                            */
} i8mm_ws_layout;

/*
 * Fill *out for a forward call of this shape.  max_outliers in [0, K].
 * The K split (and so the size) is chosen for the current device's compute
 * unit count and the split override below; size the workspace on the
 * device, and under the override, that the forward will run with.
 */
i8mm_status int8_linear_workspace_layout(int64_t T, int64_t N, int64_t K,
                                         int64_t max_outliers, i8mm_ws_layout* out);

/* out->total of the layout above (0 on invalid arguments). */
size_t int8_linear_workspace_size(int64_t T, int64_t N, int64_t K, int64_t max_outliers);

/*
 * Make a workspace ready for the forward calls below: zero-fills its head
 * (counts and the whole mask region; a fill kernel on `stream`, no memset).
 * Call it once per workspace before its first forward.  Every forward
 * leaves the mask zero again (its product kernel clears it after step 2 has
 * read it), which saves the next call a clearing launch, and the mask's
 * place does not depend on the shape: forwards of other shapes may follow
 * on the same workspace without a new initialization.  A workspace whose
 * forward returned an error, or that held something else meanwhile, must be
 * initialized again.  Arguments as int8_linear_workspace_layout (the shape
 * only checks them); ws 256-byte aligned.
 */
i8mm_status int8_linear_workspace_init(void* ws, int64_t T, int64_t N, int64_t K,
                                       int64_t max_outliers, hipStream_t stream);

/*
 * The layer (steps 1-3 of "LLM.int8() の核心アイデア"):
 *
 *   O      = ascending { k : exists i, |X[i,k]| >= threshold }
 *   sx[i]  = max_{k not in O} |X[i,k]|
 *   Xq     = rhaz(fl32(X * 127) / sx[i]) on columns not in O, 0 on O
 *   acc    = Xq . CB^T                                   (exact, int32)
 *   Wo     = fp16(fl32(fl32(CB[:,O] * SCB[j]) / 127))
 *   Y[i,j] = fp16( acc*sx[i]*SCB[j]/127^2 + sum_o X[i,O_o]*Wo[j,o] + bias[j] )
 *            (fp32 arithmetic, one final round-to-nearest-even)
 *
 *   X        : fp16 [T, K]
 *   CB, SCB  : from int8_quantize_weight, [N, K] and [N]
 *   bias     : fp16 [N], or NULL for no bias
 *   threshold: > 0; +inf means no column is an outlier (plain vector-wise
 *              int8).  NaN or <= 0 -> I8MM_ERR_INVALID_ARG.
 *   Y        : fp16 [T, N] out; must not overlap X, CB or the workspace
 *   ws       : device workspace, 256-byte aligned, ws_bytes >=
 *              int8_linear_workspace_size(T, N, K, max_outliers),
 *              initialized (int8_linear_workspace_init) before its first
 *              forward; its regions hold the intermediate results after
 *              the call (see i8mm_ws_layout), except the mask, which the
 *              call leaves zero
 *   max_outliers: capacity of O, in [0, K]; K is always enough.  If the
 *              device finds more, Y is undefined and int8_linear_status
 *              returns I8MM_ERR_OUTLIER_OVERFLOW; no memory outside the
 *              arguments is touched.
 * T, N, K >= 0; T == 0 or N == 0 is a no-op; K == 0 gives Y = bias (or 0).
 */
i8mm_status int8_linear_forward(const void* X, int64_t T, int64_t K,
                                const int8_t* CB, const float* SCB, int64_t N,
                                const void* bias, float threshold, void* Y,
                                void* ws, size_t ws_bytes, int64_t max_outliers,
                                hipStream_t stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, serving
 * loops that forbid hipMalloc, harnesses that do): int8_linear_forward
 * without a workspace argument.  Its workspace is a library-owned device
 * array of I8MM_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from the
 * first call on that GPU until the process ends.  The call itself allocates
 * nothing (no hipMalloc, no allocating library routine).
 *
 *   X, CB, SCB, bias, threshold, Y, max_outliers, stream:
 *            as int8_linear_forward; same kernels, so Y is bit-identical to
 *            that call's with the same max_outliers.
 *   status : NULL, or caller-owned device memory of 4 int32 (4-byte
 *            aligned) that receives [outlier columns found, 1 if more than
 *            max_outliers (Y then undefined) else 0, 0, 0] when the stream
 *            reaches the end of the call.  The intermediate results stay in
 *            the library's array and are not exposed.
 *
 * I8MM_ERR_WORKSPACE when int8_linear_workspace_size(T, N, K, max_outliers)
 * exceeds I8MM_NOALLOC_SCRATCH_BYTES (for example T = 2048, K = 5120,
 * N = 13824 fits up to about 1500 outlier columns).  Every call on a GPU
 * uses that GPU's one array: calls whose execution overlaps on one GPU
 * (other streams, other threads) race and give undefined results; calls in
 * one stream order are safe.  Each call clears the part of the array that
 * must start at zero (a fill kernel, not a memset).
 */
#define I8MM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
i8mm_status int8_linear_forward_noalloc(const void* X, int64_t T, int64_t K,
                                        const int8_t* CB, const float* SCB, int64_t N,
                                        const void* bias, float threshold, void* Y,
                                        int64_t max_outliers, int32_t* status,
                                        hipStream_t stream);

/*
 * The layer with the fp16 weight kept (the pages' Linear8bitLt interface has
 * a has_fp16_weights flag; this is the True side of it, in the reading that
 * the layer then quantizes W on every call and takes the outlier weight dims
 * from W itself):
 *
 *   CB, SCB = int8_quantize_weight(W)            (written to CB/SCB)
 *   Wo      = W[:, O]                            (exact, no CB round trip)
 *   Y       = as int8_linear_forward with that Wo
 *
 *   W   : fp16 [N, K], 2-byte aligned
 *   CB  : int8 [N, K] out (overwritten every call), SCB : fp32 [N] out
 * Other arguments, the workspace and the errors as int8_linear_forward.
 * K == 0 gives Y = bias (or 0) and leaves CB/SCB unwritten.
 */
i8mm_status int8_linear_forward_fp16w(const void* X, int64_t T, int64_t K, const void* W,
                                      int64_t N, const void* bias, float threshold, int8_t* CB,
                                      float* SCB, void* Y, void* ws, size_t ws_bytes,
                                      int64_t max_outliers, hipStream_t stream);

/*
 * Zero-point (asymmetric) activation quantization ("Zeropoint Quantization"
 * section of the zenn.dev LLM.int8() summary: S = 127*2 / (max - min),
 * X8 = INT8(X*S - Z); zero is an integer code as in the Hugging Face
 * summary's affine scheme).  Per row i over the columns not in O:
 *
 *   a = min(0, min x), b = max(0, max x), d = fl32(b - a)
 *   S = fl32(254 / d), Z[i] = rhaz(fl32(a * S)) + 127
 *   Xq = clamp(rhaz(fl32(fl32(x * S) - Z)), -127, 127), 0 on O
 *   sx[i] = d / 2                       (x ~= (Xq + Z) * sx / 127)
 *   (b == a: S = Z = sx = 0, codes 0)
 *   Y[i,j] = fp16( (acc + Z[i] * R[j]) * sx[i] * SCB[j] / 127^2
 *                  + sum_o X[i,O_o] * Wo[j,o] + bias[j] )
 *   with R[j] = sum over the columns not in O of CB[j, k]
 *
 * The weight side is unchanged (int8_quantize_weight).  rsum = CB's row sums
 * over all K, int32 [N], from int8_weight_rowsum (once per weight).  The
 * offset term is added in fp32 (as the product of a per-row and a
 * per-channel factor); everything else, the workspace (zp and osum regions)
 * and the errors are as int8_linear_forward.
 */
i8mm_status int8_weight_rowsum(const int8_t* CB, int64_t N, int64_t K, int32_t* rsum,
                               hipStream_t stream);
i8mm_status int8_linear_forward_zeropoint(const void* X, int64_t T, int64_t K, const int8_t* CB,
                                          const float* SCB, const int32_t* rsum, int64_t N,
                                          const void* bias, float threshold, void* Y, void* ws,
                                          size_t ws_bytes, int64_t max_outliers,
                                          hipStream_t stream);

/*
 * Synchronizes `stream`, then reads the counts of the last forward call that
 * used `ws`: *n_outliers = number of outlier columns found (may exceed
 * max_outliers).  Returns I8MM_ERR_OUTLIER_OVERFLOW if it did, else I8MM_OK.
 * n_outliers may be NULL.
 */
i8mm_status int8_linear_status(const void* ws, int32_t* n_outliers, hipStream_t stream);

/* ---- stage entry points (the same kernels the forward runs) -------------- */

/*
 * Step 1 alone.  Writes the bit mask mask[ceil(K/32)] (bit k%32 of word
 * k/32 set iff some |X[i,k]| >= threshold), counts[0] = n_o, counts[1] =
 * overflow (n_o > max_outliers), counts[2..3] = 0, and O[0 .. min(n_o,
 * max_outliers)) ascending.  counts: int32[4].  T, K > 0.
 * (The forward runs the same detection kernel; the list O and the counts
 * are then produced by the step-2 kernel from the same mask.)
 */
i8mm_status int8_find_outliers(const void* X, int64_t T, int64_t K, float threshold,
                               int32_t* O, int32_t* counts, uint32_t* mask,
                               int64_t max_outliers, hipStream_t stream);

/*
 * Step 2, activation side, for the outlier set given as a bit mask
 * (mask[ceil(K/32)], bit k%32 of word k/32; only the first max_outliers
 * outlier columns are gathered):
 *   sx[T], Xq[T][ldq] (ldq >= K bytes, multiple of 16; columns K..ldq-1 and
 *   outlier columns written as 0), Xo[T][ldo] fp16 = X[:, O] with columns
 *   n..roundup(n,32)-1 written as 0, n = min(n_o, max_outliers) (ldo a
 *   multiple of 32, ldo >= roundup(max_outliers, 32)).
 */
i8mm_status int8_quantize_rows(const void* X, int64_t T, int64_t K, const uint32_t* mask,
                               int64_t max_outliers, int8_t* Xq, int64_t ldq, float* sx,
                               void* Xo, int64_t ldo, hipStream_t stream);

/*
 * Step 2, weight side, for the outlier set given as a bit mask: Wo[N][ldo]
 * fp16, Wo[j,o] = fp16(fl32(fl32(CB[j,O[o]] * SCB[j]) / 127)) for o < n,
 * 0 for n <= o < roundup(n, 32), n = min(n_o, max_outliers).
 */
i8mm_status int8_outlier_weights(const int8_t* CB, const float* SCB, int64_t N, int64_t K,
                                 const uint32_t* mask, int64_t max_outliers, void* Wo,
                                 int64_t ldo, hipStream_t stream);

/*
 * The int8 product of step 2 with its int32 accumulators written out:
 *   C[i,j] = sum_k A[i,k] * B[j,k]   (exact; caller keeps K*127^2 < 2^31)
 *   A: int8 [T][lda], B: int8 [N][ldb], C: int32 [T][N].  lda, ldb >= K.
 */
i8mm_status int8_gemm_s32(const int8_t* A, int64_t lda, const int8_t* B, int64_t ldb,
                          int32_t* C, int64_t T, int64_t N, int64_t K, hipStream_t stream);

/* ---- instrumentation ------------------------------------------------------ */

/*
 * When enabled, every int8_linear_forward call records HIP events on its
 * stream around its stages: 0 = detect (step 1), 1 = quantize and gather
 * (step 2 prep), 2 = the fused int8/fp16 product and epilogue, 3 = the whole
 * call.  i8mm_profile_read synchronizes those events and returns, per stage,
 * the summed milliseconds and the number of calls timed since the last
 * enable (arrays of 4; either pointer may be NULL).  At most 4096 calls are
 * kept; later calls are not timed.
 */
i8mm_status i8mm_profile_enable(int on);
i8mm_status i8mm_profile_read(double* ms_sum, int64_t* calls);

#ifdef __cplusplus
}
#endif

#endif /* I8MM_H */
