"""CPU oracle for the LLM.int8() mixed-precision linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product (the HIP
library and its Python binding) never calls it and shares no code with it.

What it computes, and where the pages say so:

* Hugging Face "LLM.int8() を Transformers と Accelerate に統合" summary
  (agentlenshq.com), section "LLM.int8() の核心アイデア": three steps --
  (1) find the hidden dims (columns of the hidden-state matrix X) holding a
  value whose magnitude crosses a threshold of about 6; (2) multiply those
  columns in fp16 and everything else in int8, with vector-wise quantization
  (one scale per row of X, one per output channel of W); (3) dequantize the
  int8 result to fp16 and add the fp16 outlier result.
* Same page, section "量子化の仕組み：ゼロポイント vs. absmax": absmax
  quantization divides a vector by its largest magnitude, multiplies by 127
  and rounds, so codes stay in [-127, 127]; worked example
  [1.2, -0.5, -4.3, ..., 5.4] -> scale 127/5.4 ~= 23.5.
* Same page, section "transformers への統合": after the move to the GPU the
  weight is an int8 tensor in [-127, 127] (``weight.CB``) and the fp16 weight
  is recovered as CB * SCB / 127; ``Linear8bitLt`` keeps no fp16 weight when
  ``has_fp16_weights=False`` and the default threshold is 6.0 (section
  "accelerate を使ったゼロメモリモデル構築").
* zenn.dev summary of the LLM.int8() paper, section "手法": the outlier dims
  are split off by the input's hidden dims, the matching weight dims are split
  off too, and the outlier part runs in 16 bit to avoid cancellation and
  overflow.

Readings where the pages leave a step open (each also listed in the design
notes of the repository):

* threshold test is ``|x| >= threshold``, over all rows of this call;
* the row scale of X is the absmax over the non-outlier columns only;
* the weight scale is the absmax of the whole output-channel row of W;
* scales are stored as the absmax itself (5.4 in the worked example), fp32;
* a code is round-half-away-from-zero of the fp32 quotient fl32(x*127)/s,
  with s == 0 giving code 0; x*127 is exact in fp32 for fp16 x;
* the outlier weights are dequantized from CB: Wo = fp16(fl32(fl32(c*s)/127));
* the outlier product and the final sum are evaluated in float64 here and
  rounded once to fp16 (round to nearest even).

Floating point in this module is float64 except where the method's integer
codes are decided: those quotients are formed in float32, the precision the
HIP kernels use, so both sides make the same decision.

Pins (what ties this module to something other than itself) live in
``tests/test_oracle.py``: the worked absmax example, the CB*SCB/127 identity
bound, code-range/row-max/sign invariants, pure-Python brute force for the
detection and the integer product, a brute-force float64 X.W^T + b within the
analytic quantization-error bound, and the two special cases that reduce to a
plain product (no outliers; every column an outlier).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rhaz", "absmax_codes", "quantize_weight", "find_outliers", "quantize_rows",
    "gather_outliers", "int8_matmul", "outlier_matmul", "aggregate",
    "linear_forward", "linear_forward_fp16w", "linear_forward_sampled", "error_bound",
    "quantize_rows_zeropoint", "linear_forward_zeropoint", "error_bound_zeropoint",
]

INT8_MAX = 127


def rhaz(v: np.ndarray) -> np.ndarray:
    """Round half away from zero.

    ``v`` holds float32 values; widening to float64 makes ``v + 0.5`` exact
    for |v| <= 127, so ``trunc`` gives the exact rounding.  NumPy's
    ``round`` rounds half to even and is deliberately not used.
    """
    v64 = np.asarray(v, dtype=np.float64)
    return np.trunc(v64 + np.copysign(0.5, v64))


def absmax_codes(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """int8 codes of ``x`` under absmax scale ``s`` (broadcast), absmax section.

    code = rhaz(fl32(fl32(x * 127) / s)); a zero scale gives code 0.
    """
    x32 = np.asarray(x, dtype=np.float32)
    s32 = np.asarray(s, dtype=np.float32)
    num = (x32 * np.float32(INT8_MAX)).astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1), s32).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (num / safe).astype(np.float32)
    q = rhaz(quot)
    q = np.where(s32 == 0, 0.0, q)
    assert np.all(np.abs(q) <= INT8_MAX), "absmax code out of [-127,127]"
    return q.astype(np.int8)


def quantize_weight(W: np.ndarray):
    """Weight -> (CB int8 [N,K], SCB fp32 [N]).

    One scale per output channel, i.e. per row of W[N,K] ("重みは列単位" on the
    Hugging Face summary, core-idea section, read for the nn.Linear layout),
    taken over the whole row because the weight is quantized at load time,
    before any activation is seen (section "transformers への統合").
    """
    W = np.asarray(W)
    assert W.dtype == np.float16 and W.ndim == 2
    a = np.abs(W.astype(np.float32))
    SCB = a.max(axis=1) if W.shape[1] > 0 else np.zeros(W.shape[0], np.float32)
    CB = absmax_codes(W, SCB[:, None])
    return CB, SCB.astype(np.float32)


def find_outliers(X: np.ndarray, threshold: float) -> np.ndarray:
    """Step (1): ascending indices of the columns of X with any |x| >= threshold."""
    X = np.asarray(X)
    assert X.dtype == np.float16 and X.ndim == 2
    assert np.all(np.isfinite(X)), "non-finite activations are out of contract"
    thr = np.float32(threshold)
    flag = (np.abs(X.astype(np.float32)) >= thr).any(axis=0)
    return np.flatnonzero(flag).astype(np.int64)


def quantize_rows(X: np.ndarray, O: np.ndarray):
    """Step (2), activation side: (Xq int8 [T,K], sx fp32 [T]).

    sx[i] is the absmax of row i over the columns not in O (0 when none is
    left); Xq[:, O] = 0 because those columns go through the fp16 product.
    """
    X = np.asarray(X)
    T, K = X.shape
    keep = np.ones(K, dtype=bool)
    keep[np.asarray(O, dtype=np.int64)] = False
    a = np.abs(X.astype(np.float32))
    a_kept = np.where(keep[None, :], a, np.float32(0))
    sx = a_kept.max(axis=1) if K > 0 else np.zeros(T, np.float32)
    X_kept = np.where(keep[None, :], X, np.float16(0))
    Xq = absmax_codes(X_kept, sx[:, None])
    return Xq, sx.astype(np.float32)


def quantize_rows_zeropoint(X: np.ndarray, O: np.ndarray):
    """Zero-point (asymmetric) row quantization of X's kept columns:
    (Xq int8 [T,K], sx fp32 [T], Z int32 [T]).

    The zenn.dev summary's "Zeropoint Quantization" section: absmax leaves
    half of [-127, 127] unused for one-signed inputs (ReLU outputs), so the
    row is min-max normalized with S = 127*2 / (max - min) and an offset Z,
    X8 = INT8(X*S - Z), X = (X8 + Z) / S.  The offset's own formula is lost
    on the page; the Hugging Face summary's affine scheme ("Affine
    Quantization Scheme" section) fixes that zero must map to an integer code.
    Reading, per row over the columns not in O:
      a = min(0, min x), b = max(0, max x)    (the range holds 0)
      d = fl32(b - a); S = fl32(254 / d); Z = rhaz(fl32(a * S)) + 127
      code = clamp(rhaz(fl32(fl32(x * S) - Z)), -127, 127), 0 on O
      sx = fl32(d / 2), so that x ~= (code + Z) * sx / 127
    A row with b == a (all kept values 0, or none kept) gets S = Z = sx = 0
    and codes 0.  Zero maps to the code -Z exactly.
    """
    X = np.asarray(X)
    T, K = X.shape
    keep = np.ones(K, dtype=bool)
    keep[np.asarray(O, dtype=np.int64)] = False
    x32 = X.astype(np.float32)
    Xq = np.zeros((T, K), dtype=np.int8)
    sx = np.zeros(T, dtype=np.float32)
    Z = np.zeros(T, dtype=np.int32)
    for i in range(T):
        v = x32[i, keep]
        a = np.float32(min(0.0, float(v.min()))) if v.size else np.float32(0)
        b = np.float32(max(0.0, float(v.max()))) if v.size else np.float32(0)
        if b == a:
            continue
        d = np.float32(b - a)
        S = np.float32(np.float32(2 * INT8_MAX) / d)
        z = int(rhaz(np.float32(a * S))) + INT8_MAX
        t = (x32[i] * S).astype(np.float32)
        t = (t - np.float32(z)).astype(np.float32)
        q = np.clip(rhaz(t), -INT8_MAX, INT8_MAX)
        q = np.where(keep, q, 0.0)
        Xq[i] = q.astype(np.int8)
        sx[i] = np.float32(d / np.float32(2))
        Z[i] = z
    return Xq, sx, Z


def gather_outliers(X: np.ndarray, CB: np.ndarray, SCB: np.ndarray, O: np.ndarray):
    """Step (2), outlier side: Xo = X[:, O] (fp16) and the matching weight dims.

    The weight dims are recovered from the int8 weight as CB * SCB / 127
    ("transformers への統合"): Wo[j, o] = fp16(fl32(fl32(CB[j, O[o]] * SCB[j]) / 127)).
    """
    O = np.asarray(O, dtype=np.int64)
    Xo = np.asarray(X)[:, O].astype(np.float16)
    c = CB[:, O].astype(np.float32)
    prod = (c * SCB.astype(np.float32)[:, None]).astype(np.float32)
    Wo = (prod / np.float32(INT8_MAX)).astype(np.float32).astype(np.float16)
    return Xo, Wo


def int8_matmul(Xq: np.ndarray, CB: np.ndarray) -> np.ndarray:
    """Step (2), int8 side: acc[i, j] = sum_k Xq[i, k] * CB[j, k], exact.

    Evaluated as a float64 product: every partial sum is an integer of
    magnitude <= K * 127^2 < 2^53, so the result is exact.  Returned as int64
    after checking it fits the int32 accumulator the method uses.
    """
    acc = Xq.astype(np.float64) @ CB.astype(np.float64).T
    out = acc.astype(np.int64)
    assert np.array_equal(out.astype(np.float64), acc)
    assert np.all(np.abs(out) < 2 ** 31), "int32 accumulator overflow"
    return out


def outlier_matmul(Xo: np.ndarray, Wo: np.ndarray) -> np.ndarray:
    """Step (2), fp16 side: P = Xo . Wo^T, in float64."""
    return Xo.astype(np.float64) @ Wo.astype(np.float64).T


def aggregate(acc, sx, SCB, P, bias):
    """Step (3): Y = fp16(acc * sx[i] * SCB[j] / 127^2 + P + bias[j]), float64 inside."""
    Y = acc.astype(np.float64) * (sx.astype(np.float64)[:, None]
                                  * SCB.astype(np.float64)[None, :]) / float(INT8_MAX ** 2)
    Y = Y + P
    if bias is not None:
        Y = Y + np.asarray(bias).astype(np.float64)[None, :]
    return Y.astype(np.float16)


def linear_forward(X, CB, SCB, bias, threshold, return_stages=False):
    """The whole layer: Y fp16 [T,N] for X fp16 [T,K] and the int8 weight (CB, SCB)."""
    O = find_outliers(X, threshold)
    Xq, sx = quantize_rows(X, O)
    Xo, Wo = gather_outliers(X, CB, SCB, O)
    acc = int8_matmul(Xq, CB)
    P = outlier_matmul(Xo, Wo)
    Y = aggregate(acc, sx, SCB, P, bias)
    if return_stages:
        return Y, dict(O=O, Xq=Xq, sx=sx, Xo=Xo, Wo=Wo, acc=acc, P=P)
    return Y


def linear_forward_fp16w(X, W, bias, threshold, return_stages=False):
    """The layer with the fp16 weight kept (``Linear8bitLt`` has a
    ``has_fp16_weights`` flag; the pages show only its False side).  Reading
    for the True side: W is quantized on every call exactly as above, and the
    outlier weight dims are W's own values, Wo = W[:, O] -- the outlier part
    then multiplies the original fp16 numbers, which is what splitting off the
    weight dims in 16 bit ("手法" section of the zenn.dev summary) means when
    the fp16 weight is at hand."""
    CB, SCB = quantize_weight(W)
    O = find_outliers(X, threshold)
    Xq, sx = quantize_rows(X, O)
    Xo = np.asarray(X)[:, O].astype(np.float16)
    Wo = np.asarray(W)[:, O].astype(np.float16)
    acc = int8_matmul(Xq, CB)
    P = outlier_matmul(Xo, Wo)
    Y = aggregate(acc, sx, SCB, P, bias)
    if return_stages:
        return Y, dict(O=O, Xq=Xq, sx=sx, Xo=Xo, Wo=Wo, acc=acc, P=P, CB=CB, SCB=SCB)
    return Y


def linear_forward_zeropoint(X, CB, SCB, bias, threshold, return_stages=False):
    """The layer with zero-point activation quantization (see
    ``quantize_rows_zeropoint``); the weight side is unchanged.  Since
    x ~= (q + Z) sx / 127 on the kept columns, the int8 part is
    (sx s / 127^2) (sum_k q c + Z R_j), with R_j = sum of CB[j, k] over the
    kept columns -- an exact integer correction, then the same dequantize and
    aggregate step."""
    O = find_outliers(X, threshold)
    Xq, sx, Z = quantize_rows_zeropoint(X, O)
    Xo, Wo = gather_outliers(X, CB, SCB, O)
    K = X.shape[1]
    keep = np.ones(K, dtype=bool)
    keep[O] = False
    R = (CB.astype(np.int64) * keep[None, :]).sum(axis=1)
    acc = int8_matmul(Xq, CB) + Z.astype(np.int64)[:, None] * R[None, :]
    P = outlier_matmul(Xo, Wo)
    Y = aggregate(acc, sx, SCB, P, bias)
    if return_stages:
        return Y, dict(O=O, Xq=Xq, sx=sx, Z=Z, R=R, Xo=Xo, Wo=Wo, acc=acc, P=P)
    return Y


def error_bound_zeropoint(X, W, CB, SCB, O, Xq, sx, Z, Y):
    """``error_bound`` for the zero-point layer: a kept activation is
    x = (sx/127)(q + Z + d) with |d| <= 1/2 plus the fp32 roundings of x*S,
    of S and of sx (relative 2^-22 of |q + Z| at most), so |q| becomes
    |q + Z| in the int8 term."""
    T, K = X.shape
    keep = np.ones(K, dtype=bool)
    keep[np.asarray(O, dtype=np.int64)] = False
    qz = np.abs(Xq.astype(np.float64) + Z.astype(np.float64)[:, None]) * keep[None, :]
    c = np.abs(CB.astype(np.float64))
    nk = keep.sum()
    csum = (c * keep[None, :]).sum(1)[None, :]
    term_int = 0.5 * qz.sum(1)[:, None] + 0.5 * csum + 0.25 * nk
    term_int = term_int + (2.0 ** -15) * (qz.sum(1)[:, None] + csum + nk)
    scale = sx.astype(np.float64)[:, None] * SCB.astype(np.float64)[None, :] / 127.0 ** 2
    ax = np.abs(X.astype(np.float64))
    xo = (ax * (~keep)[None, :]).sum(1)
    term_out = xo[:, None] * (SCB.astype(np.float64)[None, :] * (1.0 / 254 + 2.0 ** -10))
    slack = 1e-6 * (ax @ np.abs(W.astype(np.float64)).T)
    return scale * term_int + term_out + 0.5 * ulp16(Y) + slack


def linear_forward_sampled(X, CB_rows, SCB_rows, bias_rows, threshold, rows, O=None):
    """Y restricted to rows ``rows`` of X and the output channels whose weight
    rows are given (CB_rows, SCB_rows, bias_rows); detection still sees all of X.
    """
    if O is None:
        O = find_outliers(X, threshold)
    Xs = np.asarray(X)[np.asarray(rows)]
    Xq, sx = quantize_rows(Xs, O)
    Xo, Wo = gather_outliers(Xs, CB_rows, SCB_rows, O)
    acc = int8_matmul(Xq, CB_rows)
    P = outlier_matmul(Xo, Wo)
    return aggregate(acc, sx, SCB_rows, P, bias_rows), O


def ulp16(y: np.ndarray) -> np.ndarray:
    """Spacing of fp16 at |y| (subnormal spacing 2^-24 near zero)."""
    a = np.abs(np.asarray(y, dtype=np.float16))
    return np.spacing(a).astype(np.float64)


def error_bound(X, W, CB, SCB, O, Xq, sx, Y):
    """Analytic bound on |Y - (X.W^T + b)| per element (float64 [T,N]).

    Writing a kept activation as x = (sx/127)(q + d) and a weight as
    w = (s/127)(c + e) with |d|, |e| <= 1/2 (plus the fp32 quotient's own
    rounding), the int8 part misses (sx*s/127^2)(|q|/2 + |c|/2 + 1/4) per
    kept k.  An outlier k uses the exact x and Wo, which is within s/254 of w
    plus Wo's fp16 rounding (<= 2^-10 s).  Y adds half an fp16 ulp, and a
    1e-6 relative slack covers float64/float32 noise.
    """
    T, K = X.shape
    keep = np.ones(K, dtype=bool)
    keep[np.asarray(O, dtype=np.int64)] = False
    q = np.abs(Xq.astype(np.float64)) * keep[None, :]
    c = np.abs(CB.astype(np.float64))
    nk = keep.sum()
    term_int = 0.5 * (q.sum(1)[:, None]) + 0.5 * ((c * keep[None, :]).sum(1)[None, :]) + 0.25 * nk
    # fp32 quotient rounding adds at most 127*2^-24 to each |d|, |e|
    term_int = term_int + (2.0 ** -17) * (q.sum(1)[:, None] + (c * keep[None, :]).sum(1)[None, :] + nk)
    scale = sx.astype(np.float64)[:, None] * SCB.astype(np.float64)[None, :] / 127.0 ** 2
    ax = np.abs(X.astype(np.float64))
    xo = (ax * (~keep)[None, :]).sum(1)
    term_out = xo[:, None] * (SCB.astype(np.float64)[None, :] * (1.0 / 254 + 2.0 ** -10))
    slack = 1e-6 * (ax @ np.abs(W.astype(np.float64)).T)
    return scale * term_int + term_out + 0.5 * ulp16(Y) + slack
