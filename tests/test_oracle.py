"""Pins for the CPU oracle: what ties it to the pages and to mathematics.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something fixed outside of it (a value the pages print, a closed form, a
brute-force loop, an analytic error bound).  ``test_pins`` runs them all on
the oracle as it is; ``test_planted_mistake_is_caught`` plants one plausible
mistake at a time in the oracle (on the CPU, via monkeypatch) and checks that
at least one pin fails, so the pins are known to bite.
"""
import math

import numpy as np
import pytest

import oracle.llm_int8 as O
from tests.conftest import read_golden
from workloads import make_random_case, make_inputs


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def pin_worked_example():
    """Absmax section of the Hugging Face summary: scale 127/5.4 ~= 23.5."""
    g = read_golden("absmax_worked_example.txt")
    vals = np.array([float(v) for v in g["values"][0]])
    absmax = float(g["absmax"][0][0])
    codes = np.array([int(c) for c in g["codes"][0]])
    dec = int(g["scale_decimals"][0][0])
    assert round(127.0 / absmax, dec) == float(g["scale_printed"][0][0])
    for dtype in (np.float64, np.float16):
        v = vals.astype(dtype)
        s = np.abs(v.astype(np.float32)).max()
        q = O.absmax_codes(v, s)
        assert q.dtype == np.int8
        assert np.array_equal(q.astype(int), codes), (dtype, q)
    # same through the row quantizer with no outlier columns
    Xq, sx = O.quantize_rows(vals.astype(np.float16)[None, :], np.zeros(0, np.int64))
    assert np.array_equal(Xq[0].astype(int), codes)
    assert sx[0] == np.float32(np.float16(absmax))


def pin_rounding_ties():
    g = read_golden("rounding_ties.txt")
    vals = np.array([float(v) for v in g["values"][0]], dtype=np.float16)
    codes = np.array([int(c) for c in g["codes"][0]])
    q = O.absmax_codes(vals, np.float32(float(g["absmax"][0][0])))
    assert np.array_equal(q.astype(int), codes), q
    # the same row through the weight quantizer (its absmax is 127)
    CB, SCB = O.quantize_weight(vals[None, :])
    assert SCB[0] == 127.0
    assert np.array_equal(CB[0].astype(int), codes)


def pin_threshold_tie():
    g = read_golden("threshold_tie.txt")
    X = np.array([[float(v) for v in r] for r in g["row"]], dtype=np.float16)
    thr = float(g["threshold"][0][0])
    want = np.array([int(c) for c in g["outliers"][0]])
    got = O.find_outliers(X, thr)
    assert np.array_equal(got, want), got


def _detect_bruteforce(X, thr):
    T, K = X.shape
    out = []
    for k in range(K):
        for i in range(T):
            if abs(float(X[i, k])) >= thr:
                out.append(k)
                break
    return out


def pin_detect_bruteforce():
    for seed in range(6):
        rng = np.random.default_rng(100 + seed)
        T, K = int(rng.integers(1, 9)), int(rng.integers(1, 40))
        X = (rng.standard_normal((T, K)) * 3.0).astype(np.float16)
        thr = float(rng.choice([6.0, 4.5, 1e-3, np.inf]))
        got = O.find_outliers(X, thr)
        assert list(got) == _detect_bruteforce(X, thr)


def pin_weight_identity():
    """CB in [-127,127], row max -> +-127, |W - CB*SCB/127| <= SCB/254."""
    rng = np.random.default_rng(7)
    for N, K in [(5, 7), (17, 64), (3, 1), (40, 129)]:
        W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
        W[rng.integers(0, N)] = 0  # an all-zero row
        CB, SCB = O.quantize_weight(W)
        assert CB.dtype == np.int8 and CB.itemsize == 1 and SCB.dtype == np.float32
        assert CB.shape == (N, K) and SCB.shape == (N,)
        w = W.astype(np.float64)
        assert np.array_equal(SCB.astype(np.float64), np.abs(w).max(1))
        assert np.all(np.abs(CB.astype(int)) <= 127)
        for j in range(N):
            if SCB[j] > 0:
                kmax = int(np.argmax(np.abs(w[j])))
                assert abs(int(CB[j, kmax])) == 127
                assert np.all(np.sign(CB[j]) == np.sign(w[j]) * (CB[j] != 0))
            else:
                assert np.all(CB[j] == 0)
        rec = CB.astype(np.float64) * SCB.astype(np.float64)[:, None] / 127.0
        bound = SCB.astype(np.float64)[:, None] / 254.0 * (1 + 1e-5)
        assert np.all(np.abs(w - rec) <= bound)


def pin_row_invariants():
    for name in ("tiny",):
        d = make_inputs(name)
        X, thr = d["X"], d["threshold"]
        Ox = O.find_outliers(X, thr)
        assert set(d["planted"].tolist()) <= set(Ox.tolist())
        Xq, sx = O.quantize_rows(X, Ox)
        x = X.astype(np.float64)
        keep = np.ones(X.shape[1], bool)
        keep[Ox] = False
        assert np.all(Xq[:, ~keep] == 0)
        assert np.all(sx < thr)
        assert np.array_equal(sx.astype(np.float64), np.abs(x[:, keep]).max(1))
        assert np.all(np.abs(Xq.astype(int)) <= 127)
        for i in range(X.shape[0]):
            if sx[i] > 0:
                kk = np.flatnonzero(keep)
                kmax = kk[int(np.argmax(np.abs(x[i, kk])))]
                assert abs(int(Xq[i, kmax])) == 127
                u = x[i, keep] * 127.0 / float(sx[i])
                assert np.all(np.abs(Xq[i, keep] - u) <= 0.5 + 1e-5)
        assert np.all((np.sign(Xq[:, keep]) == np.sign(x[:, keep])) | (Xq[:, keep] == 0))


def pin_int_gemm_bruteforce():
    rng = np.random.default_rng(11)
    for T, N, K in [(3, 5, 5), (3, 4, 5), (1, 1, 1), (2, 7, 13)]:
        A = rng.integers(-127, 128, size=(T, K)).astype(np.int8)
        B = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
        got = O.int8_matmul(A, B)
        for i in range(T):
            for j in range(N):
                s = 0
                for k in range(K):
                    s += int(A[i, k]) * int(B[j, k])
                assert int(got[i, j]) == s
    # the int32 range claim at the largest K of the workloads
    assert 12288 * 127 * 127 < 2 ** 31


def _bruteforce_linear(X, W, b):
    """float64 X.W^T + b with the original (unquantized) weight, plain loops."""
    T, K = X.shape
    N = W.shape[0]
    x = X.astype(np.float64)
    w = W.astype(np.float64)
    Y = np.zeros((T, N))
    for i in range(T):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += x[i, k] * w[j, k]
            Y[i, j] = s + (float(b[j]) if b is not None else 0.0)
    return Y


def _bound_check(X, W, b, thr):
    CB, SCB = O.quantize_weight(W)
    Y, st = O.linear_forward(X, CB, SCB, b, thr, return_stages=True)
    ref = _bruteforce_linear(X, W, b)
    B = O.error_bound(X, W, CB, SCB, st["O"], st["Xq"], st["sx"], Y)
    err = np.abs(Y.astype(np.float64) - ref)
    assert np.all(err <= B), float((err - B).max())
    return Y, st


def pin_forward_bruteforce():
    shapes = [(1, 1, 1), (1, 7, 3), (3, 5, 2), (4, 9, 11), (2, 33, 5), (5, 16, 8), (3, 1, 4)]
    for s, (T, K, N) in enumerate(shapes):
        for planted in (0, 2):
            d = make_random_case(200 + s, T, K, N, n_planted=min(planted, K),
                                 bias=(s % 2 == 0))
            _bound_check(d["X"], d["W"], d["bias"], d["threshold"])
    d = make_inputs("tiny")
    _bound_check(d["X"], d["W"], d["bias"], d["threshold"])


def pin_no_outliers_is_plain_vectorwise():
    """threshold = +inf: no column is split off, sx is the full row absmax."""
    d = make_random_case(300, 4, 24, 6, n_planted=2)
    X, W, b = d["X"], d["W"], d["bias"]
    Y, st = _bound_check(X, W, b, np.inf)
    assert len(st["O"]) == 0
    assert np.array_equal(st["sx"].astype(np.float64), np.abs(X.astype(np.float64)).max(1))
    assert st["Xo"].shape == (4, 0) and st["Wo"].shape == (6, 0)


def pin_all_outliers_is_fp16_product():
    """A threshold below every |x|: all columns go through the fp16 product,
    so Y = fp16(X . Wdq^T + b) with Wdq = fp16(CB*SCB/127) -- a plain product."""
    d = make_random_case(301, 5, 12, 7)
    X, W, b = d["X"], d["W"], d["bias"]
    assert np.all(X != 0)
    CB, SCB = O.quantize_weight(W)
    Y, st = O.linear_forward(X, CB, SCB, b, 1e-6, return_stages=True)
    assert len(st["O"]) == X.shape[1]
    assert np.all(st["Xq"] == 0) and np.all(st["sx"] == 0)
    Wdq = np.array([[float(np.float16(np.float32(np.float32(int(CB[j, k]) * SCB[j]) / np.float32(127))))
                     for k in range(W.shape[1])] for j in range(W.shape[0])])
    ref = _bruteforce_linear(X, Wdq, b)
    assert np.all(np.abs(Y.astype(np.float64) - ref) <= 0.5 * O.ulp16(Y) + 1e-12)


def pin_sampled_matches_full():
    d = make_random_case(302, 9, 40, 11, n_planted=3)
    CB, SCB = O.quantize_weight(d["W"])
    Y = O.linear_forward(d["X"], CB, SCB, d["bias"], 6.0)
    rows = np.array([0, 4, 8])
    cols = np.array([1, 2, 10])
    Ys, _ = O.linear_forward_sampled(d["X"], CB[cols], SCB[cols], d["bias"][cols], 6.0, rows)
    assert np.array_equal(Ys, Y[np.ix_(rows, cols)])


def pin_fp16w_all_outliers_is_the_plain_product():
    """fp16-weight variant, every column an outlier: nothing is quantized on
    either side, so Y = fp16(X . W^T + b) with the original W -- the textbook
    product, to within half an fp16 ulp (one final rounding)."""
    for seed, (T, K, N) in enumerate([(5, 12, 7), (3, 33, 4), (1, 1, 2)]):
        d = make_random_case(310 + seed, T, K, N)
        X, W, b = d["X"], d["W"], d["bias"]
        assert np.all(X != 0)
        Y, st = O.linear_forward_fp16w(X, W, b, 1e-6, return_stages=True)
        assert len(st["O"]) == K and np.all(st["Xq"] == 0)
        ref = _bruteforce_linear(X, W, b)
        assert np.all(np.abs(Y.astype(np.float64) - ref) <= 0.5 * O.ulp16(Y) + 1e-12)


def pin_fp16w_reduces_to_int8_weight_form():
    """fp16-weight variant: with no outlier the fp16 weight is not used
    beyond its quantization, so Y equals the int8-weight layer bit for bit;
    with outliers it differs only through the outlier dims, and stays within
    the analytic bound of the brute-force product."""
    d = make_random_case(320, 6, 40, 9, n_planted=3)
    X, W, b = d["X"], d["W"], d["bias"]
    CB, SCB = O.quantize_weight(W)
    assert np.array_equal(O.linear_forward_fp16w(X, W, b, np.inf).view(np.uint16),
                          O.linear_forward(X, CB, SCB, b, np.inf).view(np.uint16))
    Y, st = O.linear_forward_fp16w(X, W, b, 6.0, return_stages=True)
    assert len(st["O"]) == 3
    assert np.array_equal(st["Wo"].view(np.uint16), W[:, st["O"]].view(np.uint16))
    ref = _bruteforce_linear(X, W, b)
    B = O.error_bound(X, W, CB, SCB, st["O"], st["Xq"], st["sx"], Y)
    assert np.all(np.abs(Y.astype(np.float64) - ref) <= B)


def pin_zeropoint_relu_row_uses_the_full_range():
    """The zenn.dev summary's "Zeropoint Quantization" motivation: a
    one-signed (post-ReLU) row uses only half of the codes under absmax but
    all of [-127, 127] under zero-point; zero maps to the integer code -Z
    (the affine scheme's zero point); the scale and offset follow the page's
    S = 127*2 / (max - min)."""
    x = np.array([[0.0, 0.5, 1.2, 5.4, 2.0, 0.0, 3.3, 0.25]], dtype=np.float16)
    q_abs, _ = O.quantize_rows(x, np.array([], dtype=np.int64))
    assert q_abs.min() >= 0 and q_abs.max() == 127
    q, sx, Z = O.quantize_rows_zeropoint(x, np.array([], dtype=np.int64))
    assert q.min() == -127 and q.max() == 127
    b = float(np.float16(5.4))
    S = np.float32(254) / np.float32(b)
    assert Z[0] == 127                       # a = 0: zero is the lowest code
    assert np.all(q[0][x[0] == 0] == -Z[0])
    assert sx[0] == np.float32(np.float32(b) / 2)
    # codes by hand for two values: x*S - Z, rounded half away from zero
    assert q[0, 2] == int(np.trunc(float(np.float32(np.float32(np.float16(1.2)) * S)) - 127 - 0.5))
    assert q[0, 4] == int(np.trunc(float(np.float32(np.float32(2.0) * S)) - 127 - 0.5))  # -32.9
    # a two-signed row with min = -max: the offset is 0, as for absmax
    q2, sx2, Z2 = O.quantize_rows_zeropoint(np.array([[-2.0, 1.0, 2.0, 0.5]], np.float16),
                                            np.array([], dtype=np.int64))
    assert Z2[0] == 0 and sx2[0] == np.float32(2.0) and q2[0, 0] == -127 and q2[0, 2] == 127


def pin_zeropoint_roundtrip_and_zero_rows():
    """Every kept x is within half a step of (q + Z) sx / 127 (plus fp32
    roundings); outlier columns get code 0; an all-zero row gets S = Z = 0."""
    d = make_random_case(330, 7, 50, 3, n_planted=2, row_frac=0.5)
    X = d["X"].copy()
    X[2] = np.abs(X[2])          # one-signed rows
    X[3] = -np.abs(X[3])
    X[4] = 0                     # all zero
    Oo = O.find_outliers(X, 6.0)
    q, sx, Z = O.quantize_rows_zeropoint(X, Oo)
    keep = np.ones(X.shape[1], bool)
    keep[Oo] = False
    assert np.all(q[:, Oo] == 0)
    assert sx[4] == 0 and Z[4] == 0 and np.all(q[4] == 0)
    xh = (q.astype(np.float64) + Z[:, None]) * sx.astype(np.float64)[:, None] / 127
    err = np.abs(xh - X.astype(np.float64))[:, keep]
    step = sx.astype(np.float64)[:, None] / 127
    assert np.all(err <= 0.5 * step * (1 + 2.0 ** -12) + 1e-12)
    assert np.all(np.abs(Z) <= 127)


def _bound_check_zeropoint(X, W, b, thr):
    CB, SCB = O.quantize_weight(W)
    Y, st = O.linear_forward_zeropoint(X, CB, SCB, b, thr, return_stages=True)
    ref = _bruteforce_linear(X, W, b)
    B = O.error_bound_zeropoint(X, W, CB, SCB, st["O"], st["Xq"], st["sx"], st["Z"], Y)
    err = np.abs(Y.astype(np.float64) - ref)
    assert np.all(err <= B), float((err - B).max())
    return Y, st


def pin_zeropoint_forward_bruteforce():
    """The zero-point layer against the brute-force float64 X.W^T + b (with
    the original W), within its analytic bound, on two-signed, one-signed and
    zero rows, with and without outliers."""
    shapes = [(1, 1, 1), (1, 7, 3), (3, 5, 2), (4, 9, 11), (2, 33, 5), (5, 16, 8)]
    for s_, (T, K, N) in enumerate(shapes):
        for planted in (0, 2):
            d = make_random_case(340 + s_, T, K, N, n_planted=min(planted, K), bias=(s_ % 2 == 0))
            X = d["X"].copy()
            X[0] = np.abs(X[0])
            _bound_check_zeropoint(X, d["W"], d["bias"], d["threshold"])
    # the int8 product alone would be off by sx*s/127^2 * Z*R: the bound
    # holds only with the correction
    d = make_random_case(350, 4, 64, 6)
    X = np.abs(d["X"])
    Y, st = _bound_check_zeropoint(X, d["W"], d["bias"], np.inf)
    assert np.all(st["Z"] == 127)


PINS = [pin_worked_example, pin_rounding_ties, pin_threshold_tie, pin_detect_bruteforce,
        pin_weight_identity, pin_row_invariants, pin_int_gemm_bruteforce,
        pin_forward_bruteforce, pin_no_outliers_is_plain_vectorwise,
        pin_all_outliers_is_fp16_product, pin_sampled_matches_full,
        pin_fp16w_all_outliers_is_the_plain_product, pin_fp16w_reduces_to_int8_weight_form,
        pin_zeropoint_relu_row_uses_the_full_range, pin_zeropoint_roundtrip_and_zero_rows,
        pin_zeropoint_forward_bruteforce]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pins(pin):
    pin()


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

def _m_round_half_even(mp):
    mp.setattr(O, "rhaz", lambda v: np.round(np.asarray(v, dtype=np.float64)))


def _m_strict_threshold(mp):
    def bad(X, threshold):
        flag = (np.abs(X.astype(np.float32)) > np.float32(threshold)).any(axis=0)
        return np.flatnonzero(flag).astype(np.int64)
    mp.setattr(O, "find_outliers", bad)


def _m_descending_outliers(mp):
    good = O.find_outliers
    mp.setattr(O, "find_outliers", lambda X, t: good(X, t)[::-1].copy())


def _m_row_scale_unmasked(mp):
    good = O.quantize_rows

    def bad(X, Oi):
        Xq, sx = good(X, np.zeros(0, np.int64))
        Xq[:, np.asarray(Oi, dtype=np.int64)] = 0
        return Xq, sx
    mp.setattr(O, "quantize_rows", bad)


def _m_outliers_not_zeroed(mp):
    def bad(X, Oi):
        keep = np.ones(X.shape[1], bool)
        keep[np.asarray(Oi, dtype=np.int64)] = False
        a = np.where(keep[None, :], np.abs(X.astype(np.float32)), 0)
        sx = a.max(1).astype(np.float32)
        Xq = np.clip(O.rhaz((X.astype(np.float32) * 127) / np.where(sx == 0, 1, sx)[:, None]), -127, 127)
        return Xq.astype(np.int8), sx
    mp.setattr(O, "quantize_rows", bad)


def _m_drop_bias(mp):
    good = O.aggregate
    mp.setattr(O, "aggregate", lambda acc, sx, s, P, b: good(acc, sx, s, P, None))


def _m_scale_127(mp):
    def bad(acc, sx, s, P, b):
        Y = acc * (sx.astype(np.float64)[:, None] * s.astype(np.float64)[None, :]) / 127.0 + P
        if b is not None:
            Y = Y + b.astype(np.float64)[None, :]
        return Y.astype(np.float16)
    mp.setattr(O, "aggregate", bad)


def _m_wo_no_scale(mp):
    def bad(X, CB, SCB, Oi):
        Oi = np.asarray(Oi, dtype=np.int64)
        return X[:, Oi].astype(np.float16), CB[:, Oi].astype(np.float16)
    mp.setattr(O, "gather_outliers", bad)


def _m_untransposed_gemm(mp):
    def bad(A, B):  # the weight used without its transpose (square shapes only)
        return (A.astype(np.float64) @ B.astype(np.float64)).astype(np.int64)
    mp.setattr(O, "int8_matmul", bad)


def _m_weight_per_column(mp):
    def bad(W):
        a = np.abs(W.astype(np.float32))
        s = a.max(axis=0)
        CB = O.absmax_codes(W, s[None, :])
        return CB, a.max(axis=1).astype(np.float32)
    mp.setattr(O, "quantize_weight", bad)


def _m_outlier_sign(mp):
    good = O.outlier_matmul
    mp.setattr(O, "outlier_matmul", lambda a, b: -good(a, b))


# zero-point layer (reading R18 of the zenn.dev "Zeropoint Quantization"
# section): the offset term, its column set, its sign, and 0 in the range

def _zp_forward(X, CB, SCB, bias, threshold, offset_cols="kept", with_offset=True):
    Oi = O.find_outliers(X, threshold)
    Xq, sx, Z = O.quantize_rows_zeropoint(X, Oi)
    Xo, Wo = O.gather_outliers(X, CB, SCB, Oi)
    keep = np.ones(X.shape[1], dtype=bool)
    if offset_cols == "kept":
        keep[Oi] = False
    R = (CB.astype(np.int64) * keep[None, :]).sum(axis=1)
    acc = O.int8_matmul(Xq, CB)
    if with_offset:
        acc = acc + Z.astype(np.int64)[:, None] * R[None, :]
    return O.aggregate(acc, sx, SCB, O.outlier_matmul(Xo, Wo), bias)


def _m_zp_drop_offset(mp):
    mp.setattr(O, "linear_forward_zeropoint",
               lambda X, CB, SCB, b, t, return_stages=False: _zp_forward(X, CB, SCB, b, t,
                                                                         with_offset=False))


def _m_zp_offset_over_all_columns(mp):
    mp.setattr(O, "linear_forward_zeropoint",
               lambda X, CB, SCB, b, t, return_stages=False: _zp_forward(X, CB, SCB, b, t,
                                                                         offset_cols="all"))


def _m_zp_offset_sign(mp):
    good = O.quantize_rows_zeropoint

    def bad(X, Oi):
        Xq, sx, Z = good(X, Oi)
        return Xq, sx, -Z
    mp.setattr(O, "quantize_rows_zeropoint", bad)


def _m_zp_range_without_zero(mp):
    def bad(X, Oi):
        T, K = X.shape
        keep = np.ones(K, dtype=bool)
        keep[np.asarray(Oi, dtype=np.int64)] = False
        x32 = X.astype(np.float32)
        Xq = np.zeros((T, K), dtype=np.int8)
        sx = np.zeros(T, dtype=np.float32)
        Z = np.zeros(T, dtype=np.int32)
        for i in range(T):
            v = x32[i, keep]
            if v.size == 0 or v.max() == v.min():
                continue
            a, b = np.float32(v.min()), np.float32(v.max())   # 0 not forced in
            d = np.float32(b - a)
            S = np.float32(np.float32(254) / d)
            z = int(O.rhaz(np.float32(a * S))) + 127
            t = ((x32[i] * S).astype(np.float32) - np.float32(z)).astype(np.float32)
            Xq[i] = np.where(keep, np.clip(O.rhaz(t), -127, 127), 0).astype(np.int8)
            sx[i] = np.float32(d / np.float32(2))
            Z[i] = z
        return Xq, sx, Z
    mp.setattr(O, "quantize_rows_zeropoint", bad)


MUTATIONS = [_m_round_half_even, _m_strict_threshold, _m_descending_outliers,
             _m_row_scale_unmasked, _m_outliers_not_zeroed, _m_drop_bias, _m_scale_127,
             _m_wo_no_scale, _m_untransposed_gemm, _m_weight_per_column, _m_outlier_sign,
             _m_zp_drop_offset, _m_zp_offset_over_all_columns, _m_zp_offset_sign,
             _m_zp_range_without_zero]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_planted_mistake_is_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutation.__name__}"


def test_planted_columns_are_the_outliers():
    """Under N(0,1) the chance of a natural |x| >= 6 is ~2e-9 per element, so
    on the unit-sigma workloads the outlier set is exactly the planted one."""
    for name in ("tiny", "6.7b", "13b", "13b-down", "13b-attn", "decode1", "decode8", "decode32"):
        d = make_inputs(name, with_weight=False)
        got = O.find_outliers(d["X"], d["threshold"])
        assert np.array_equal(got, np.sort(d["planted"])), name
    d = make_inputs("175b", with_weight=False)
    got = O.find_outliers(d["X"], d["threshold"])
    # sigma 1.5 puts the threshold at 4 sigma: ~23% of columns trip it naturally
    assert set(d["planted"].tolist()) <= set(got.tolist())
    p = 1 - (1 - math.erfc(4 / math.sqrt(2))) ** 4096
    assert abs(len(got) / 12288 - p) < 0.02
