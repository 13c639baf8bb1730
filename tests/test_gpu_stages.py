"""Bit-exact parity of each GPU stage with the CPU oracle.

Stages: weight quantization (CB, SCB), outlier detection (O, n_o, mask),
masked row quantization (sx, Xq, Xo), dequantized outlier weights (Wo), and
the int32 accumulators of the int8 product.  Shapes span several tiles and a
ragged tail; every input comes from the seeded generators in ``workloads``.
"""
import numpy as np
import pytest

import oracle.llm_int8 as O
from tests.gpu_util import dev, host, say
from workloads import make_random_case, make_weight

pytestmark = pytest.mark.gpu

SHAPES = [  # (T, K, N)
    (16, 64, 64), (300, 1024, 517), (257, 1000, 300), (5, 24, 7), (1, 8, 1), (3, 1, 2),
    (130, 4104, 260),
]


@pytest.fixture(scope="module")
def i8():
    from tests.conftest import ensure_built
    ensure_built()
    import int8_mixed_precision_detect_amd as m
    return m


def _weight_cases():
    rng = np.random.default_rng(5)
    for T, K, N in SHAPES:
        W = make_weight(rng, N, K, 0.02)
        if N > 2:
            W[1] = 0                               # all-zero row -> SCB 0, CB 0
            W[2, : min(K, 9)] = np.array([127, 0.5, -0.5, 2.5, -2.5, 1.5, -1.5, 0.25, -126.5],
                                         dtype=np.float16)[: min(K, 9)]
        yield (N, K), W


@pytest.mark.parametrize("case", list(range(len(SHAPES))))
def test_quantize_weight_bitexact(i8, case):
    (N, K), W = list(_weight_cases())[case]
    say("quantize_weight", N, K)
    CB, SCB = i8.quantize_weight(dev(W))
    CBo, SCBo = O.quantize_weight(W)
    assert np.array_equal(host(SCB).view(np.uint32), SCBo.view(np.uint32))
    assert np.array_equal(host(CB), CBo)


def _detect_cases():
    for s, (T, K, N) in enumerate(SHAPES):
        d = make_random_case(40 + s, T, K, N, n_planted=min(3, K), row_frac=0.3)
        yield d["X"], 6.0
    X = np.zeros((3, 70), dtype=np.float16)        # ties at the threshold
    X[0, 5] = 6.0
    X[1, 6] = np.float16(5.99609375)
    X[2, 69] = -6.0
    X[2, 33] = np.float16(6.00390625)
    yield X, 6.0
    d = make_random_case(60, 40, 96, 8)
    yield d["X"], float("inf")                      # no outliers
    yield d["X"], 1e-6                              # every non-zero column
    d = make_random_case(61, 2048, 512, 8, x_sigma=1.5)
    yield d["X"], 6.0                               # many natural outliers
    d = make_random_case(63, 24, 20000, 8, n_planted=9)
    X = d["X"].copy()
    X[5, 19999] = 7.0                               # outliers in mask words past 512
    X[7, 16400] = -9.0
    yield X, 6.0


N_DETECT_CASES = len(SHAPES) + 5


@pytest.mark.parametrize("case", list(range(N_DETECT_CASES)))
def test_find_outliers_bitexact(i8, case):
    X, thr = list(_detect_cases())[case]
    T, K = X.shape
    say("find_outliers", T, K, thr)
    Og, counts, mask = i8.find_outliers(dev(X), thr)
    Oo = O.find_outliers(X, thr)
    c = host(counts)
    assert c[0] == len(Oo) and c[1] == 0
    assert np.array_equal(host(Og)[: len(Oo)], Oo.astype(np.int32))
    want = np.zeros((K + 31) // 32, dtype=np.uint32)
    for k in Oo:
        want[k // 32] |= np.uint32(1) << np.uint32(k % 32)
    assert np.array_equal(host(mask).view(np.uint32), want)


def test_find_outliers_overflow(i8):
    d = make_random_case(62, 64, 256, 8, n_planted=10)
    X = d["X"]
    Oo = O.find_outliers(X, 6.0)
    assert len(Oo) == 10
    say("find_outliers overflow")
    Og, counts, _ = i8.find_outliers(dev(X), 6.0, max_outliers=4)
    c = host(counts)
    assert c[0] == 10 and c[1] == 1
    assert np.array_equal(host(Og)[:4], Oo[:4].astype(np.int32))


def _mask_of(Oo, K):
    m = np.zeros((K + 31) // 32, dtype=np.uint32)
    for k in Oo:
        m[k // 32] |= np.uint32(1) << np.uint32(k % 32)
    return m.view(np.int32)


@pytest.mark.parametrize("case", list(range(N_DETECT_CASES)))
def test_quantize_rows_bitexact(i8, case):
    X, thr = list(_detect_cases())[case]
    T, K = X.shape
    if case == 0:
        X = X.copy()
        X[1] = 0                                    # an all-zero row -> sx 0, codes 0
    Oo = O.find_outliers(X, thr)
    Xqo, sxo = O.quantize_rows(X, Oo)
    Xoo = X[:, Oo]
    n = len(Oo)
    say("quantize_rows", T, K, n)
    for source in ("oracle mask", "gpu mask"):
        if source == "gpu mask":
            _, _, mask = i8.find_outliers(dev(X), thr)
        else:
            mask = dev(_mask_of(Oo, K))
        Xq, sx, Xo = i8.quantize_rows(dev(X), mask, K)
        Xq, sx, Xo = host(Xq), host(sx), host(Xo)
        assert np.array_equal(sx.view(np.uint32), sxo.view(np.uint32))
        assert np.array_equal(Xq[:, :K], Xqo)
        assert np.all(Xq[:, K:] == 0)
        npad = ((n + 31) // 32) * 32
        assert np.array_equal(Xo[:, :n].view(np.uint16), Xoo.view(np.uint16))
        assert np.all(Xo[:, n:npad].view(np.uint16) == 0)


def test_quantize_rows_capped(i8):
    """max_outliers below n_o: only the first max_outliers outlier columns are gathered."""
    d = make_random_case(63, 40, 256, 8, n_planted=10)
    X = d["X"]
    Oo = O.find_outliers(X, 6.0)
    say("quantize_rows capped")
    Xq, sx, Xo = i8.quantize_rows(dev(X), dev(_mask_of(Oo, 256)), 4)
    Xqo, sxo = O.quantize_rows(X, Oo)
    assert np.array_equal(host(Xq)[:, :256], Xqo)
    assert np.array_equal(host(Xo)[:, :4].view(np.uint16), X[:, Oo[:4]].view(np.uint16))


@pytest.mark.parametrize("case", list(range(len(SHAPES) + 2)))
def test_outlier_weights_bitexact(i8, case):
    if case < len(SHAPES):
        (N, K), W = list(_weight_cases())[case]
        rng = np.random.default_rng(70 + case)
        n = int(rng.integers(0, K + 1))
    else:  # wide outlier sets, where CB rows are staged in LDS
        rng = np.random.default_rng(80 + case)
        N, K = 300, 2048 if case == len(SHAPES) else 12288
        W = make_weight(rng, N, K, 0.02)
        n = int(K * 0.23)
    Oo = np.sort(rng.choice(K, size=n, replace=False)).astype(np.int64)
    CBo, SCBo = O.quantize_weight(W)
    _, Woo = O.gather_outliers(np.zeros((1, K), np.float16), CBo, SCBo, Oo)
    say("outlier_weights", N, K, n)
    Wo = host(i8.outlier_weights(dev(CBo), dev(SCBo), dev(_mask_of(Oo, K)), K))
    npad = ((n + 31) // 32) * 32
    assert np.array_equal(Wo[:, :n].view(np.uint16), Woo.view(np.uint16))
    assert np.all(Wo[:, n:npad].view(np.uint16) == 0)


# Wide outlier sets (at least one column in 64): whole CB rows stream
# through LDS, two rows in flight, when K is a multiple of 16 up to 16384 and
# the set has at most 4096 columns; otherwise the gathers.  Cases: K not a
# multiple of the 4 KB row piece, the largest set and one past it, the
# largest K and one chunk past it, K not a multiple of 16, an odd number of
# channels in the last block of 16, the smallest wide set.
@pytest.mark.parametrize("N,K,n", [
    (37, 5136, 1300), (300, 8192, 4096), (300, 8192, 4097), (19, 16384, 2000),
    (40, 16400, 1000), (33, 1000, 200), (17, 4096, 64),
])
def test_outlier_weights_wide_sets(i8, N, K, n):
    rng = np.random.default_rng(N * 31 + K + n)
    W = make_weight(rng, N, K, 0.02)
    Oo = np.sort(rng.choice(K, size=n, replace=False)).astype(np.int64)
    CBo, SCBo = O.quantize_weight(W)
    _, Woo = O.gather_outliers(np.zeros((1, K), np.float16), CBo, SCBo, Oo)
    say("outlier_weights wide", N, K, n)
    Wo = host(i8.outlier_weights(dev(CBo), dev(SCBo), dev(_mask_of(Oo, K)), K))
    npad = ((n + 31) // 32) * 32
    assert np.array_equal(Wo[:, :n].view(np.uint16), Woo.view(np.uint16))
    assert np.all(Wo[:, n:npad].view(np.uint16) == 0)


GEMM_SHAPES = [(16, 64, 64), (300, 517, 1024), (257, 300, 1000), (1, 1, 1), (5, 7, 24),
               (513, 257, 2048), (64, 1024, 4160), (2, 3, 12288),
               # large enough for the 320-channel tile (2 full waves of
               # workgroups instead of 2.5), with a ragged last channel tile
               (2048, 20380, 320),
               # few tokens (the thin tiles): ragged channels, K not a
               # multiple of the 128-byte slice, both tile shapes (T <= 16
               # and T <= 32)
               (32, 1000, 4160), (17, 517, 1040), (1, 33, 16), (9, 4096, 12288), (4, 40, 0),
               # one to four tokens (the row-streaming kernel): ragged rows,
               # K past one 1 KB piece and not a multiple of it
               (1, 1000, 3000), (2, 9, 1024), (3, 64, 2064), (4, 17, 12288)]


@pytest.mark.parametrize("T,N,K", GEMM_SHAPES)
def test_gemm_s32_bitexact(i8, T, N, K):
    rng = np.random.default_rng(T * 7 + N * 3 + K)
    A = rng.integers(-127, 128, size=(T, K)).astype(np.int8)
    B = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    A[0, :] = 127
    B[0, :] = -127                                   # the largest-magnitude sums
    say("gemm_s32", T, N, K)
    C = host(i8.gemm_s32(dev(A), dev(B)))
    assert np.array_equal(C.astype(np.int64), O.int8_matmul(A, B))


def test_gemm_s32_padded_leading_dims(i8):
    rng = np.random.default_rng(3)
    T, N, K = 100, 200, 300
    A = rng.integers(-127, 128, size=(T, 320)).astype(np.int8)
    B = rng.integers(-127, 128, size=(N, 304)).astype(np.int8)
    say("gemm_s32 lda/ldb")
    C = host(i8.gemm_s32(dev(A), dev(B), K=K))
    assert np.array_equal(C.astype(np.int64), O.int8_matmul(A[:, :K], B[:, :K]))
