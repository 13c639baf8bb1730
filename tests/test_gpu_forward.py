"""End-to-end parity of int8_linear_forward with the CPU oracle.

Y must be within 2e-3 * max|Y| + 1 fp16 ulp of the oracle per element; the
intermediate results the forward leaves in its workspace (O, n_o, sx, Xq, Xo,
Wo) must match the oracle bit for bit.  Small shapes are checked in full;
the workloads at full size are checked on sampled rows and output channels
(detection still runs over all of X on both sides).
"""
import numpy as np
import pytest

import oracle.llm_int8 as O
from tests.gpu_util import assert_y_close, dev, host, say
from workloads import WORKLOADS, make_inputs, make_random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def i8():
    from tests.conftest import ensure_built
    ensure_built()
    import int8_mixed_precision_detect_amd as m
    return m


def _run(i8, X, W, bias, thr, max_outliers=None):
    import torch
    T, K = X.shape
    N = W.shape[0]
    Xd, Wd = dev(X), dev(W)
    CB, SCB = i8.quantize_weight(Wd)
    bd = None if bias is None else dev(bias)
    mo = K if max_outliers is None else max_outliers
    ws = i8.alloc_workspace(T, N, K, mo)
    Y = i8.linear_forward(Xd, CB, SCB, bd, thr, max_outliers=mo, workspace=ws)
    torch.cuda.synchronize()
    return Y, ws, CB, SCB


def _ws_views(i8, ws, T, N, K, mo):
    lay = i8.workspace_layout(T, N, K, mo)
    b = host(ws)
    cnt = b[lay["counts"]: lay["counts"] + 16].view(np.int32)
    n = int(cnt[0])
    nu = min(n, mo)
    Og = b[lay["outliers"]: lay["outliers"] + 4 * nu].view(np.int32)
    sx = b[lay["sx"]: lay["sx"] + 4 * T].view(np.float32)
    ldq, ldo = lay["ldq"], lay["ldo"]
    Xq = b[lay["xq"]: lay["xq"] + T * ldq].view(np.int8).reshape(T, ldq)
    Xo = b[lay["xo"]: lay["xo"] + T * ldo * 2].view(np.float16).reshape(T, ldo)
    Wo = b[lay["wo"]: lay["wo"] + N * ldo * 2].view(np.float16).reshape(N, ldo)
    return dict(counts=cnt, O=Og, sx=sx, Xq=Xq, Xo=Xo, Wo=Wo)


def _full_check(i8, X, W, bias, thr, what):
    T, K = X.shape
    N = W.shape[0]
    say("forward", what, T, K, N, thr)
    Y, ws, CB, SCB = _run(i8, X, W, bias, thr)
    CBo, SCBo = O.quantize_weight(W)
    Yo, st = O.linear_forward(X, CBo, SCBo, bias, thr, return_stages=True)
    err = assert_y_close(host(Y), Yo, what)
    v = _ws_views(i8, ws, T, N, K, K)
    n = len(st["O"])
    assert v["counts"][0] == n and v["counts"][1] == 0
    assert np.array_equal(v["O"], st["O"].astype(np.int32))
    assert np.array_equal(v["sx"].view(np.uint32), st["sx"].view(np.uint32))
    assert np.array_equal(v["Xq"][:, :K], st["Xq"])
    assert np.all(v["Xq"][:, K:] == 0)
    assert np.array_equal(v["Xo"][:, :n].view(np.uint16), st["Xo"].view(np.uint16))
    assert np.array_equal(v["Wo"][:, :n].view(np.uint16), st["Wo"].view(np.uint16))
    npad = ((n + 31) // 32) * 32
    assert np.all(v["Xo"][:, n:npad].view(np.uint16) == 0)
    assert np.all(v["Wo"][:, n:npad].view(np.uint16) == 0)
    code, nn = i8.linear_status(ws)
    assert code == 0 and nn == n
    return Y, Yo, err


def test_tiny_workload(i8):
    d = make_inputs("tiny")
    _, _, err = _full_check(i8, d["X"], d["W"], d["bias"], d["threshold"], "tiny")
    print("tiny max err", err)


RAGGED = [  # (T, K, N, planted, bias)
    (300, 1024, 517, 3, True), (257, 1000, 300, 2, False), (513, 2048, 777, 40, True),
    (1, 64, 1, 1, True), (2, 8, 3, 0, False), (600, 520, 1030, 5, True), (64, 4160, 256, 33, True),
    (33, 1, 5, 1, True),
]


@pytest.mark.parametrize("T,K,N,planted,bias", RAGGED)
def test_ragged_shapes(i8, T, K, N, planted, bias):
    d = make_random_case(T + 3 * K + 7 * N, T, K, N, n_planted=planted, row_frac=0.5, bias=bias)
    _full_check(i8, d["X"], d["W"], d["bias"], 6.0, f"ragged {T}x{K}x{N}")


def test_no_outliers_threshold_inf(i8):
    d = make_random_case(901, 200, 512, 300, n_planted=4)
    _, _, _ = _full_check(i8, d["X"], d["W"], d["bias"], float("inf"), "thr=inf")


def test_every_column_outlier(i8):
    d = make_random_case(902, 96, 256, 130)
    assert np.all(d["X"] != 0)
    _full_check(i8, d["X"], d["W"], d["bias"], 1e-6, "n_o=K")


def test_zero_rows_and_threshold_tie(i8):
    d = make_random_case(903, 70, 320, 90, n_planted=2)
    X, W = d["X"].copy(), d["W"].copy()
    X[3] = 0                       # all-zero activation row
    W[5] = 0                       # all-zero weight row
    X[10, 7] = 6.0                 # exactly the threshold: column 7 is an outlier
    X[:, 8] = np.float16(5.99609375)  # just below it: column 8 is not
    _full_check(i8, X, W, d["bias"], 6.0, "zero rows / tie")


@pytest.mark.parametrize("T", [1, 5, 8, 9])
@pytest.mark.parametrize("thr", [6.0, 6.1, 5.999, 1e-4, 3e-8, 65504.0, 65505.0, float("inf")])
def test_threshold_edges(i8, T, thr):
    # Values on both sides of the threshold, for thresholds that fp16 holds
    # exactly (6.0, 65504) and that it does not (6.1, 5.999, a subnormal
    # one, one below the smallest fp16 value, one above the largest, +inf);
    # T <= 8 takes steps 1-2 in one launch (an integer test on the fp16
    # bits), T = 9 the detection launch (an fp32 compare): the same outliers
    # as the oracle's fp32 test
    K, N = 1024, 48
    d = make_random_case(int(T * 1000 + 7), T, K, N, n_planted=0, bias=True)
    scale = min(1e-5, thr / 1e3)  # the base values stay far below the threshold
    X = (d["X"].astype(np.float64) * scale).astype(np.float16)
    t32 = np.float32(thr)
    h = np.float16(min(float(t32), 65504.0))
    up = np.nextafter(h, np.float16(np.inf)) if h < np.float16(65504.0) else h
    cands = [h, np.nextafter(h, np.float16(0)), up,
             np.float16(6.0), np.float16(65504.0), np.float16(1e-4), np.float16(6e-8)]
    cols = np.arange(0, K, K // (2 * len(cands)))[:2 * len(cands)]
    for q, v in enumerate(cands):
        if np.isfinite(v):
            X[(q % T), cols[2 * q]] = v
            X[((q + 1) % T), cols[2 * q + 1]] = -v
    want = O.find_outliers(X, thr)
    assert 0 < len(want) < 2 * len(cands) or (thr > 65504.0 and len(want) == 0)
    _full_check(i8, X, d["W"], d["bias"], thr, f"{T} tokens, threshold {thr}")


def test_wide_channel_tile(i8):
    # 2048 x 20380 outputs take the 320-channel tile configuration; the last
    # channel tile is ragged (220 of 320 rows)
    d = make_random_case(906, 2048, 256, 20380, n_planted=5, row_frac=0.3)
    _full_check(i8, d["X"], d["W"], d["bias"], 6.0, "320-channel tiles 2048x256x20380")


@pytest.mark.parametrize("T,K,N,planted", [(1, 1040, 70, 3), (5, 1040, 70, 40), (32, 2048, 1000, 6),
                                            (17, 12288, 300, 12)])
def test_few_tokens(i8, T, K, N, planted):
    # T <= 32 runs the few-token tiles, which pick the outlier weights out of
    # the CB bytes they stage; an outlier in the last, partial slice of K
    # exercises the K tail
    d = make_random_case(T * 11 + K + N, T, K, N, n_planted=planted, bias=True)
    X = d["X"].copy()
    X[0, K - 1] = 9.0
    _full_check(i8, X, d["W"], d["bias"], 6.0, f"few tokens {T}x{K}x{N}")


@pytest.mark.parametrize("T,n,seed", [(1, 63, 76), (9, 64, 181), (16, 65, 273), (32, 100, 516),
                                       (3, 128, 167), (20, 128, 389)])
def test_few_tokens_outlier_window(i8, T, n, seed):
    # the few-token tiles extract up to 128 outlier columns themselves; each
    # lane keeps the last 64 values of its Wo row in registers and stores
    # them after the K loop (and at every 64th column inside it), so n_o of
    # 63, 64, 65, 100 and 128 cover a partial window, a full one, one flush
    # plus a remainder and two flushes; K = 2064 ends in a 16-byte slice
    K, N = 2064, 200
    d = make_random_case(seed, T, K, N, n_planted=n - 1, bias=True)
    X = d["X"].copy()
    X[0, K - 1] = 9.0
    assert len(O.find_outliers(X, 6.0)) == n
    _full_check(i8, X, d["W"], d["bias"], 6.0, f"few tokens {T}x{K}x{N}, n_o={n}")


def test_few_tokens_wide_outlier_set(i8):
    # more outlier columns than the few-token tiles extract themselves (128):
    # they take Wo from the workspace, built by the step-2 kernel
    d = make_random_case(907, 16, 2048, 300, n_planted=0, bias=True)
    n = len(O.find_outliers(d["X"], 2.5))
    assert n > 128
    _full_check(i8, d["X"], d["W"], d["bias"], 2.5, "few tokens, wide set")


@pytest.mark.parametrize("T,K,N,thr", [(64, 2048, 200, 3.0), (48, 8192, 96, 2.0)])
def test_wide_outlier_sets(i8, T, K, N, thr):
    # ~16% and ~89% of the columns are outliers; the second set is larger
    # than the outlier list step 2 keeps in LDS, so it takes the path that
    # enumerates the mask instead
    d = make_random_case(T * 7 + K, T, K, N, n_planted=0, bias=True)
    _full_check(i8, d["X"], d["W"], d["bias"], thr, f"wide set {T}x{K}x{N} thr={thr}")


# One to four tokens: the row-streaming kernel (1 KB pieces of each weight
# row, dot products on the lanes).  Cases: the outlier weights picked out of
# the pieces (up to 128 columns), the fp16 pass over the workspace's Wo / Xo
# for wider sets, N not a multiple of the 8 rows a workgroup takes, K below,
# at and past one piece and not a multiple of it.
@pytest.mark.parametrize("T,K,N,planted,thr", [
    (1, 16, 37, 1, 6.0), (2, 1024, 64, 5, 6.0), (3, 1040, 70, 40, 6.0), (4, 3000, 90, 12, 6.0),
    (1, 4096, 17, 0, 2.0), (4, 2048, 33, 0, 2.0), (2, 4096, 8, 0, float("inf")),
])
def test_one_to_four_tokens(i8, T, K, N, planted, thr):
    d = make_random_case(T * 11 + K + N, T, K, N, n_planted=planted, bias=True)
    _full_check(i8, d["X"], d["W"], d["bias"], thr, f"row-streaming {T}x{K}x{N} thr={thr}")


@pytest.mark.parametrize("T,K,N,planted", [(1, 1040, 70, 40), (3, 2000, 45, 3), (4, 4096, 64, 12)])
def test_one_to_four_tokens_fp16w_and_zeropoint(i8, T, K, N, planted):
    # both layers build Wo in step 2: the row-streaming kernel's fp16 pass
    d = make_random_case(T * 13 + K + N, T, K, N, n_planted=planted, bias=True)
    _fp16w_check(i8, d["X"], d["W"], d["bias"], 6.0, f"fp16 weight {T}x{K}x{N}")
    _zp_check(i8, d["X"], d["W"], d["bias"], 6.0, f"zero-point {T}x{K}x{N}")


# One to eight tokens, absmax layer: by default one launch of one workgroup
# takes steps 1-2 for the rows (no mask, no detection launch) and the
# product takes the weights of every outlier set out of CB itself (sets
# wider than 128 columns too); the switch runs the detection and step-2
# launches instead.  Both leave the same bits in the workspace (Wo
# included), and the same Y for sets of up to 128 columns.  Cases: K of one
# chunk a lane, an outlier in the last column of a partial piece, K past one
# chunk round of the workgroup, the largest K its registers take and one
# past it (the other launches), no outliers, a set wider than 128 columns;
# one token, the row-streaming product (2-4 tokens) and the thin tiles (5-8).
ROW_PREP_CASES = [
    (16, 37, 1, 6.0), (1040, 70, 3, 6.0), (12304, 4099, 12, 6.0), (16384, 260, 40, 6.0),
    (16400, 33, 5, 6.0), (2048, 90, 0, 6.0), (4096, 300, 0, 2.0),
]


@pytest.mark.parametrize("T", [1, 3, 8])
@pytest.mark.parametrize("K,N,planted,thr", ROW_PREP_CASES)
def test_one_token_row_prep(i8, T, K, N, planted, thr):
    _row_prep_case(i8, T, K, N, planted, thr)


@pytest.mark.parametrize("T,K,N,planted,thr", [
    (2, 1040, 70, 3, 6.0), (4, 4096, 300, 0, 2.0), (5, 12304, 4099, 12, 6.0), (6, 2048, 90, 0, 6.0),
    (7, 4096, 300, 0, 2.0), (5, 16384, 260, 40, 6.0), (8, 4096, 33, 0, 1.0),
])
def test_few_tokens_row_prep(i8, T, K, N, planted, thr):
    _row_prep_case(i8, T, K, N, planted, thr)


def _row_prep_case(i8, T, K, N, planted, thr):
    d = make_random_case(K + 5 * N + planted + 1000 * (T - 1), T, K, N, n_planted=planted, bias=True)
    X = d["X"].copy()
    X[T - 1, K - 1] = 9.0 if planted else X[T - 1, K - 1]
    runs = {}
    try:
        for on in (True, False):
            i8.set_row_prep(on)
            Y, _, _ = _full_check(i8, X, d["W"], d["bias"], thr, f"{T} tokens {K}x{N} row_prep={on}")
            _, ws, _, _ = _run(i8, X, d["W"], d["bias"], thr)
            runs[on] = (host(Y), _ws_views(i8, ws, T, N, K, K))
    finally:
        i8.set_row_prep(True)
    (Y1, v1), (Y3, v3) = runs[True], runs[False]
    npad = ((int(v1["counts"][0]) + 31) // 32) * 32  # Xo / Wo columns written
    for key in ("counts", "O", "sx", "Xq", "Xo", "Wo"):
        a, b = v1[key], v3[key]
        if key in ("Xo", "Wo"):
            a, b = a[:, :npad], b[:, :npad]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), key
    if int(v1["counts"][0]) <= 128:
        assert np.array_equal(Y1.view(np.uint16), Y3.view(np.uint16))


@pytest.mark.parametrize("T", [1, 6])
def test_one_token_row_prep_overflow(i8, T):
    # more outlier columns than max_outliers: the first max_outliers take the
    # fp16 path, the rest are dropped, as with the other launches; the status
    # says so
    K, N, mo = 2048, 64, 40
    d = make_random_case(5151 + T, T, K, N, n_planted=0, bias=False)
    n = len(O.find_outliers(d["X"], 2.0))
    assert n > mo
    outs = {}
    try:
        for on in (True, False):
            i8.set_row_prep(on)
            Y, ws, _, _ = _run(i8, d["X"], d["W"], None, 2.0, max_outliers=mo)
            code, nn = i8.linear_status(ws)
            assert i8._lib.STATUS[code] == "I8MM_ERR_OUTLIER_OVERFLOW" and nn == n
            outs[on] = (host(Y), _ws_views(i8, ws, T, N, K, mo))
    finally:
        i8.set_row_prep(True)
    (Y1, v1), (Y3, v3) = outs[True], outs[False]
    npad = ((mo + 31) // 32) * 32
    for key in ("O", "sx", "Xq"):
        assert np.array_equal(v1[key].view(np.uint8), v3[key].view(np.uint8)), key
    for key in ("Xo", "Wo"):
        assert np.array_equal(v1[key][:, :npad].view(np.uint16), v3[key][:, :npad].view(np.uint16)), key
    assert np.array_equal(Y1.view(np.uint16), Y3.view(np.uint16))


@pytest.mark.parametrize("T", [1, 8])
def test_one_token_repeats_and_graph_replays(i8, T):
    # calls in a row on one workspace (shapes alternating), and a captured
    # graph replayed with other work in between, give the eager result
    # every time
    import torch
    K, N = 4096, 1000
    d = make_random_case(4242, T, K, N, n_planted=6, bias=True)
    d2 = make_random_case(4243, T, 2048, 64, n_planted=2, bias=False)
    Xd, Wd, bd = dev(d["X"]), dev(d["W"]), dev(d["bias"])
    X2, W2 = dev(d2["X"]), dev(d2["W"])
    CB, SCB = i8.quantize_weight(Wd)
    CB2, SCB2 = i8.quantize_weight(W2)
    ws = i8.alloc_workspace(T, N, K)
    say("few tokens: repeated calls", T)
    Yref = host(i8.linear_forward(Xd, CB, SCB, bd, 6.0, workspace=ws)).view(np.uint16)
    Y2ref = host(i8.linear_forward(X2, CB2, SCB2, None, 6.0, workspace=ws)).view(np.uint16)
    for _ in range(3):
        assert np.array_equal(host(i8.linear_forward(Xd, CB, SCB, bd, 6.0, workspace=ws)).view(np.uint16), Yref)
        assert np.array_equal(host(i8.linear_forward(X2, CB2, SCB2, None, 6.0, workspace=ws)).view(np.uint16), Y2ref)
    say("one token: graph replays")
    Y = torch.empty((T, N), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        i8.linear_forward(Xd, CB, SCB, bd, 6.0, workspace=ws, out=Y)  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        i8.linear_forward(Xd, CB, SCB, bd, 6.0, workspace=ws, out=Y)
    for r in range(4):
        Y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y).view(np.uint16), Yref), f"replay {r}"
        # eager work on the same workspace between replays
        assert np.array_equal(host(i8.linear_forward(X2, CB2, SCB2, None, 6.0, workspace=ws)).view(np.uint16), Y2ref)
    code, n = i8.linear_status(ws)
    assert code == 0


def test_k_zero_gives_bias(i8):
    import torch
    T, N = 5, 7
    bias = np.arange(N, dtype=np.float16)
    say("forward K=0")
    X = torch.empty((T, 0), dtype=torch.float16, device="cuda")
    CB = torch.empty((N, 0), dtype=torch.int8, device="cuda")
    SCB = torch.zeros(N, dtype=torch.float32, device="cuda")
    Y = i8.linear_forward(X, CB, SCB, dev(bias), 6.0)
    assert np.array_equal(host(Y), np.broadcast_to(bias, (T, N)))
    Y = i8.linear_forward(X, CB, SCB, None, 6.0)
    assert np.all(host(Y) == 0)


@pytest.mark.parametrize("T,K,N,planted", [(300, 4112, 700, 5), (513, 2048, 777, 40),
                                            (40, 1040, 300, 3), (257, 256, 64, 2)])
def test_split_k_is_bit_identical(i8, T, K, N, planted):
    # split K: each split's workgroups store int32 partial tiles, a second
    # launch adds them (exact) and runs the same epilogue, so Y and the
    # intermediates must not depend on the split.  K = 4112 ends in a partial
    # slice; K = 256 has two slices, so 3 and 4 splits clamp to 2.
    d = make_random_case(T + K + N, T, K, N, n_planted=planted, bias=True)
    outs = []
    try:
        for sp in (1, 2, 3, 4):
            i8.set_split_override(sp)
            lay = i8.workspace_layout(T, N, K)
            assert lay["splits"] == min(sp, -(-K // 128))
            Y, _, _ = _full_check(i8, d["X"], d["W"], d["bias"], 6.0,
                                     f"split K x{sp} {T}x{K}x{N}")
            outs.append(host(Y).view(np.uint16))
    finally:
        i8.set_split_override(0)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("T,K,N,planted", [(600, 4112, 1000, 5), (2048, 1024, 5000, 40),
                                            (257, 520, 700, 3)])
def test_tile_configs_are_bit_identical(i8, T, K, N, planted):
    # the four wide tiles (320, 256, 192 channels x 256 tokens, 320 x 128)
    # compute each
    # element with the same operations in the same order: Y is the same bits,
    # unsplit and with K split in two; every one within the oracle's bound.
    # Ragged channel and token tiles; K = 4112 ends in a partial slice.
    d = make_random_case(T * 3 + K + N, T, K, N, n_planted=planted, bias=True)
    outs = []
    try:
        for sp in (1, 2):
            i8.set_split_override(sp)
            for cfg in (0, 1, 2, 3):
                i8.set_tile_override(cfg)
                Y, _, _ = _full_check(i8, d["X"], d["W"], d["bias"], 6.0,
                                      f"tile {cfg} split {sp} {T}x{K}x{N}")
                outs.append(host(Y).view(np.uint16))
    finally:
        i8.set_tile_override(-1)
        i8.set_split_override(0)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("T,K,N", [(600, 1024, 1000), (40, 256, 64)])
def test_bias_at_an_unaligned_address(i8, T, K, N):
    # a bias view one element into a buffer (2-byte but not 8-byte aligned):
    # the wide tiles then read it element by element; Y must be the same bits
    # as with an aligned copy of the same values
    import torch
    d = make_random_case(T + K + N + 5, T, K, N, n_planted=3, bias=True)
    Xd = dev(d["X"])
    CB, SCB = i8.quantize_weight(dev(d["W"]))
    ws = i8.alloc_workspace(T, N, K)
    b_aligned = dev(d["bias"])
    buf = torch.zeros(N + 1, dtype=torch.float16, device="cuda")
    buf[1:] = b_aligned
    b_off = buf[1:]
    assert b_off.data_ptr() % 8 != 0
    say("forward unaligned bias", T, K, N)
    Y1 = host(i8.linear_forward(Xd, CB, SCB, b_aligned, 6.0, workspace=ws)).view(np.uint16)
    Y2 = host(i8.linear_forward(Xd, CB, SCB, b_off, 6.0, workspace=ws)).view(np.uint16)
    assert np.array_equal(Y1, Y2)
    CBo, SCBo = O.quantize_weight(d["W"])
    Yo = O.linear_forward(d["X"], CBo, SCBo, d["bias"], 6.0)
    assert_y_close(Y2.view(np.float16), Yo, "unaligned bias")


def test_down_projection_plans_a_split(i8):
    # 13B down projection: 128 output tiles for 256 compute units
    lay = i8.workspace_layout(2048, 5120, 20480)
    assert lay["splits"] == 2


def _fp16w_check(i8, X, W, bias, thr, what):
    import torch
    T, K = X.shape
    N = W.shape[0]
    say("forward fp16 weight", what, T, K, N, thr)
    Yo, st = O.linear_forward_fp16w(X, W, bias, thr, return_stages=True)
    ws = i8.alloc_workspace(T, N, K)
    Y, CB, SCB = i8.linear_forward_fp16w(dev(X), dev(W), None if bias is None else dev(bias), thr,
                                         workspace=ws)
    torch.cuda.synchronize()
    err = assert_y_close(host(Y), Yo, what)
    assert np.array_equal(host(CB), st["CB"])
    assert np.array_equal(host(SCB).view(np.uint32), st["SCB"].view(np.uint32))
    v = _ws_views(i8, ws, T, N, K, K)
    n = len(st["O"])
    assert v["counts"][0] == n
    assert np.array_equal(v["O"], st["O"].astype(np.int32))
    assert np.array_equal(v["sx"].view(np.uint32), st["sx"].view(np.uint32))
    assert np.array_equal(v["Xq"][:, :K], st["Xq"])
    assert np.array_equal(v["Xo"][:, :n].view(np.uint16), st["Xo"].view(np.uint16))
    # the outlier weights are W's own fp16 values
    assert np.array_equal(v["Wo"][:, :n].view(np.uint16), st["Wo"].view(np.uint16))
    npad = ((n + 31) // 32) * 32
    assert np.all(v["Wo"][:, n:npad].view(np.uint16) == 0)
    return Y, err


@pytest.mark.parametrize("T,K,N,planted,thr", [
    (300, 1024, 517, 3, 6.0),     # wide tiles
    (5, 1040, 70, 40, 6.0),       # few tokens: Wo from W, fp16 tail instead of CB extraction
    (32, 2048, 1000, 6, 6.0),
    (17, 12288, 300, 12, 6.0),
    (16, 2048, 300, 0, 2.5),      # few tokens, more than 128 outlier columns
    (40, 1000, 130, 5, 6.0),      # K not a multiple of 16: the generic product
    (64, 256, 96, 0, 1e-6),       # every column an outlier
])
def test_fp16_weight_variant(i8, T, K, N, planted, thr):
    d = make_random_case(T * 5 + K + N + 11, T, K, N, n_planted=planted, bias=True)
    _fp16w_check(i8, d["X"], d["W"], d["bias"], thr, f"fp16 weight {T}x{K}x{N} thr={thr}")


def test_fp16_weight_variant_split_k(i8):
    d = make_random_case(77, 300, 4112, 700, n_planted=5, bias=True)
    try:
        i8.set_split_override(2)
        _fp16w_check(i8, d["X"], d["W"], d["bias"], 6.0, "fp16 weight, split K x2")
    finally:
        i8.set_split_override(0)


def test_fp16_weight_calls_and_graph_replays(i8):
    # the per-call weight quantization on a non-default stream: calls in a
    # row with another layer in between, and a captured graph replayed
    # several times (CB zeroed before each), give the eager result
    import torch
    T, K, N = 96, 2048, 700
    d = make_random_case(4711, T, K, N, n_planted=5, bias=True)
    d2 = make_random_case(4712, T, K, 300, n_planted=3, bias=False)
    Xd, Wd, bd = dev(d["X"]), dev(d["W"]), dev(d["bias"])
    X2, W2 = dev(d2["X"]), dev(d2["W"])
    s = torch.cuda.Stream()
    ws = i8.alloc_workspace(T, N, K)
    ws2 = i8.alloc_workspace(T, 300, K)
    Y = torch.empty((T, N), dtype=torch.float16, device="cuda")
    CB = torch.empty((N, K), dtype=torch.int8, device="cuda")
    SCB = torch.empty((N,), dtype=torch.float32, device="cuda")
    say("fp16 weight: eager calls on a side stream, then graph replays")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        i8.linear_forward_fp16w(Xd, Wd, bd, 6.0, workspace=ws, out=Y, CB=CB, SCB=SCB)
        Yref, CBref, SCBref = host(Y).view(np.uint16), host(CB), host(SCB).view(np.uint32)
        Y2ref = host(i8.linear_forward_fp16w(X2, W2, None, 6.0, workspace=ws2)[0]).view(np.uint16)
        for _ in range(2):
            CB.zero_()
            i8.linear_forward_fp16w(Xd, Wd, bd, 6.0, workspace=ws, out=Y, CB=CB, SCB=SCB)
            assert np.array_equal(host(Y).view(np.uint16), Yref)
            assert np.array_equal(host(CB), CBref)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    Yo = O.linear_forward_fp16w(d["X"], d["W"], d["bias"], 6.0)
    assert_y_close(Yref.view(np.float16), Yo, "fp16 weight, repeated calls")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        i8.linear_forward_fp16w(Xd, Wd, bd, 6.0, workspace=ws, out=Y, CB=CB, SCB=SCB)
    for r in range(4):
        Y.fill_(0)
        CB.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(Y).view(np.uint16), Yref), f"replay {r}"
        assert np.array_equal(host(CB), CBref) and np.array_equal(host(SCB).view(np.uint32), SCBref)
        assert np.array_equal(host(i8.linear_forward_fp16w(X2, W2, None, 6.0, workspace=ws2)[0]).view(np.uint16), Y2ref)


@pytest.mark.parametrize("N,K", [(7, 5), (300, 1024), (65, 1000), (1, 12288)])
def test_weight_rowsum_exact(i8, N, K):
    rng = np.random.default_rng(N + K)
    CB = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    say("weight_rowsum", N, K)
    got = host(i8.weight_rowsum(dev(CB)))
    assert np.array_equal(got.astype(np.int64), CB.astype(np.int64).sum(1))


def _zp_check(i8, X, W, bias, thr, what):
    import torch
    T, K = X.shape
    N = W.shape[0]
    say("forward zero-point", what, T, K, N, thr)
    CBo, SCBo = O.quantize_weight(W)
    Yo, st = O.linear_forward_zeropoint(X, CBo, SCBo, bias, thr, return_stages=True)
    CB, SCB = dev(CBo), dev(SCBo)
    rsum = i8.weight_rowsum(CB)
    ws = i8.alloc_workspace(T, N, K)
    Y = i8.linear_forward_zeropoint(dev(X), CB, SCB, rsum, None if bias is None else dev(bias),
                                    thr, workspace=ws)
    torch.cuda.synchronize()
    err = assert_y_close(host(Y), Yo, what)
    v = _ws_views(i8, ws, T, N, K, K)
    n = len(st["O"])
    assert v["counts"][0] == n
    assert np.array_equal(v["O"], st["O"].astype(np.int32))
    assert np.array_equal(v["sx"].view(np.uint32), st["sx"].view(np.uint32))
    assert np.array_equal(v["Xq"][:, :K], st["Xq"])
    lay = i8.workspace_layout(T, N, K)
    b = host(ws)
    zp = b[lay["zp"]: lay["zp"] + 4 * T].view(np.int32)
    assert np.array_equal(zp, st["Z"])
    assert np.array_equal(v["Xo"][:, :n].view(np.uint16), st["Xo"].view(np.uint16))
    assert np.array_equal(v["Wo"][:, :n].view(np.uint16), st["Wo"].view(np.uint16))
    if n:
        osum = b[lay["osum"]: lay["osum"] + 4 * N].view(np.int32)
        assert np.array_equal(osum.astype(np.int64), CBo[:, st["O"]].astype(np.int64).sum(1))
    return err


@pytest.mark.parametrize("T,K,N,planted,thr,relu", [
    (300, 1024, 517, 3, 6.0, False),   # wide tiles
    (300, 1024, 517, 3, 6.0, True),    # one-signed rows: Z = 127
    (5, 1040, 70, 40, 6.0, True),      # few tokens (Wo from step 2, fp16 tail)
    (17, 12288, 300, 12, 6.0, False),
    (32, 2048, 1000, 6, 6.0, True),
    (16, 2048, 300, 0, 2.5, False),    # few tokens, > 128 outlier columns
    (40, 1000, 130, 5, 6.0, True),     # K not a multiple of 16: the generic product
    (64, 256, 96, 0, 1e-6, False),     # every column an outlier
    (2048, 512, 640, 4, 6.0, True),    # several waves of wide tiles
])
def test_zero_point_variant(i8, T, K, N, planted, thr, relu):
    d = make_random_case(T * 3 + K + N + 29, T, K, N, n_planted=planted, bias=True)
    X = d["X"].copy()
    if relu:
        X = np.abs(X)
        X[1] = 0                     # an all-zero row: S = Z = sx = 0
    _zp_check(i8, X, d["W"], d["bias"], thr, f"zero-point {T}x{K}x{N} thr={thr} relu={relu}")


def test_zero_point_variant_split_k(i8):
    d = make_random_case(78, 300, 4112, 700, n_planted=5, bias=True)
    try:
        i8.set_split_override(2)
        assert i8.workspace_layout(300, 700, 4112)["splits"] == 2
        _zp_check(i8, np.abs(d["X"]), d["W"], d["bias"], 6.0, "zero-point, split K x2")
    finally:
        i8.set_split_override(0)


def test_outlier_overflow_is_reported(i8):
    d = make_random_case(904, 64, 256, 64, n_planted=10)
    say("forward overflow")
    Y, ws, _, _ = _run(i8, d["X"], d["W"], d["bias"], 6.0, max_outliers=4)
    code, n = i8.linear_status(ws)
    assert code == 5 and n == 10


def test_deterministic(i8):
    d = make_random_case(905, 513, 2048, 700, n_planted=7)
    say("forward determinism")
    Y1, _, _, _ = _run(i8, d["X"], d["W"], d["bias"], 6.0)
    Y2, _, _, _ = _run(i8, d["X"], d["W"], d["bias"], 6.0)
    assert np.array_equal(host(Y1).view(np.uint16), host(Y2).view(np.uint16))


# ---------------------------------------------------------------------------
# full-size workloads, sampled
# ---------------------------------------------------------------------------

def _sampled_check(i8, name, n_rows=48, n_cols=384, cache={}):
    import torch
    wl = WORKLOADS[name]
    key = "decode" if name.startswith("decode") else name
    if key not in cache:
        cache.clear()
        dW = make_inputs(name)
        Wd = dev(dW["W"])
        CB, SCB = i8.quantize_weight(Wd)
        cache[key] = (dW["W"], CB, SCB)
    W, CB, SCB = cache[key]
    d = make_inputs(name, with_weight=False)
    X, bias, thr = d["X"], d["bias"], d["threshold"]
    T, K, N = wl.T, wl.K, wl.N
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(T, size=min(n_rows, T), replace=False))
    cols = np.sort(rng.choice(N, size=min(n_cols, N), replace=False))
    # CB/SCB on the sampled channels: bit-exact against the oracle
    CBo, SCBo = O.quantize_weight(W[cols])
    assert np.array_equal(host(CB[torch.from_numpy(cols).cuda()]), CBo)
    assert np.array_equal(host(SCB[torch.from_numpy(cols).cuda()]).view(np.uint32),
                          SCBo.view(np.uint32))
    say("forward full-size", name, T, K, N)
    ws = i8.alloc_workspace(T, N, K)
    Y = i8.linear_forward(dev(X), CB, SCB, None if bias is None else dev(bias), thr, workspace=ws)
    Ys = host(Y[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    Yo, Oo = O.linear_forward_sampled(X, CBo, SCBo, None if bias is None else bias[cols], thr, rows)
    err = assert_y_close(Ys, Yo, name)
    code, n = i8.linear_status(ws)
    assert code == 0 and n == len(Oo)
    v = _ws_views(i8, ws, T, N, K, K)
    assert np.array_equal(v["O"], Oo.astype(np.int32))
    Xqo, sxo = O.quantize_rows(X[rows], Oo)
    assert np.array_equal(v["sx"][rows].view(np.uint32), sxo.view(np.uint32))
    assert np.array_equal(v["Xq"][rows, :K], Xqo)
    print(name, "n_o", n, "max err", err)
    return n


@pytest.mark.parametrize("name", ["6.7b", "13b", "13b-down", "13b-attn", "175b", "decode1",
                                  "decode8", "decode32"])
def test_full_size_workload_sampled(i8, name):
    n = _sampled_check(i8, name)
    if name != "175b":
        assert n == WORKLOADS[name].n_planted


@pytest.mark.parametrize("name", ["6.7b", "13b", "13b-down", "13b-attn", "decode1", "decode8",
                                  "decode32", "175b-n8", "175b"])
def test_full_size_workload_every_output(i8, name):
    """All of Y at the workloads' full sizes against the oracle, over output
    channel blocks (the oracle sees every row and all of X for detection);
    CB / SCB, counts, O, sx, Xq, Xo and Wo bit for bit."""
    import torch
    wl = WORKLOADS[name]
    T, K, N = wl.T, wl.K, wl.N
    d = make_inputs(name)
    X, W, bias, thr = d["X"], d["W"], d["bias"], d["threshold"]
    say("forward full-size, every output", name, T, K, N)
    Wd = dev(W)
    CB, SCB = i8.quantize_weight(Wd)
    del Wd
    ws = i8.alloc_workspace(T, N, K)
    Y = i8.linear_forward(dev(X), CB, SCB, None if bias is None else dev(bias), thr, workspace=ws)
    Yh, CBh, SCBh = host(Y), host(CB), host(SCB)
    del Y, CB, SCB
    Oo = O.find_outliers(X, thr)
    v = _ws_views(i8, ws, T, N, K, K)
    n = len(Oo)
    assert v["counts"][0] == n and v["counts"][1] == 0
    assert np.array_equal(v["O"], Oo.astype(np.int32))
    Xqo, sxo = O.quantize_rows(X, Oo)
    assert np.array_equal(v["sx"].view(np.uint32), sxo.view(np.uint32))
    assert np.array_equal(v["Xq"][:, :K], Xqo)
    assert np.array_equal(v["Xo"][:, :n].view(np.uint16), X[:, Oo].view(np.uint16))
    rows = np.arange(T)
    worst = 0.0
    step = 8192
    for c0 in range(0, N, step):
        c1 = min(N, c0 + step)
        CBo, SCBo = O.quantize_weight(W[c0:c1])
        assert np.array_equal(CBh[c0:c1], CBo), (name, c0)
        assert np.array_equal(SCBh[c0:c1].view(np.uint32), SCBo.view(np.uint32)), (name, c0)
        _, Wo = O.gather_outliers(X[:1], CBo, SCBo, Oo)
        assert np.array_equal(v["Wo"][c0:c1, :n].view(np.uint16), Wo.view(np.uint16)), (name, c0)
        Yo, _ = O.linear_forward_sampled(X, CBo, SCBo, None if bias is None else bias[c0:c1], thr,
                                         rows, O=Oo)
        worst = max(worst, assert_y_close(Yh[:, c0:c1], Yo, f"{name} channels {c0}:{c1}"))
    print(name, "n_o", n, "max err", worst)


@pytest.mark.parametrize("layer,name", [("fp16w", "13b"), ("zeropoint", "13b"),
                                        ("zeropoint", "decode1"), ("fp16w", "decode8")])
def test_full_size_layer_variants(i8, layer, name):
    """The fp16-weight and zero-point layers at full workload sizes (the 13B
    first-FF shape and the 175B-width decode shapes they are timed on): every
    output against the oracle, and their stage values (CB, SCB, O, sx, Xq,
    Xo, Wo; Z and the outlier code sums) bit for bit."""
    d = make_inputs(name)
    if layer == "fp16w":
        _fp16w_check(i8, d["X"], d["W"], d["bias"], d["threshold"], f"{name} fp16-weight layer")
    else:
        _zp_check(i8, d["X"], d["W"], d["bias"], d["threshold"], f"{name} zero-point layer")


@pytest.mark.parametrize("T", [8, 300])
def test_weight_above_2gib(i8, T):
    # an int8 weight of 65600 x 32768 (2.15e9 bytes, more than 2^31): the
    # tiled product addresses each tile's rows from the tile's own base, so
    # channels past byte 2^31 (j >= 65536) are checked with the rest
    import torch
    N, K = 65600, 32768
    g = torch.Generator(device="cuda").manual_seed(77)
    CB = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    SCB = torch.rand(N, device="cuda", generator=g) * 0.5 + 0.01
    rng = np.random.default_rng(T)
    X = rng.standard_normal((T, K)).astype(np.float16)
    X[:, [5, 20000, 32767]] = np.float16(9.0)
    rows = np.sort(rng.choice(T, size=min(T, 24), replace=False))
    cols = np.concatenate([np.sort(rng.choice(65536, size=160, replace=False)),
                           np.arange(65536 - 8, N)])
    say("forward above 2 GiB", T, K, N)
    Y = i8.linear_forward(dev(X), CB, SCB, None, 6.0)
    ci = torch.from_numpy(cols).cuda()
    Ys = host(Y[torch.from_numpy(rows).cuda()][:, ci])
    Yo, Oo = O.linear_forward_sampled(X, host(CB[ci]), host(SCB[ci]), None, 6.0, rows)
    assert list(Oo) == [5, 20000, 32767]
    assert_y_close(Ys, Yo, "above 2 GiB")
