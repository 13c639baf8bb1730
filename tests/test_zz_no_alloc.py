"""The allocation-free forward (int8_linear_forward_noalloc) against the
workspace forward (int8_linear_forward), both called through the C ABI.

Both run the same kernels, so with the same max_outliers Y must agree bit
for bit, and the status block must carry the outlier count the workspace
forward leaves in its workspace.  Calls follow each other on one stream,
each on a smaller problem than the last (the scratch array keeps the last
call's contents, and a smaller layout puts its mask where the larger one
kept other data).  The small case is also held against the oracle.
"""
import ctypes

import numpy as np
import pytest

import oracle.llm_int8 as O
from tests.gpu_util import assert_y_close, dev, host, say
from workloads import make_inputs, make_random_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def i8():
    from tests.conftest import ensure_built
    ensure_built()
    import int8_mixed_precision_detect_amd as m
    return m


def _p(t):
    return None if t is None else t.data_ptr()


def _workspace_forward(i8, L, Xd, CB, SCB, bd, thr, mo):
    import torch
    T, K = Xd.shape
    N = CB.shape[0]
    ws = i8.alloc_workspace(T, N, K, mo)
    Y = torch.empty((T, N), dtype=torch.float16, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    rc = L.int8_linear_forward(_p(Xd), T, K, _p(CB), _p(SCB), N, _p(bd), float(thr), _p(Y),
                               _p(ws), ws.numel(), mo, st)
    assert rc == 0, rc
    n = ctypes.c_int32(-1)
    assert L.int8_linear_status(_p(ws), ctypes.byref(n), st) in (0, 5)
    return host(Y), int(n.value)


def _noalloc_forward(L, Xd, CB, SCB, bd, thr, mo, Y, status):
    import torch
    T, K = Xd.shape
    N = CB.shape[0]
    st = torch.cuda.current_stream().cuda_stream
    return L.int8_linear_forward_noalloc(_p(Xd), T, K, _p(CB), _p(SCB), N, _p(bd), float(thr),
                                         _p(Y), mo, _p(status), st)


def _case(i8, L, X, W, bias, thr, mo, what, oracle=False):
    import torch
    T, K = X.shape
    N = W.shape[0]
    say("noalloc", what, T, K, N, "max_outliers", mo)
    Xd, Wd = dev(X), dev(W)
    CB, SCB = i8.quantize_weight(Wd)
    bd = None if bias is None else dev(bias)
    # outputs first, so the no-allocation call is made with everything in place
    Y = torch.full((T, N), float("nan"), dtype=torch.float16, device="cuda")
    status = torch.full((4,), -7, dtype=torch.int32, device="cuda")
    assert _noalloc_forward(L, Xd, CB, SCB, bd, thr, mo, Y, status) == 0
    Yn = host(Y)
    sn = host(status)
    Yw, nw = _workspace_forward(i8, L, Xd, CB, SCB, bd, thr, mo)
    assert int(sn[0]) == nw, (what, sn, nw)
    assert int(sn[1]) == (1 if nw > mo else 0)
    assert int(sn[2]) == 0 and int(sn[3]) == 0
    if nw <= mo:
        assert np.array_equal(Yn.view(np.uint16), Yw.view(np.uint16)), what
    if oracle:
        CBo, SCBo = O.quantize_weight(W)
        assert_y_close(Yn, O.linear_forward(X, CBo, SCBo, bias, thr), what)
    return nw


def test_noalloc_matches_workspace_forward_on_shrinking_calls(i8):
    from int8_mixed_precision_detect_amd._lib import lib
    L = lib()
    d = make_inputs("13b")
    # full 13B first-FF shape, then a ragged small case with a bias, then a
    # few-token case (the decode kernel path), then one token (steps 1-2 in
    # one workgroup's launch, counts written to the caller's status)
    n1 = _case(i8, L, d["X"], d["W"], d["bias"], d["threshold"], 256, "13b")
    assert n1 > 0
    c = make_random_case(11, 77, 1000, 300, n_planted=5)
    n2 = _case(i8, L, c["X"], c["W"], c["bias"], c["threshold"], 64, "ragged 77x1000x300",
               oracle=True)
    assert n2 >= 5
    c = make_random_case(12, 8, 512, 200, n_planted=3, bias=False)
    _case(i8, L, c["X"], c["W"], None, c["threshold"], 32, "decode 8x512x200", oracle=True)
    c = make_random_case(13, 20, 1024, 100, n_planted=3, bias=False)
    _case(i8, L, c["X"], c["W"], None, c["threshold"], 32, "few tokens 20x1024x100", oracle=True)
    c = make_random_case(15, 1, 2048, 130, n_planted=4, bias=True)
    n4 = _case(i8, L, c["X"], c["W"], c["bias"], c["threshold"], 32, "one token 1x2048x130",
               oracle=True)
    assert n4 >= 4


def test_noalloc_reports_overflow_and_rejects_oversize(i8):
    import torch
    from int8_mixed_precision_detect_amd._lib import lib
    L = lib()
    c = make_random_case(13, 40, 256, 96, n_planted=6)
    n = _case(i8, L, c["X"], c["W"], c["bias"], c["threshold"], 2, "overflow 40x256x96")
    assert n > 2
    # a layout larger than the scratch array is refused before any launch
    X = torch.zeros((2048, 5120), dtype=torch.float16, device="cuda")
    CB = torch.zeros((20480, 5120), dtype=torch.int8, device="cuda")
    SCB = torch.ones((20480,), dtype=torch.float32, device="cuda")
    Y = torch.empty((2048, 20480), dtype=torch.float16, device="cuda")
    assert L.int8_linear_workspace_size(2048, 20480, 5120, 5120) > i8.NOALLOC_SCRATCH_BYTES
    assert _noalloc_forward(L, X, CB, SCB, None, 6.0, 5120, Y, None) == 2
    # and the entry point still works afterwards
    c = make_random_case(14, 33, 128, 64, n_planted=2)
    _case(i8, L, c["X"], c["W"], c["bias"], c["threshold"], 16, "after refusal 33x128x64",
          oracle=True)
