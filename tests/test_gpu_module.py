"""Int8Linear on the GPU: the pages' workflow ("transformers への統合"
section of the Hugging Face summary) -- two 64x64 layers, an fp16 state
dict saved and loaded into the int8 modules, then the move to the GPU, which
quantizes -- and the persistence of the int8 form."""
import io

import numpy as np
import pytest
import torch

import oracle.llm_int8 as O
from tests.gpu_util import assert_y_close, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def i8():
    from tests.conftest import ensure_built
    ensure_built()
    import int8_mixed_precision_detect_amd as m
    return m


def _fp16_model(seed=0):
    torch.manual_seed(seed)
    return torch.nn.Sequential(torch.nn.Linear(64, 64), torch.nn.Linear(64, 64)).half()


def _input(T=16, seed=1):
    g = torch.Generator().manual_seed(seed)
    X = torch.randn(T, 64, generator=g)
    X[:, 3] = 9.0  # an outlier column
    return X.to(torch.float16)


def test_pages_workflow_and_persistence(i8):
    fp16 = _fp16_model()
    buf = io.BytesIO()
    torch.save(fp16.state_dict(), buf)
    buf.seek(0)
    int8 = torch.nn.Sequential(i8.Int8Linear(64, 64, has_fp16_weights=False),
                               i8.Int8Linear(64, 64, has_fp16_weights=False))
    int8.load_state_dict(torch.load(buf, weights_only=True))
    say("module: move to the GPU quantizes")
    int8 = int8.to("cuda")
    for layer, ref in zip(int8, fp16):
        assert layer.weight is None and layer.CB.dtype == torch.int8
        CBo, SCBo = O.quantize_weight(ref.weight.detach().numpy())
        assert np.array_equal(host(layer.CB), CBo)
        assert np.array_equal(host(layer.SCB).view(np.uint32), SCBo.view(np.uint32))
    X = _input()
    Y = int8(X.cuda())
    # against the oracle, layer by layer on the same inputs
    h = X.cuda()
    for layer, ref in zip(int8, fp16):
        out = layer(h)
        CBo, SCBo = O.quantize_weight(ref.weight.detach().numpy())
        assert_y_close(host(out), O.linear_forward(host(h), CBo, SCBo,
                                                   ref.bias.detach().numpy(), 6.0), "Int8Linear")
        h = out
    assert np.array_equal(host(h).view(np.uint16), host(Y).view(np.uint16))
    # the int8 form persists: saved, loaded into fresh modules, same output bits
    buf2 = io.BytesIO()
    torch.save(int8.state_dict(), buf2)
    buf2.seek(0)
    sd = torch.load(buf2, weights_only=True)
    assert not any(k.endswith("weight") for k in sd)
    again = torch.nn.Sequential(i8.Int8Linear(64, 64), i8.Int8Linear(64, 64))
    again.load_state_dict(sd)
    again = again.to("cuda")
    Y2 = again(X.cuda())
    assert np.array_equal(host(Y2).view(np.uint16), host(Y).view(np.uint16))


def test_fp16_weights_module_and_batched_input(i8):
    lin = torch.nn.Linear(64, 48).half()
    m = i8.Int8Linear.from_linear(lin, has_fp16_weights=True).to("cuda")
    assert m.weight is not None and m.CB is None
    X = torch.stack([_input(5, 2), _input(5, 3)])  # [2, 5, 64]
    say("module: fp16 weights, 3-D input")
    Y = m(X.cuda())
    assert tuple(Y.shape) == (2, 5, 48)
    Yo = O.linear_forward_fp16w(X.reshape(10, 64).numpy(), lin.weight.detach().numpy(),
                                lin.bias.detach().numpy(), 6.0)
    assert_y_close(host(Y).reshape(10, 48), Yo, "fp16-weight module")
    # the same layer in int8 form differs only through the outlier weight dims
    q = i8.Int8Linear.from_linear(lin).to("cuda")
    Yq = q(X.cuda())
    CBo, SCBo = O.quantize_weight(lin.weight.detach().numpy())
    assert_y_close(host(Yq).reshape(10, 48),
                   O.linear_forward(X.reshape(10, 64).numpy(), CBo, SCBo,
                                    lin.bias.detach().numpy(), 6.0), "int8-form module")


def test_modules_share_one_workspace_and_keep_scales_fp32(i8):
    # layers of different shapes (and one decode-sized call) take turns on
    # the stream's one workspace; after .half() the scales are still fp32
    torch.manual_seed(5)
    shapes = [(64, 96), (96, 40), (40, 64)]
    lins = [torch.nn.Linear(a, b).half() for a, b in shapes]
    mods = [i8.Int8Linear.from_linear(l).to("cuda").half() for l in lins]
    for m in mods:
        assert m.SCB.dtype == torch.float32 and m.CB.dtype == torch.int8
    for rnd, T in enumerate([16, 3, 40, 8, 1]):
        x = torch.randn(T, 64)
        x[:, 5] = 8.0
        h = x.to(torch.float16)
        for l, m in zip(lins, mods):
            say("module chain", rnd, T, l.in_features, l.out_features)
            y = m(h.cuda())
            CBo, SCBo = O.quantize_weight(l.weight.detach().numpy())
            yo = O.linear_forward(h.numpy(), CBo, SCBo, l.bias.detach().numpy(), 6.0)
            assert_y_close(host(y), yo, f"layer {l.in_features}x{l.out_features}, T={T}")
            h = torch.from_numpy(yo)
    ws = i8.shared_workspace(1, 1, 1)
    assert ws.numel() >= max(i8.workspace_size(40, b, a) for a, b in shapes)
    assert not any(torch.is_tensor(v) and v.numel() >= ws.numel() for m in mods
                   for v in vars(m).values())
