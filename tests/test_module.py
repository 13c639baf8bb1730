"""Host-side behaviour of the Int8Linear module (no GPU): the two state-dict
forms the pages' workflow goes through ("transformers への統合" section of
the Hugging Face summary: load an fp16 nn.Linear state dict, move to the
GPU, which quantizes), and that nothing computes on the CPU."""
import io

import pytest
import torch

from int8_mixed_precision_detect_amd import Int8Linear


def _fp16_state(n_in=64, n_out=32, bias=True, seed=0):
    g = torch.Generator().manual_seed(seed)
    lin = torch.nn.Linear(n_in, n_out, bias=bias)
    with torch.no_grad():
        lin.weight.copy_(torch.randn(n_out, n_in, generator=g) * 0.02)
        if bias:
            lin.bias.copy_(torch.randn(n_out, generator=g) * 0.01)
    return lin


def test_fp16_state_dict_loads_before_the_move():
    lin = _fp16_state()
    m = Int8Linear(64, 32, bias=True, has_fp16_weights=False)
    m.load_state_dict(lin.state_dict())
    assert m.CB is None and m.SCB is None  # quantized by the move to the GPU, not before
    assert torch.equal(m.weight, lin.weight.to(torch.float16))
    assert set(m.state_dict()) == {"weight", "bias"}


def test_int8_state_dict_loads_without_a_weight():
    CB = torch.randint(-127, 128, (32, 64), dtype=torch.int8)
    SCB = torch.rand(32) + 0.5
    bias = torch.randn(32).to(torch.float16)
    m = Int8Linear(64, 32, bias=True)
    m.load_state_dict({"CB": CB, "SCB": SCB, "bias": bias})
    assert m.weight is None
    assert torch.equal(m.CB, CB) and torch.equal(m.SCB, SCB) and torch.equal(m.bias, bias)
    sd = m.state_dict()
    assert set(sd) == {"CB", "SCB", "bias"}
    # persistence of the int8 form through a weights-only load
    buf = io.BytesIO()
    torch.save(sd, buf)
    buf.seek(0)
    back = torch.load(buf, weights_only=True)
    m2 = Int8Linear(64, 32, bias=True)
    m2.load_state_dict(back)
    assert torch.equal(m2.CB, CB) and torch.equal(m2.SCB, SCB)


def test_from_linear_and_repr():
    lin = _fp16_state(bias=False)
    m = Int8Linear.from_linear(lin, threshold=5.0)
    assert m.bias is None and m.threshold == 5.0
    assert "quantized=False" in repr(m)


def test_no_cpu_compute():
    m = Int8Linear(64, 32)
    with pytest.raises(RuntimeError):
        m(torch.zeros(4, 64, dtype=torch.float16))


def test_half_keeps_the_int8_form_dtypes():
    # .half() / .to(dtype) must not cast the scales (SCB stays fp32, CB int8)
    CB = torch.randint(-127, 128, (32, 64), dtype=torch.int8)
    SCB = torch.rand(32) * 3 + 0.1234567
    m = Int8Linear(64, 32, bias=True)
    m.load_state_dict({"CB": CB, "SCB": SCB, "bias": torch.zeros(32, dtype=torch.float16)})
    m.half()
    assert m.CB.dtype == torch.int8 and m.SCB.dtype == torch.float32
    assert torch.equal(m.SCB, SCB) and torch.equal(m.CB, CB)
    m.to(torch.float32)
    assert m.SCB.dtype == torch.float32 and torch.equal(m.SCB, SCB)


def test_int8_form_holds_less_than_the_fp16_weight():
    # what a quantized module keeps between calls: CB, SCB, bias (the
    # workspace of a call is shared by all modules of a device and stream)
    n_out, n_in = 320, 512
    m = Int8Linear(n_in, n_out, bias=True)
    m.load_state_dict({"CB": torch.zeros(n_out, n_in, dtype=torch.int8),
                       "SCB": torch.ones(n_out), "bias": torch.zeros(n_out, dtype=torch.float16)})
    held = sum(t.numel() * t.element_size() for t in list(m.parameters()) + list(m.buffers()))
    held += sum(v.numel() * v.element_size() for v in vars(m).values() if torch.is_tensor(v))
    assert held < 0.6 * (2 * n_out * n_in)
