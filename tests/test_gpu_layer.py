"""The autograd module over the C-ABI (needs an MI355X): gradients from torch.autograd through
QLoRALinear equal the oracle's dX, dA, dB, the frozen weight gets none, and the LoRA-FA mode (A
frozen) gives dX and dB without keeping the layer input."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Case, assert_close, bits_to_bf16, say

pytestmark = pytest.mark.gpu

layer = pytest.importorskip("bit_quantized_finetuning_amd.layer")


def _module(case, freeze_A=False):
    d = case.device_inputs()
    m = layer.QLoRALinear(d["W"], r=case.r, alpha=case.alpha, freeze_A=freeze_A)
    with torch.no_grad():
        m.A.copy_(d["A"])
        m.B.copy_(d["B"])
    return m, d


@pytest.mark.parametrize("T", [4, 300])
def test_autograd_matches_oracle(T):
    say(f"autograd T={T}")
    case = Case(272, 320, 64, T, cfg=120)
    m, d = _module(case)
    x = d["x"].clone().requires_grad_(True)
    h = m(x)
    (h.float() * d["dY"].float()).sum().backward()
    torch.cuda.synchronize()
    h_ref, _ = case.oracle_forward()
    dX_ref, dA_ref, dB_ref = case.oracle_backward()
    assert_close("h", h, h_ref)
    assert_close("dX", x.grad, dX_ref)
    assert_close("dA", m.A.grad, dA_ref)
    assert_close("dB", m.B.grad, dB_ref)
    assert not any(b.requires_grad for b in m.buffers())


def test_lora_fa_mode_keeps_no_input():
    say("autograd LoRA-FA")
    case = Case(272, 320, 64, 300, cfg=121)
    m, d = _module(case, freeze_A=True)
    x = d["x"].clone().requires_grad_(True)
    h = m(x)
    node = h.grad_fn
    while type(node).__name__ != "QLoRALinearFunctionBackward":
        node = node.next_functions[0][0]
    assert node.saved_tensors[0] is None  # no layer input kept
    (h.float() * d["dY"].float()).sum().backward()
    torch.cuda.synchronize()
    dX_ref, _, dB_ref = case.oracle_backward()
    assert m.A.grad is None
    assert_close("dX", x.grad, dX_ref)
    assert_close("dB", m.B.grad, dB_ref)


def test_new_module_is_the_base_layer_and_merges():
    """B = 0 at creation: the module's output is the adapter-free forward, and its merged weight is the
    plain restore."""
    say("module init / merge")
    case = Case(80, 320, 16, 16, cfg=122)
    d = case.device_inputs()
    m = layer.QLoRALinear(d["W"], r=16, alpha=16.0)
    h = m(d["x"])
    torch.cuda.synchronize()
    wb = case.oracle_quant()[4]
    assert_close("h", h, oracle.lora_forward(wb, case.x, None, None, 16.0, 0)[0])
    assert np.array_equal(m.merged_weight().float().cpu().numpy(), wb)
