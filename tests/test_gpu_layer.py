"""The autograd module over the C-ABI (needs an MI355X): gradients from torch.autograd through
QLoRALinear equal the oracle's dX, dA, dB, the frozen weight gets none, and the LoRA-FA mode (A
frozen) gives dX and dB without keeping the layer input."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Case, assert_close, bits_to_bf16, say, product

pytestmark = pytest.mark.gpu

layer = product("layer")


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


# ---------------------------------------------------------------------------
# layer driver: q/k/v as one call, gradient checkpointing, chained layers
# ---------------------------------------------------------------------------

def _fused_inputs(T, cfg, shapes=((256, 256), (64, 256), (64, 256)), r=8):
    """Seeded q/k/v-style weights sharing one input, adapters on the first and last (q and v)."""
    cases = [Case(d_out, d_in, r, T, cfg=cfg, proj=i) for i, (d_out, d_in) in enumerate(shapes)]
    x_case = cases[0]
    return cases, x_case


@pytest.mark.parametrize("T", [4, 300])
def test_fused_qkv_matches_separate_projections(T):
    """One fused call equals the three projections computed separately by the oracle: outputs per projection,
    dX summed over them, dA/dB of q and v; the stacked quantization is bit-identical to quantizing each
    projection alone (every projection holds whole 256-block groups here)."""
    say(f"fused q/k/v T={T}")
    cases, xc = _fused_inputs(T, cfg=123)
    Ws = [torch.from_numpy(c.W).cuda() for c in cases]
    m = layer.QLoRAFusedLinear(Ws, r=8, alpha=16.0, adapted=[True, False, True])
    with torch.no_grad():
        for k, c in enumerate((cases[0], cases[2])):
            m.A[k].copy_(bits_to_bf16(c.A_bits))
            m.B[k].copy_(bits_to_bf16(c.B_bits))
    torch.cuda.synchronize()
    # stacked quantization == separate quantization
    sep = [oracle.quantize(c.W) for c in cases]
    assert np.array_equal(m.codes.cpu().numpy(), np.concatenate([s[0] for s in sep]))
    assert np.array_equal(m.qscale.cpu().numpy(), np.concatenate([s[1] for s in sep]))
    assert np.array_equal(m.smax.cpu().numpy().view(np.uint32), np.concatenate([s[2] for s in sep]).view(np.uint32))

    x = bits_to_bf16(xc.x_bits).clone().requires_grad_(True)
    dYs = [torch.from_numpy(c.dY).to(torch.bfloat16).cuda() for c in cases]
    outs = m(x)
    loss = sum((o.float() * g.float()).sum() for o, g in zip(outs, dYs))
    loss.backward()
    torch.cuda.synchronize()
    dX_ref = 0.0
    for i, c in enumerate(cases):
        wb = c.oracle_quant()[4]
        ad = i != 1
        A = c.A if ad else None
        B = c.B if ad else None
        h_ref, _ = oracle.lora_forward(wb, xc.x, A, B, 16.0, 8 if ad else 0)
        assert_close(f"h[{i}]", outs[i], h_ref)
        dYi = dYs[i].float().cpu().numpy().astype(np.float64)
        dX_i, dA_i, dB_i = oracle.lora_backward(wb, xc.x, dYi, A, B, 16.0, 8 if ad else 0)
        dX_ref = dX_ref + dX_i
        if ad:
            k = 0 if i == 0 else 1
            assert_close(f"dA[{i}]", m.A[k].grad, dA_i)
            assert_close(f"dB[{i}]", m.B[k].grad, dB_i)
            # the float32 gradients kept for the optimizer: the stacked call's blocks of this adapter, of which
            # autograd's bf16 gradients are the rounding
            assert_close(f"dA32[{i}]", m.A[k].grad_fp32, dA_i)
            assert_close(f"dB32[{i}]", m.B[k].grad_fp32, dB_i)
            for p in (m.A[k], m.B[k]):
                assert p.grad_fp32.dtype == torch.float32 and p.grad_fp32.shape == p.shape
                assert torch.equal(p.grad_fp32.to(torch.bfloat16).view(torch.int16), p.grad.view(torch.int16))
    assert_close("dX", x.grad, dX_ref)


def test_checkpointed_module_recomputes_identically():
    """Under gradient checkpointing the forward (and so u) is recomputed in the backward; the kernels are
    deterministic, so every gradient is bit-identical to the plain run and nothing but the input is kept."""
    say("checkpointed module")
    from torch.utils.checkpoint import checkpoint
    case = Case(272, 320, 64, 300, cfg=124)
    m, d = _module(case)
    grads = []
    for ckpt in (False, True):
        m.zero_grad(set_to_none=True)
        x = d["x"].clone().requires_grad_(True)
        h = checkpoint(m, x, use_reentrant=False) if ckpt else m(x)
        (h.float() * d["dY"].float()).sum().backward()
        torch.cuda.synchronize()
        grads.append([x.grad.clone(), m.A.grad.clone(), m.B.grad.clone()])
    for a, b in zip(*grads):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_two_chained_layers_match_oracle():
    """x -> layer 1 (320 -> 256) -> layer 2 (256 -> 320): the second layer's input is the first's bf16 output,
    and dX of the second is the upstream gradient of the first."""
    say("chained layers")
    c1 = Case(256, 320, 16, 100, cfg=125, proj=0)
    c2 = Case(320, 256, 16, 100, cfg=125, proj=1)
    m1, d1 = _module(c1)
    m2, d2 = _module(c2)
    x = d1["x"].clone().requires_grad_(True)
    h1 = m1(x)
    h2 = m2(h1)
    (h2.float() * d2["dY"].float()).sum().backward()
    torch.cuda.synchronize()
    wb1, wb2 = c1.oracle_quant()[4], c2.oracle_quant()[4]
    h1_ref, _ = oracle.lora_forward(wb1, c1.x, c1.A, c1.B, 16.0, 16)
    assert_close("h1", h1, h1_ref)
    h1_bf = h1.detach().float().cpu().numpy().astype(np.float64)   # what layer 2 actually consumed
    h2_ref, _ = oracle.lora_forward(wb2, h1_bf, c2.A, c2.B, 16.0, 16)
    assert_close("h2", h2, h2_ref)
    dH1, dA2, dB2 = oracle.lora_backward(wb2, h1_bf, c2.dY, c2.A, c2.B, 16.0, 16)
    assert_close("dA2", m2.A.grad, dA2)
    assert_close("dB2", m2.B.grad, dB2)
    # layer 1 sees layer 2's dX rounded to bf16 (the library's dX dtype)
    dH1_bf = oracle.bf16_round_f64(dH1)
    dX1, dA1, dB1 = oracle.lora_backward(wb1, c1.x, dH1_bf, c1.A, c1.B, 16.0, 16)
    assert_close("dA1", m1.A.grad, dA1)
    assert_close("dB1", m1.B.grad, dB1)
    assert_close("dX1", x.grad, dX1)


@pytest.mark.parametrize("T", [16, 300])
def test_recompute_u_keeps_no_intermediate(T):
    """recompute_u: the layer keeps x but not u, the backward forms u again, and the gradients match the oracle
    (and the saved-u run within the same tolerance)."""
    say(f"recompute_u T={T}")
    case = Case(272, 320, 64, T, cfg=126)
    d = case.device_inputs()
    grads = {}
    for rec in (False, True):
        m = layer.QLoRALinear(d["W"], r=case.r, alpha=case.alpha, recompute_u=rec)
        with torch.no_grad():
            m.A.copy_(d["A"])
            m.B.copy_(d["B"])
        x = d["x"].clone().requires_grad_(True)
        h = m(x)
        node = h.grad_fn
        while type(node).__name__ != "QLoRALinearFunctionBackward":
            node = node.next_functions[0][0]
        saved = node.saved_tensors
        assert (saved[3] is None) == rec and saved[0] is not None
        (h.float() * d["dY"].float()).sum().backward()
        torch.cuda.synchronize()
        grads[rec] = (x.grad.clone(), m.A.grad.clone(), m.B.grad.clone())
    dX_ref, dA_ref, dB_ref = case.oracle_backward()
    for rec in (False, True):
        assert_close(f"dX rec={rec}", grads[rec][0], dX_ref)
        assert_close(f"dA rec={rec}", grads[rec][1], dA_ref)
        assert_close(f"dB rec={rec}", grads[rec][2], dB_ref)


def test_state_dict_round_trip_after_dtype_cast():
    """A dtype cast leaves the quantized buffers (float32 group maxima included) and the bf16 adapters as they
    are; state_dict then reloads into a fresh module bit for bit, and the reloaded module computes from the
    loaded buffers (its output equals the original's)."""
    say("state_dict after .to(bfloat16)")
    torch.manual_seed(5)
    W = (torch.randn(256, 320) * 0.02).cuda()
    m = layer.QLoRALinear(W, r=8, alpha=16.0)
    with torch.no_grad():
        m.B.copy_((torch.randn(256, 8) * 0.02).to(torch.bfloat16))
    smax0 = m.smax.clone()
    m.to(torch.bfloat16)
    m.half()
    assert m.smax.dtype == torch.float32 and torch.equal(m.smax.view(torch.int32), smax0.view(torch.int32))
    assert m.A.dtype == torch.bfloat16 and m.B.dtype == torch.bfloat16
    sd = m.state_dict()
    W2 = (torch.randn(256, 320) * 0.02).cuda()  # another weight: every buffer differs until loaded
    m2 = layer.QLoRALinear(W2, r=8, alpha=16.0)
    m2.load_state_dict(sd)
    for k in ("codes", "qscale", "smax", "A", "B"):
        a, b = getattr(m, k), getattr(m2, k)
        assert a.dtype == b.dtype and torch.equal(a.view(torch.uint8), b.view(torch.uint8)), k
    x = torch.randn(16, 320).to(torch.bfloat16).cuda()
    with torch.no_grad():
        assert torch.equal(m(x).view(torch.int16), m2(x).view(torch.int16))
