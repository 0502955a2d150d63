"""GPU parity of the absmax-only storage (4.5 bits per weight, no double quantization).

With qscale = NULL every entry point reads one float32 scale per 64-weight block
(the variant the first page prices at 4.5 bits per parameter, section "메모리 회계",
before double quantization takes it to 4.13). Bit-exact: codes (the same as with
double quantization), block scales, float32 and bf16 restores. Within tolerance
(gpu_common): h, u, dX, dA, dB, against the oracle run on the absmax restore.
Shapes cover the skinny kernel's word-wise scale-code path (blocks per row a
multiple of 4) and its byte-wise one (80 x 320: 5 blocks per row), the GEMMs'
ragged row and K tiles, and the merge.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import Case, assert_close, assert_within_one_bf16_ulp, merge_float32_slack, say, product

pytestmark = pytest.mark.gpu

q = product("qlora")
layer = product("layer")


class AbsmaxCase(Case):
    def oracle_quant(self):
        if self._q is None:
            codes, s = oracle.quantize_absmax(self.W)
            w32, wb = oracle.dequantize_absmax(codes, s, self.d_out, self.d_in)
            self._q = (codes, None, s, w32, wb)
        return self._q


def _quantize_and_compare(case):
    d = case.device_inputs()
    w = q.qlora_quantize(d["W"], double_quant=False)
    torch.cuda.synchronize()
    codes, _, s, _, _ = case.oracle_quant()
    assert w.qscale is None and w.smax.numel() == s.size
    assert np.array_equal(w.codes.cpu().numpy(), codes), "packed codes differ"
    assert np.array_equal(w.smax.cpu().numpy().view(np.uint32), s.view(np.uint32)), "block scales differ"
    return w, d


@pytest.mark.parametrize("d_out,d_in,wdtype", [(16, 64, "f32"), (80, 320, "f32"), (32, 5120, "bf16"),
                                               (1024, 1024, "f32")])
def test_absmax_quantize_and_restore_bit_exact(d_out, d_in, wdtype):
    say(f"absmax quantize/restore {d_out}x{d_in} {wdtype}")
    case = AbsmaxCase(d_out, d_in, 0, 1, cfg=130, wdtype=wdtype)
    w, _ = _quantize_and_compare(case)
    # the codes are those of the double-quant storage
    codes_dq = oracle.quantize(case.W)[0]
    assert np.array_equal(w.codes.cpu().numpy(), codes_dq)
    w32 = q.qlora_dequantize(w, torch.float32)
    wbf = q.qlora_dequantize(w, torch.bfloat16)
    torch.cuda.synchronize()
    _, _, _, r32, rb = case.oracle_quant()
    assert np.array_equal(w32.cpu().numpy().view(np.uint32), r32.view(np.uint32))
    assert np.array_equal(wbf.float().cpu().numpy(), rb)


@pytest.mark.parametrize("d_out,d_in,r", [(1024, 1024, 8), (80, 320, 16), (272, 5120, 64)])
@pytest.mark.parametrize("T", [1, 16, 40, 300])
def test_absmax_forward_parity(d_out, d_in, r, T):
    say(f"absmax forward {d_out}x{d_in} r={r} T={T}")
    case = AbsmaxCase(d_out, d_in, r, T, cfg=131)
    w, d = _quantize_and_compare(case)
    h, u = q.qlora_forward(w, d["x"], d["A"], d["B"], case.alpha, save_u=True)
    torch.cuda.synchronize()
    h_ref, u_ref = case.oracle_forward()
    assert_close("h", h, h_ref)
    assert_close("u", u, u_ref)


@pytest.mark.parametrize("d_out,d_in,r", [(80, 320, 16), (272, 5120, 64)])
@pytest.mark.parametrize("T", [16, 300])
def test_absmax_backward_parity(d_out, d_in, r, T):
    say(f"absmax backward {d_out}x{d_in} r={r} T={T}")
    case = AbsmaxCase(d_out, d_in, r, T, cfg=132)
    w, d = _quantize_and_compare(case)
    dX, dA, dB = q.qlora_backward(w, d["x"], d["dY"], d["A"], d["B"], case.alpha)
    torch.cuda.synchronize()
    dX_ref, dA_ref, dB_ref = case.oracle_backward()
    assert_close("dX", dX, dX_ref)
    assert_close("dA", dA, dA_ref)
    assert_close("dB", dB, dB_ref)


@pytest.mark.parametrize("d_out,d_in,r", [(80, 320, 16), (272, 5120, 64)])
def test_absmax_merge_parity(d_out, d_in, r):
    say(f"absmax merge {d_out}x{d_in} r={r}")
    case = AbsmaxCase(d_out, d_in, r, 1, cfg=133)
    w, d = _quantize_and_compare(case)
    out = q.qlora_merge(w, d["A"], d["B"], case.alpha)
    plain = q.qlora_merge(w, None, None, case.alpha)
    torch.cuda.synchronize()
    wb = case.oracle_quant()[4]
    assert_within_one_bf16_ulp("merged", out, oracle.lora_merge(wb, case.A, case.B, case.alpha, r),
                               merge_float32_slack(wb, case.A, case.B, case.alpha, r))
    assert np.array_equal(plain.float().cpu().numpy(), wb)


def test_absmax_module_forward_backward():
    say("absmax module")
    torch.manual_seed(0)
    W = (torch.randn(272, 320) * 0.02).cuda()
    m = layer.QLoRALinear(W, r=16, alpha=32.0, double_quant=False)
    with torch.no_grad():
        m.B.copy_((torch.randn(272, 16) * 0.02).to(torch.bfloat16))
    assert m.qscale is None and m.smax.numel() == 272 * 320 // 64
    x = torch.randn(2, 24, 320).to(torch.bfloat16).cuda().requires_grad_(True)
    h = m(x)
    h.float().square().sum().backward()
    torch.cuda.synchronize()
    codes, s = oracle.quantize_absmax(W.cpu().numpy())
    wb = oracle.dequantize_absmax(codes, s, 272, 320)[1]
    xr = x.detach().float().cpu().numpy().reshape(-1, 320)
    A = m.A.detach().float().cpu().numpy()
    B = m.B.detach().float().cpu().numpy()
    h_ref, _ = oracle.lora_forward(wb, xr, A, B, 32.0, 16)
    assert_close("h", h.reshape(-1, 272), h_ref)
    dY = 2.0 * h.detach().float().cpu().numpy().reshape(-1, 272)
    dX_ref, dA_ref, dB_ref = oracle.lora_backward(wb, xr, dY, A, B, 32.0, 16)
    assert_close("dX", x.grad.reshape(-1, 320), dX_ref)
    assert_close("dA", m.A.grad, dA_ref)
    assert_close("dB", m.B.grad, dB_ref)
