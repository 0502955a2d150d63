"""PagedAdamW on a QLoRALinear (needs an MI355X): three training steps (forward, backward, update on a side
stream) against the float64 AdamW oracle run on the same float32 gradients; state paged to pinned host memory and
kept on the device."""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import say, product

pytestmark = pytest.mark.gpu

layer = product("layer")
optim = product("optim")

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.mark.parametrize("paged,update", [(True, "device"), (False, "device"), (True, "host")])
def test_paged_adamw_trains_a_layer_like_the_oracle(paged, update):
    """update="host" runs the page's own placement: gradients copied to pinned host memory, the library's host
    AdamW, the bf16 parameters copied back."""
    say(f"PagedAdamW paged={paged} update={update}")
    torch.manual_seed(3)
    W = (torch.randn(272, 320) * 0.02).cuda()
    m = layer.QLoRALinear(W, r=16, alpha=32.0)
    with torch.no_grad():
        m.B.copy_((torch.randn(272, 16) * 0.02).to(torch.bfloat16))
    opt = optim.PagedAdamW(m.parameters(), lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                           weight_decay=HP["weight_decay"], paged=paged, update=update)
    assert all(st[1].is_pinned() == paged for st in opt.state)
    ref = [[p.detach().double().cpu().numpy().reshape(-1), np.zeros(p.numel()), np.zeros(p.numel())]
           for p in opt.params]
    gmax = [0.0] * len(opt.params)
    x = torch.randn(64, 320).to(torch.bfloat16).cuda()
    target = torch.randn(64, 272).cuda()
    for step in range(1, 4):
        opt.wait()
        opt.zero_grad()
        loss = ((m(x).float() - target) ** 2).mean()
        loss.backward()
        # the optimizer steps on the library's float32 gradients, kept beside autograd's bf16 ones
        for p in opt.params:
            assert p.grad_fp32.dtype == torch.float32
            assert torch.equal(p.grad_fp32.to(torch.bfloat16).view(torch.int16), p.grad.view(torch.int16))
        grads = [p.grad_fp32.detach().cpu().numpy().astype(np.float64).reshape(-1) for p in opt.params]
        opt.step()
        for k, (st, g) in enumerate(zip(ref, grads)):
            st[0], st[1], st[2] = oracle.adamw_step(st[0], st[1], st[2], g, step, **HP)
            gmax[k] = max(gmax[k], float(np.max(np.abs(g))))
    opt.wait()
    torch.cuda.synchronize()
    ulp = 2.0 ** -24
    for p, (master, mm, vv), (rp, rm, rv), gm in zip(opt.params, opt.state, ref, gmax):
        np.testing.assert_allclose(mm.cpu().numpy(), rm, rtol=1e-5, atol=16 * ulp * gm)
        np.testing.assert_allclose(vv.cpu().numpy(), rv, rtol=1e-5, atol=16 * ulp * gm ** 2)
        np.testing.assert_allclose(master.cpu().numpy(), rp, rtol=1e-6, atol=HP["lr"] * 1e-5)
        assert torch.equal(p.detach().view(torch.int16).reshape(-1).cpu(),
                           master.to(torch.bfloat16).view(torch.int16).cpu())
