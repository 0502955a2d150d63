"""The paged AdamW step on the GPU (needs an MI355X): state in pinned host memory or in device memory,
compared with the float64 oracle over several steps; the bf16 parameters the layer reads are the
rounded master copy; pageable host memory is refused without leaving an error behind.

(First page, the paged-optimizer entry of "메모리 회계": the adapters' Adam state lives in CPU
pinned memory.)"""

import numpy as np
import pytest
import torch

import oracle
from gpu_common import say, product

pytestmark = pytest.mark.gpu

q = product("qlora")

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _state(n, pinned, rs):
    p0 = (rs.standard_normal(n) * 0.02).astype(np.float32)
    mk = (lambda a: torch.from_numpy(a).pin_memory()) if pinned else (lambda a: torch.from_numpy(a).cuda())
    return p0, mk(p0.copy()), mk(np.zeros(n, np.float32)), mk(np.zeros(n, np.float32))


@pytest.mark.parametrize("pinned", [True, False])
@pytest.mark.parametrize("n", [1000003, 64 * 5120])
def test_adamw_matches_oracle(pinned, n):
    say(f"adamw n={n} pinned={pinned}")
    rs = np.random.default_rng([7, n])
    p0, master, m, v = _state(n, pinned, rs)
    param = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    pr, mr, vr = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    gmax = 0.0
    for step in range(1, 6):
        g = rs.standard_normal(n).astype(np.float32) * np.float32(1e-3)
        gmax = max(gmax, float(np.abs(g).max()))
        q.qlora_adamw_step(step, torch.from_numpy(g).cuda(), master, m, v, param, **HP)
        pr, mr, vr = oracle.adamw_step(pr, mr, vr, g.astype(np.float64), step, **HP)
    torch.cuda.synchronize()
    pg, mg, vg = (t.cpu().numpy().astype(np.float64) for t in (master, m, v))
    # float32 arithmetic: each step rounds a few terms no larger than |g| (m) or g^2 (v) by 2^-24;
    # where a sign-changing gradient drives m towards zero that absolute error is all that is left
    ulp = 2.0 ** -24
    np.testing.assert_allclose(mg, mr, rtol=1e-5, atol=16 * ulp * gmax)
    np.testing.assert_allclose(vg, vr, rtol=1e-5, atol=16 * ulp * gmax ** 2)
    np.testing.assert_allclose(pg, pr, rtol=1e-6, atol=HP["lr"] * 1e-5)
    assert torch.equal(param.view(torch.int16).cpu(), master.to(torch.bfloat16).view(torch.int16).cpu())


def test_adamw_refuses_pageable_host_memory():
    say("adamw pageable host memory")
    n = 1024
    g = torch.zeros(n, device="cuda")
    dev = [torch.zeros(n, device="cuda") for _ in range(3)]
    pageable = torch.zeros(n)  # not pinned
    # the binding refuses it before the call ...
    with pytest.raises(ValueError, match="pinned host memory"):
        q.qlora_adamw_step(1, g, pageable, dev[1], dev[2], **HP)
    # ... and so does the library, called through the C ABI directly
    import ctypes
    hp = q.AdamWHparams(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
    st = q.lib.qlora_adamw_step(ctypes.byref(hp), 1, n, ctypes.c_void_p(g.data_ptr()),
                                ctypes.c_void_p(pageable.data_ptr()), ctypes.c_void_p(dev[1].data_ptr()),
                                ctypes.c_void_p(dev[2].data_ptr()), None,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -8
    q.qlora_adamw_step(1, g, *dev, **HP)  # the refused call left no error behind
    torch.cuda.synchronize()
