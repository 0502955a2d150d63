"""The host-CPU AdamW step (qlora_adamw_step_host; no GPU needed): the page's own placement of the paged
optimizer's update (first page, the paged-optimizer entry of "메모리 회계": the CPU updates the Adam state kept in
CPU memory while the GPU goes on). Checked against the float64 oracle over several steps, with the same
tolerances as the GPU kernel's test; the result does not depend on how many worker threads split the elements;
the bf16 parameters are the rounded master copy; bad arguments are refused without touching the state."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_finetuning_amd import build as _build

import os

if not os.path.exists(_build.LIB):  # hipcc cross-compiles for gfx950 without a GPU
    _build.build()
from bit_quantized_finetuning_amd import qlora as q  # noqa: E402

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _run(n, threads, steps=5, seed=7):
    rs = np.random.default_rng([seed, n])
    p0 = (rs.standard_normal(n) * 0.02).astype(np.float32)
    master, m, v = torch.from_numpy(p0.copy()), torch.zeros(n), torch.zeros(n)
    param = torch.empty(n, dtype=torch.bfloat16)
    pr, mr, vr = p0.astype(np.float64), np.zeros(n), np.zeros(n)
    gmax = 0.0
    for step in range(1, steps + 1):
        g = rs.standard_normal(n).astype(np.float32) * np.float32(1e-3)
        if step == 3:
            g[::7] = -g[::7]  # sign changes drive some moments towards zero
        gmax = max(gmax, float(np.abs(g).max()))
        q.qlora_adamw_step_host(step, torch.from_numpy(g), master, m, v, param, threads=threads, **HP)
        pr, mr, vr = oracle.adamw_step(pr, mr, vr, g.astype(np.float64), step, **HP)
    return master, m, v, param, (pr, mr, vr), gmax


@pytest.mark.parametrize("n", [1, 1000, 1000003])
def test_host_adamw_matches_oracle(n):
    master, m, v, param, (pr, mr, vr), gmax = _run(n, threads=0)
    ulp = 2.0 ** -24
    np.testing.assert_allclose(m.numpy().astype(np.float64), mr, rtol=1e-5, atol=16 * ulp * gmax)
    np.testing.assert_allclose(v.numpy().astype(np.float64), vr, rtol=1e-5, atol=16 * ulp * gmax ** 2)
    np.testing.assert_allclose(master.numpy().astype(np.float64), pr, rtol=1e-6, atol=HP["lr"] * 1e-5)
    # the bf16 parameters are torch's own round-to-nearest-even of the float32 master copy
    assert torch.equal(param.view(torch.int16), master.to(torch.bfloat16).view(torch.int16))


def test_host_adamw_independent_of_thread_count():
    a = _run(1000003, threads=1)
    b = _run(1000003, threads=0)
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16),
                           y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16))


def test_host_adamw_bf16_rounding_of_special_values():
    """Ties round to even, overflow goes to infinity, a NaN stays a NaN (the master copy is written as is)."""
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, 3.4e38, -0.0],
                    dtype=np.float32)
    n = vals.size
    # lr = 0 and wd = 0 leave the master copy unchanged: the step only writes bf16(master)
    master = torch.from_numpy(vals.copy())
    param = torch.empty(n, dtype=torch.bfloat16)
    q.qlora_adamw_step_host(1, torch.zeros(n), master, torch.zeros(n), torch.zeros(n), param, lr=0.0,
                            weight_decay=0.0)
    assert torch.equal(master, torch.from_numpy(vals))
    assert torch.equal(param.view(torch.int16), torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16))
    nan = torch.tensor([float("nan")] * 4)
    pn = torch.empty(4, dtype=torch.bfloat16)
    q.qlora_adamw_step_host(1, torch.zeros(4), nan.clone(), torch.zeros(4), torch.zeros(4), pn, lr=0.0)
    assert torch.isnan(pn.float()).all()


def test_host_adamw_refuses_bad_arguments():
    n = 64
    g, master, m, v = torch.zeros(n), torch.ones(n), torch.zeros(n), torch.zeros(n)
    hp = q.AdamWHparams(HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"])
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    assert q.lib.qlora_adamw_step_host(ctypes.byref(hp), 0, n, p(g), p(master), p(m), p(v), None, 0) == -9   # step
    assert q.lib.qlora_adamw_step_host(ctypes.byref(hp), 1, -1, p(g), p(master), p(m), p(v), None, 0) == -2  # n
    assert q.lib.qlora_adamw_step_host(ctypes.byref(hp), 1, n, None, p(master), p(m), p(v), None, 0) == -1   # NULL
    bad = q.AdamWHparams(HP["lr"], 1.0, HP["beta2"], HP["eps"], HP["weight_decay"])
    assert q.lib.qlora_adamw_step_host(ctypes.byref(bad), 1, n, p(g), p(master), p(m), p(v), None, 0) == -9
    assert torch.equal(master, torch.ones(n)) and torch.equal(m, torch.zeros(n))  # nothing was written
    with pytest.raises(ValueError, match="same number of elements"):
        q.qlora_adamw_step_host(1, g, master, m, torch.zeros(n + 1))
    with pytest.raises(TypeError):
        q.qlora_adamw_step_host(1, g.double(), master, m, v)
