"""Pins for the oracle's AdamW step (CPU only): closed forms the update rule implies, and an
independent implementation (torch.optim.AdamW in float64)."""

import numpy as np
import torch

import oracle

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _f32(x):
    return float(np.float32(x))


def test_first_step_closed_form():
    """From zero moments the bias corrections give m_hat = g and v_hat = g^2, so the first step is
    p (1 - lr wd) - lr g / (|g| + eps)."""
    rs = np.random.default_rng(1)
    p0, g = rs.standard_normal(1000), rs.standard_normal(1000)
    p, m, v = oracle.adamw_step(p0, np.zeros(1000), np.zeros(1000), g, 1, **HP)
    lr, wd, eps = _f32(HP["lr"]), _f32(HP["weight_decay"]), _f32(HP["eps"])
    np.testing.assert_allclose(p, p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, (1 - _f32(HP["beta1"])) * g, rtol=1e-12)
    np.testing.assert_allclose(v, (1 - _f32(HP["beta2"])) * g * g, rtol=1e-12)


def test_constant_gradient_gives_identical_steps():
    """With the same gradient every step, m_hat = g and v_hat = g^2 at every t: without decay each
    step moves p by exactly -lr g / (|g| + eps)."""
    rs = np.random.default_rng(2)
    g, p0 = rs.standard_normal(100), rs.standard_normal(100)
    hp = dict(HP, weight_decay=0.0)
    p, m, v = p0, np.zeros(100), np.zeros(100)
    for t in range(1, 31):
        p, m, v = oracle.adamw_step(p, m, v, g, t, **hp)
    lr, eps = _f32(hp["lr"]), _f32(hp["eps"])
    np.testing.assert_allclose(p, p0 - 30 * lr * g / (np.abs(g) + eps), rtol=1e-10, atol=1e-13)


def test_zero_gradient_is_pure_decay():
    p0 = np.linspace(-1, 1, 50)
    p, m, v = p0, np.zeros(50), np.zeros(50)
    for t in range(1, 6):
        p, m, v = oracle.adamw_step(p, m, v, np.zeros(50), t, **HP)
    np.testing.assert_allclose(p, p0 * (1 - _f32(HP["lr"]) * _f32(HP["weight_decay"])) ** 5, rtol=1e-13)
    assert not m.any() and not v.any()


def test_matches_torch_adamw_float64():
    """torch.optim.AdamW (decoupled decay applied before the moment update, no amsgrad), float64 on the
    CPU, from the same float32 hyperparameters, over several steps of random gradients."""
    rs = np.random.default_rng(3)
    p0 = rs.standard_normal(257)
    grads = [rs.standard_normal(257) for _ in range(7)]
    hp = {k: _f32(v) for k, v in HP.items()}
    t = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([t], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    p, m, v = p0, np.zeros(257), np.zeros(257)
    for step, g in enumerate(grads, start=1):
        t.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oracle.adamw_step(p, m, v, g, step, **hp)
    np.testing.assert_allclose(p, t.detach().numpy(), rtol=1e-12, atol=1e-15)
    st = opt.state[t]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12)
