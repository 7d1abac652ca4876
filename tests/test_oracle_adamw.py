"""Pins of the oracle's AdamW step for the adapter matrices.

The pages say the adapters keep ordinary AdamW state (katajob, "What stays in
full precision") of about 8 bytes per trainable parameter (pranaymahendrakar,
Developer level, "The walkthrough", which also uses lr = 2e-4).  The update is
pinned against torch.optim.AdamW run in float64 on the CPU (an independent
implementation of the same published algorithm) and against closed forms.
"""
import numpy as np
import pytest
import torch


def _torch_adamw(theta0, grads, lr, b1, b2, eps, wd):
    p = torch.nn.Parameter(torch.tensor(theta0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    for g in grads:
        p.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    return p.detach().numpy().copy(), st["exp_avg"].numpy().copy(), st["exp_avg_sq"].numpy().copy()


@pytest.mark.parametrize("lr,b1,b2,eps,wd", [(2e-4, 0.9, 0.999, 1e-8, 0.0), (1e-2, 0.9, 0.999, 1e-8, 0.01),
                                             (3e-3, 0.5, 0.9, 1e-6, 0.1), (1e-3, 0.0, 0.0, 1e-8, 0.05)])
def test_matches_torch_adamw_float64(oracle, lr, b1, b2, eps, wd):
    rng = np.random.default_rng(5)
    n = 1000
    theta0 = rng.standard_normal(n) * 0.02
    grads = [rng.standard_normal(n) * s for s in (1e-3, 5e-3, 2e-2, 1e-4, 1e-3, 3e-1, 1e-6)]
    grads[3][:10] = 0.0
    want = _torch_adamw(theta0, grads, lr, b1, b2, eps, wd)
    th, m, v = theta0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        oracle.adamw_step(th, g, m, v, lr, b1, b2, eps, wd, t)
    np.testing.assert_allclose(th, want[0], rtol=1e-13, atol=1e-15 * np.abs(want[0]).max())
    np.testing.assert_allclose(m, want[1], rtol=1e-13, atol=1e-30)
    np.testing.assert_allclose(v, want[2], rtol=1e-13, atol=1e-30)


def test_first_step_closed_form(oracle):
    """At t = 1 the bias-corrected moments are g and g^2: theta - lr (wd theta + g / (|g| + eps))."""
    rng = np.random.default_rng(6)
    n = 257
    th0 = rng.standard_normal(n)
    g = rng.standard_normal(n) * 10.0 ** rng.integers(-6, 1, n)
    lr, eps, wd = 1e-3, 1e-8, 0.02
    th, m, v = th0.copy(), np.zeros(n), np.zeros(n)
    oracle.adamw_step(th, g, m, v, lr, 0.9, 0.999, eps, wd, 1)
    np.testing.assert_allclose(th, th0 - lr * (wd * th0 + g / (np.abs(g) + eps)), rtol=1e-14, atol=1e-19)
    np.testing.assert_allclose(m, 0.1 * g, rtol=4e-15)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=4e-15)  # 1 - 0.999 is 0.001 only to 1e-15


def test_zero_gradient_is_pure_decay(oracle):
    th0 = np.linspace(-1, 1, 64)
    th, m, v = th0.copy(), np.zeros(64), np.zeros(64)
    oracle.adamw_step(th, np.zeros(64), m, v, 0.5, 0.9, 0.999, 1e-8, 0.1, 3)
    np.testing.assert_allclose(th, th0 * (1 - 0.05), rtol=1e-15, atol=1e-17)
    assert np.all(m == 0) and np.all(v == 0)


def test_accepts_bf16_gradients(oracle):
    g_bits = np.array([0x3F80, 0xBF80, 0x0000, 0x4000], np.uint16)  # 1, -1, 0, 2
    th, m, v = np.zeros(4), np.zeros(4), np.zeros(4)
    oracle.adamw_step(th, g_bits, m, v, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    np.testing.assert_allclose(m, [0.1, -0.1, 0.0, 0.2], rtol=1e-15)
