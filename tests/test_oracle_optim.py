"""Pins of the optimizer oracle (oracle/optim_oracle.py) against facts that do
not come from it: closed forms of Adam (Kingma and Ba 2015, Algorithm 1) and
torch.optim.Adam on the CPU in float64, the optimizer the pages train with
(ijyty.com overview, section 4; ipipp.com section 4: Adam, no weight decay
on the hash tables)."""
import numpy as np
import pytest

from oracle import optim_oracle as O

LR, B1, B2, EPS = 1e-2, 0.9, 0.999, 1e-8


def test_first_step_is_lr_times_sign():
    # From zero moments the bias corrections make m^ = g and v^ = g^2, so the
    # first update is lr * g / (|g| + eps) whatever beta1 and beta2 are.
    rng = np.random.default_rng(0)
    g = rng.standard_normal(1000)
    p0 = rng.standard_normal(1000)
    for b1, b2 in ((0.9, 0.999), (0.5, 0.9), (0.0, 0.0)):
        p, m, v = O.adam_step(p0, np.zeros(1000), np.zeros(1000), g, LR, b1, b2, EPS, 1)
        np.testing.assert_allclose(p, p0 - LR * g / (np.abs(g) + EPS), rtol=0, atol=1e-15)
        np.testing.assert_allclose(m, (1 - b1) * g, rtol=1e-15)
        np.testing.assert_allclose(v, (1 - b2) * g * g, rtol=1e-15)


def test_constant_gradient_moves_linearly():
    # With a constant gradient, m_t = (1 - beta1^t) g and v_t = (1 - beta2^t) g^2
    # exactly, so every step moves by lr * g / (|g| + eps): a wrong power t in a
    # bias correction breaks this at t >= 2.
    g = np.array([3.0, -0.25, 1e-3, -7.5])
    p = np.array([1.0, 2.0, 3.0, 4.0])
    m = np.zeros(4)
    v = np.zeros(4)
    for t in range(1, 21):
        p, m, v = O.adam_step(p, m, v, g, LR, B1, B2, EPS, t)
        np.testing.assert_allclose(m, (1 - B1 ** t) * g, rtol=1e-13)
        np.testing.assert_allclose(v, (1 - B2 ** t) * g * g, rtol=1e-12)
    np.testing.assert_allclose(p, np.array([1.0, 2.0, 3.0, 4.0]) - 20 * LR * g / (np.abs(g) + EPS), rtol=0,
                               atol=1e-12)


def test_scale_invariance_without_eps():
    # eps = 0: Adam's update does not depend on the gradient's scale.
    rng = np.random.default_rng(1)
    gs = [rng.standard_normal(64) for _ in range(5)]
    a = b = (rng.standard_normal(64), np.zeros(64), np.zeros(64))
    for t, g in enumerate(gs, start=1):
        a = O.adam_step(*a, g, LR, B1, B2, 0.0, t)
        b = O.adam_step(*b, 1000.0 * g, LR, B1, B2, 0.0, t)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-13)


def test_matches_torch_adam_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    p0 = rng.standard_normal(257)
    param = torch.nn.Parameter(torch.tensor(p0, dtype=torch.float64))
    opt = torch.optim.Adam([param], lr=LR, betas=(B1, B2), eps=EPS, weight_decay=0.0, foreach=False)
    state = (p0, np.zeros(257), np.zeros(257))
    for t in range(1, 8):
        g = rng.standard_normal(257) * (0.0 if t == 4 else 1.0)   # one all-zero gradient step
        g[::5] = 0.0                                               # entries no point touched
        param.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        state = O.adam_step(*state, g, LR, B1, B2, EPS, t)
        np.testing.assert_allclose(state[0], param.detach().numpy(), rtol=0, atol=1e-14)
        st = opt.state[param]
        np.testing.assert_allclose(state[1], st["exp_avg"].numpy(), rtol=1e-12, atol=1e-16)  # torch forms m by lerp
        np.testing.assert_allclose(state[2], st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-16)


def test_rejects_step_zero():
    with pytest.raises(ValueError):
        O.adam_step(np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1), LR, B1, B2, EPS, 0)
