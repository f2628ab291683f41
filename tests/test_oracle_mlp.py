"""Pins of the MLP oracle (oracle/mlp_oracle.py): the float64 network against
torch's float64 autograd of the same layers (the ipipp.com section 3 head,
Linear-ReLU-Linear-ReLU-Linear), central differences, and the binary16
rounding points against an explicitly rounded torch forward."""
import numpy as np
import pytest

from multiresolution_hash_grid_amd import inputs as I
from oracle import mlp_oracle as M

torch = pytest.importorskip("torch")


def params(seed=3, bias=0.1):
    return I.mlp_params(seed, bias_scale=bias)


def torch_net(e, W1, b1, W2, b2, W3, b3, rnd=False):
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    ws = [t(v) for v in (W1, b1, W2, b2, W3, b3)]
    x = t(e)
    r = (lambda v: v.to(torch.float16).to(torch.float64)) if rnd else (lambda v: v)
    h1 = r(torch.relu(torch.nn.functional.linear(r(x), ws[0], ws[1])))
    h2 = r(torch.relu(torch.nn.functional.linear(h1, ws[2], ws[3])))
    return x, ws, torch.nn.functional.linear(h2, ws[4], ws[5])


def test_float64_network_matches_torch_autograd():
    W1, b1, W2, b2, W3, b3 = params()
    rng = np.random.default_rng(0)
    e = rng.standard_normal((300, 32)) * 0.5
    dy = rng.standard_normal((300, 4))
    y, cache = M.forward(e, W1, b1, W2, b2, W3, b3, round_fp16=False)
    g = M.backward(cache, dy, W1, W2, W3)
    x, ws, ty = torch_net(e, W1, b1, W2, b2, W3, b3)
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["de"], x.grad.numpy(), rtol=0, atol=1e-12)
    for name, tw in zip(("dW1", "db1", "dW2", "db2", "dW3", "db3"), ws):
        np.testing.assert_allclose(g[name], tw.grad.numpy(), rtol=0, atol=1e-11, err_msg=name)


def test_weight_gradient_equals_central_difference():
    # The network is piecewise linear in each weight, so a small central
    # difference is exact unless a ReLU flips inside it.
    W1, b1, W2, b2, W3, b3 = [np.asarray(a, dtype=np.float64) for a in params(5)]
    rng = np.random.default_rng(1)
    e = rng.standard_normal((50, 32))
    dy = rng.standard_normal((50, 4))
    _, cache = M.forward(e, W1, b1, W2, b2, W3, b3, round_fp16=False)
    g = M.backward(cache, dy, W1, W2, W3)
    h = 1e-6

    def loss(W1, b1, W2, b2, W3, b3):
        return float(np.sum(M.forward(e, W1, b1, W2, b2, W3, b3, round_fp16=False)[0] * dy))

    base = [W1, b1, W2, b2, W3, b3]
    for pi, name in ((0, "dW1"), (2, "dW2"), (4, "dW3"), (1, "db1"), (3, "db2"), (5, "db3")):
        for _ in range(4):
            idx = tuple(rng.integers(0, s) for s in base[pi].shape)
            up = [a.copy() for a in base]
            dn = [a.copy() for a in base]
            up[pi][idx] += h
            dn[pi][idx] -= h
            fd = (loss(*up) - loss(*dn)) / (2 * h)
            assert abs(fd - g[name][idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx)


def test_rounding_points_match_rounded_torch_forward():
    W1, b1, W2, b2, W3, b3 = params(7)
    e = np.random.default_rng(2).standard_normal((200, 32)) * 0.3
    y, cache = M.forward(e, W1, b1, W2, b2, W3, b3, round_fp16=True)
    _, _, ty = torch_net(e, W1, b1, W2, b2, W3, b3, rnd=True)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=0, atol=1e-13)
    # the activations the matrix cores read are binary16 values
    for k in ("e", "h1", "h2"):
        assert np.array_equal(cache[k], cache[k].astype(np.float16).astype(np.float64))


def test_mlp_params_are_xavier_and_fp16():
    W1, b1, W2, b2, W3, b3 = I.mlp_params(11)
    assert W1.shape == (64, 32) and W2.shape == (64, 64) and W3.shape == (4, 64)
    assert W1.dtype == np.float16 and b1.dtype == np.float32
    for W, (fi, fo) in ((W1, (32, 64)), (W2, (64, 64)), (W3, (64, 4))):
        a = np.sqrt(6.0 / (fi + fo))
        assert np.max(np.abs(W.astype(np.float64))) <= a * (1 + 2 ** -10)
    assert not np.any(b1) and not np.any(b3)     # a fresh network starts with zero biases
