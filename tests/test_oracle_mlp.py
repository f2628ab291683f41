"""Pins of the MLP oracle (oracle/mlp_oracle.py): the float64 network against
torch's float64 autograd of the same layers (the ipipp.com section 3 head,
Linear-ReLU-Linear-ReLU-Linear), central differences, and the binary16
rounding points of the forward and of the backward against torch autograd
with explicit rounding (the backward's through an identity whose gradient is
rounded: at dL/dy and at the gradients of the two pre-activations, each in
the scaled domain of the call's power-of-two scale)."""
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


def test_tinynerf_input_is_the_point_then_its_encoding():
    # jsqmd.com section 4: TinyNeRF concatenates the raw point before its hash
    # features and feeds Linear(35, 64), ReLU, Linear(64, 64), ReLU,
    # Linear(64, 4).  The oracle takes that concatenation as its input u, and
    # its dL/du splits into the point's part (the first 3 columns) and the
    # encoding's (the upstream of the table backward).  Reference: the model
    # built from torch.nn layers as the page writes it, in float64.
    W1, b1, W2, b2, W3, b3 = I.mlp_params(11, sizes=(35, 64, 64, 4), bias_scale=0.1)
    rng = np.random.default_rng(4)
    x = rng.uniform(0.0, 1.0, (120, 3))
    h = rng.standard_normal((120, 32)) * 0.3
    dy = rng.standard_normal((120, 4))
    y, cache = M.forward(np.concatenate([x, h], axis=1), W1, b1, W2, b2, W3, b3, round_fp16=False)
    g = M.backward(cache, dy, W1, W2, W3)
    net = torch.nn.Sequential(torch.nn.Linear(35, 64), torch.nn.ReLU(), torch.nn.Linear(64, 64), torch.nn.ReLU(),
                              torch.nn.Linear(64, 4)).double()
    with torch.no_grad():
        for layer, (W, b) in zip((net[0], net[2], net[4]), ((W1, b1), (W2, b2), (W3, b3))):
            layer.weight.copy_(torch.tensor(np.asarray(W, dtype=np.float64)))
            layer.bias.copy_(torch.tensor(np.asarray(b, dtype=np.float64)))
    xt = torch.tensor(x, requires_grad=True)
    ht = torch.tensor(h, requires_grad=True)
    ty = net(torch.cat([xt, ht], dim=-1))
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["de"][:, 3:], ht.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["de"][:, :3], xt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dW1"], net[0].weight.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["db1"], net[0].bias.grad.numpy(), rtol=0, atol=1e-11)


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
    y, cache = M.forward(e, W1, b1, W2, b2, W3, b3, round_fp16=True, acc32=False)
    _, _, ty = torch_net(e, W1, b1, W2, b2, W3, b3, rnd=True)
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=0, atol=1e-13)
    # the activations the matrix cores read are binary16 values
    for k in ("e", "h1", "h2"):
        assert np.array_equal(cache[k], cache[k].astype(np.float16).astype(np.float64))


def _half(v: "torch.Tensor") -> "torch.Tensor":
    """float64 -> binary16 (one rounding to nearest even) -> float64.  torch's
    own cast goes through float32 first, a double rounding that differs on
    rare values; numpy rounds the float64 value directly."""
    return torch.from_numpy(v.detach().numpy().astype(np.float16).astype(np.float64))


class _RoundGrad(torch.autograd.Function):
    """Identity whose backward rounds the incoming gradient g to binary16 in
    the scaled domain: g -> fp16(g * s) / s (s a power of two)."""

    @staticmethod
    def forward(ctx, v, s):
        ctx.s = s
        return v.view_as(v)

    @staticmethod
    def backward(ctx, g):
        s = ctx.s
        return _half(g * s) / s, None


def torch_rounded_backward(e, W1, b1, W2, b2, W3, b3, dy, s):
    """torch float64 autograd of the head with binary16 rounding of the
    forward activations (e, h1, h2) and of the gradients reaching y, z2, z1."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    ws = [t(v) for v in (W1, b1, W2, b2, W3, b3)]
    x = t(e)
    # binary16 value, identity gradient (a dtype cast would round the gradient too)
    r = lambda v: v + (_half(v) - v.detach())
    lin = torch.nn.functional.linear
    z1 = _RoundGrad.apply(lin(r(x), ws[0], ws[1]), s)
    h1 = r(torch.relu(z1))
    z2 = _RoundGrad.apply(lin(h1, ws[2], ws[3]), s)
    h2 = r(torch.relu(z2))
    y = _RoundGrad.apply(lin(h2, ws[4], ws[5]), s)
    y.backward(torch.tensor(np.asarray(dy, dtype=np.float64)))
    return x, ws


@pytest.mark.parametrize("dy_scale,bias", [(1.0, 0.1), (1e-7, 0.1), (3e3, "linear"), (1e-7, 0.0)])
def test_backward_rounding_points_match_rounded_torch_autograd(dy_scale, bias):
    # The straight-through rounding of binary16 in the forward (h = fp16(relu(z)))
    # passes gradient as the identity, as the GPU's backward does; the ReLU mask
    # is z > 0.  dy of 1e-7 (a mean loss over millions of points) is where the
    # scale matters: rounded unscaled it would fall into binary16's subnormals.
    W1, b1, W2, b2, W3, b3 = I.mlp_params(17, bias_scale=bias)
    rng = np.random.default_rng(4)
    e = rng.standard_normal((400, 32)) * 0.3
    dy = (rng.standard_normal((400, 4)) * dy_scale).astype(np.float32)
    _, cache = M.forward(e, W1, b1, W2, b2, W3, b3, round_fp16=True, acc32=False)
    g = M.backward(cache, dy, W1, W2, W3)
    s = g["scale"]
    m = np.max(np.abs(dy.astype(np.float64)))
    assert 1.0 <= m * s < 2.0 and s == 2.0 ** np.round(np.log2(s))
    x, ws = torch_rounded_backward(e, W1, b1, W2, b2, W3, b3, dy, s)
    # x.grad is d/de of the rounded input, i.e. the straight-through de
    np.testing.assert_allclose(g["de"], x.grad.numpy(), rtol=1e-12, atol=1e-12 * np.max(np.abs(g["de"])))
    for name, tw in zip(("dW1", "db1", "dW2", "db2", "dW3", "db3"), ws):
        ref = tw.grad.numpy()
        np.testing.assert_allclose(g[name], ref, rtol=1e-12, atol=1e-12 * np.max(np.abs(ref)), err_msg=name)


@pytest.mark.parametrize("bias,e_scale", [("linear", 0.3), (0.0, 1e-4)])
def test_pre_activations_are_fp32_sums(bias, e_scale):
    # With round_fp16 the pre-activations that get rounded are fp32 sums of the
    # binary16 operands: fp32 values, within the fp32 summation bound of the
    # exact (float64) sum, and near torch's own fp32 linear layer.
    W1, b1, W2, b2, W3, b3 = I.mlp_params(19, bias_scale=bias)
    e = np.random.default_rng(5).uniform(-1, 1, (500, 32)) * e_scale
    _, c32 = M.forward(e, W1, b1, W2, b2, W3, b3, round_fp16=True)
    _, c64 = M.forward(e, W1, b1, W2, b2, W3, b3, round_fp16=True, acc32=False)
    assert c32["acc32"] and not c64["acc32"]
    t32 = lambda a: torch.tensor(np.asarray(a, dtype=np.float32))
    for z, a, W, b, k in (("z1", c32["e"], W1, b1, 32), ("z2", c32["h1"], W2, b2, 64)):
        got = c32[z]
        assert np.array_equal(got, got.astype(np.float32).astype(np.float64)), z
        exact = a @ np.asarray(W, dtype=np.float64).T + np.asarray(b, dtype=np.float64)
        mag = np.abs(a) @ np.abs(np.asarray(W, dtype=np.float64)).T + np.abs(np.asarray(b, dtype=np.float64))
        assert np.all(np.abs(got - exact) <= (k + 1) * 2.0 ** -24 * mag), z
        tor = torch.nn.functional.linear(t32(a), t32(W), t32(b)).numpy().astype(np.float64)
        assert np.all(np.abs(got - tor) <= 2 * (k + 1) * 2.0 ** -24 * mag), z
        assert np.any(got != exact), z  # genuinely rounded to fp32


def test_gradient_scale_rule():
    assert M.grad_scale(np.array([0.0, -0.0])) == 1.0
    assert M.grad_scale(np.array([1.0])) == 1.0
    assert M.grad_scale(np.array([-1.5, 0.25])) == 1.0
    assert M.grad_scale(np.array([2.0])) == 0.5
    assert M.grad_scale(np.array([1e-7, -3e-8])) == 2.0 ** 24       # 1e-7 in [2^-24, 2^-23)
    assert M.grad_scale(np.array([np.nan, np.inf, 0.75])) == 2.0   # non-finite values are ignored


def test_mlp_params_are_xavier_and_fp16():
    W1, b1, W2, b2, W3, b3 = I.mlp_params(11)
    assert W1.shape == (64, 32) and W2.shape == (64, 64) and W3.shape == (4, 64)
    assert W1.dtype == np.float16 and b1.dtype == np.float32
    for W, (fi, fo) in ((W1, (32, 64)), (W2, (64, 64)), (W3, (64, 4))):
        a = np.sqrt(6.0 / (fi + fo))
        assert np.max(np.abs(W.astype(np.float64))) <= a * (1 + 2 ** -10)
    # biases as torch.nn.Linear draws them: U(-1/sqrt(fan_in), 1/sqrt(fan_in))
    for b, fi in ((b1, 32), (b2, 64), (b3, 64)):
        assert b.dtype == np.float32 and np.any(b) and np.max(np.abs(b)) <= 1.0 / np.sqrt(fi)
    assert not any(np.any(v) for v in I.mlp_params(11, bias_scale=0.0)[1::2])
