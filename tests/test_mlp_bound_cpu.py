"""The MLP head's element-wise error bound (tests/mlp_error_bound.py) holds for
an fp32 evaluation of the head that rounds to binary16 at the oracle's points
-- the arithmetic class of the matrix-core kernels -- in the regime where a
fixed relative bar fails: zero biases and encodings of a freshly initialised
table (|e| <= 1e-4, binary16 subnormal activations), and with tiny dL/dy."""
import numpy as np
import pytest

from multiresolution_hash_grid_amd import inputs as I
from oracle import mlp_oracle as M

import mlp_error_bound as EB


def f16(a):
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)


def seq(a, B, c=None):
    """a @ B (+ c) in fp32, adding the contraction terms one at a time from
    the last to the first: a summation order unlike the oracle's library sgemm."""
    a, B = np.asarray(a, dtype=np.float32), np.asarray(B, dtype=np.float32)
    acc = np.zeros((a.shape[0], B.shape[1]), dtype=np.float32) if c is None else \
        np.broadcast_to(np.asarray(c, dtype=np.float32), (a.shape[0], B.shape[1])).copy()
    for k in range(a.shape[1] - 1, -1, -1):
        acc = (acc + a[:, k:k + 1] * B[k:k + 1, :]).astype(np.float32)
    return acc


def fp32_head(e_exact, params, dy):
    """Forward and backward in fp32 with binary16 operands at the oracle's
    rounding points and the same power-of-two gradient scale."""
    W1, b1, W2, b2, W3, b3 = (np.asarray(p, dtype=np.float32) for p in params)
    e = f16(e_exact.astype(np.float32))
    z1 = seq(e, W1.T, b1)
    h1 = f16(np.maximum(z1, 0))
    z2 = seq(h1, W2.T, b2)
    h2 = f16(np.maximum(z2, 0))
    y = seq(h2, W3.T, b3)
    s = np.float32(M.grad_scale(dy))
    g3 = f16(dy.astype(np.float32) * s)
    dz2 = f16(seq(g3, W3) * (z2 > 0))
    dz1 = f16(seq(dz2, W2) * (z1 > 0))
    inv = np.float32(1.0) / s
    ones = np.ones((1, e.shape[0]), dtype=np.float32)
    return dict(y=y, de=seq(dz1, W1) * inv, dW3=seq(g3.T, h2) * inv, db3=seq(ones, g3)[0] * inv,
                dW2=seq(dz2.T, h1) * inv, db2=seq(ones, dz2)[0] * inv, dW1=seq(dz1.T, e) * inv,
                db1=seq(ones, dz1)[0] * inv)


@pytest.mark.parametrize("bias,dy_scale,e_scale", [(0.0, 1.0, 1e-4), (0.0, 1e-7, 1e-4), ("linear", 1.0, 0.3),
                                                   (0.1, 1e-7, 1e-4)])
def test_fp32_head_within_bound(bias, dy_scale, e_scale):
    rng = np.random.default_rng(21)
    n = 4096
    params = I.mlp_params(23, bias_scale=bias)
    e_exact = rng.uniform(-1, 1, (n, 32)) * e_scale
    dy = (rng.standard_normal((n, 4)) * dy_scale).astype(np.float32)
    W1, b1, W2, b2, W3, b3 = params
    y_ref, cache = M.forward(e_exact, W1, b1, W2, b2, W3, b3, round_fp16=True)
    g_ref = M.backward(cache, dy, W1, W2, W3)
    # the fp32 encoding differs from the exact one by its own rounding
    bd = EB.bounds(e_exact, 2.0 ** -24 * e_scale, params, cache, g_ref, dy)
    got = fp32_head(e_exact, params, dy)
    ref = dict(g_ref, y=y_ref)
    for k in ("y", "de", "dW1", "db1", "dW2", "db2", "dW3", "db3"):
        diff = np.abs(got[k].astype(np.float64) - ref[k])
        assert np.all(diff <= bd[k]), (k, float(np.max(diff - bd[k])))


@pytest.mark.parametrize("bias,e_scale", [("linear", 0.3), (0.0, 1e-4)])
def test_bound_is_tight_where_no_rounding_can_flip(bias, e_scale):
    # The bound only grows where a rounding or a ReLU decision can flip: y
    # stays near one binary16 rounding of its inputs (~1e-3), most of dL/de
    # far below, and the weight gradients, which sum every point including
    # the few with an uncertain ReLU, within a few per cent.
    rng = np.random.default_rng(22)
    params = I.mlp_params(24, bias_scale=bias)
    e_exact = rng.uniform(-1, 1, (4096, 32)) * e_scale
    dy = rng.standard_normal((4096, 4)).astype(np.float32)
    W1, b1, W2, b2, W3, b3 = params
    y_ref, cache = M.forward(e_exact, W1, b1, W2, b2, W3, b3, round_fp16=True)
    g_ref = M.backward(cache, dy, W1, W2, W3)
    bd = EB.bounds(e_exact, 2.0 ** -24 * e_scale, params, cache, g_ref, dy)
    assert bd["uncertain_relu"] < 1e-3 * 4096 * 128
    rel = bd["y"] / np.max(np.abs(y_ref))
    assert np.median(rel) < 3e-3 and np.max(rel) < 0.05
    rel = bd["de"] / np.max(np.abs(g_ref["de"]))
    assert np.median(rel) < 3e-4 and np.mean(rel > 1e-2) < 0.02
    for k in ("dW1", "dW2", "dW3", "db1", "db2", "db3"):
        assert np.max(bd[k]) / np.max(np.abs(g_ref[k])) < 0.1, k


def test_ulp16():
    assert EB.ulp16(1.0) == 2.0 ** -10
    assert EB.ulp16(1.5) == 2.0 ** -10
    assert EB.ulp16(2.0 ** -14) == 2.0 ** -24
    assert EB.ulp16(1e-6) == 2.0 ** -24
    assert EB.ulp16(65504.0) == 32.0
    # the ulp is the gap to the next binary16 value
    for v in (0.1, 3.0, 1e-3, 7e-6, 1000.0):
        h = np.float16(v)
        assert float(np.nextafter(h, np.float16(np.inf))) - float(h) == EB.ulp16(float(h))
