"""Element-wise bound on how far the matrix-core MLP head may lie from its
oracle (oracle/mlp_oracle.py).

Test infrastructure: the GPU parity tests of the head use it in the regime
where a fixed relative bar cannot hold -- zero biases on freshly initialised
tables, whose hidden activations are binary16 subnormals with about three
significant digits.  The kernels and the oracle round the same tensors to
binary16 (e, h1, h2; the scaled dL/dy, dz2, dz1) from fp32 sums of the same
binary16 operands, in different summation orders, so:
  - an fp32 sum of k terms lies within (k + 1) u sum|terms| of the exact sum
    (u = 2^-24), and two such sums within twice that of each other;
  - two values within d of each other round to the same binary16 value unless
    one lies within d of a rounding boundary (the midpoint between two
    neighbouring binary16 values); there the results differ by at most
    d + one binary16 ulp;
  - a gradient whose ReLU decision is uncertain (|z| within its bound) may be
    its whole value on one side and zero on the other;
  - outputs (y, dL/de) are fp32 sums on the GPU against float64 in the
    oracle, and the weight and bias gradients sum over points along the
    kernels' fp32 chain (16 products per MFMA, the tiles of one wave, the wave
    partials in two passes), each step adding at most u of the magnitudes.
Differences are propagated forward through the layers with the oracle's own
values.  Where no rounding can flip, the bound is a few fp32 roundings of the
element; it grows only where a flip is possible.  The table gradient's bound
is the oracle's table backward of the dL/de bound (the weights are
non-negative), plus the binned path's 20-bit products and the 1e-5 per-level
bar of the table backward itself.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24


def ulp16(a) -> np.ndarray:
    """One binary16 ulp at |a| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(a, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.exp2(np.maximum(e - 10.0, -24.0))


def boundary_distance(v) -> np.ndarray:
    """Distance from v to the nearest binary16 rounding boundary."""
    v = np.asarray(v, dtype=np.float64)
    r = v.astype(np.float16)
    up = np.nextafter(r, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(r, np.float16(-np.inf)).astype(np.float64)
    r = r.astype(np.float64)
    return np.minimum((r + up) / 2 - v, v - (r + dn) / 2)


def rounding_step(v, d) -> np.ndarray:
    """Bound on |fp16(v') - fp16(v)| for |v' - v| <= d."""
    d = np.asarray(d, dtype=np.float64)
    return np.where(boundary_distance(v) > d, 0.0, d + ulp16(np.abs(v) + d))


def gamma(k: int) -> float:
    return (k + 1) * U


def chain_steps(n: int) -> int:
    """fp32 additions along one weight-gradient sum of the kernels over n
    points: 16 per MFMA, the tiles of a wave, the two reduction passes."""
    tiles = (n + 15) // 16
    grid = min((tiles + 3) // 4, 1024)
    waves = 4 * grid
    per_wave = (tiles + waves - 1) // waves
    return 16 + per_wave + (waves + 63) // 64 + 64 + 2


def _f32sum(a, W):
    return (np.asarray(a, dtype=np.float32) @ np.asarray(W, dtype=np.float32)).astype(np.float64)


def bounds(e_exact, e_err, params, cache, grads, dy):
    """Bounds for y, de, dW1, db1, dW2, db2, dW3, db3 (the oracle's output
    keys, plus 'y'), and the count of uncertain ReLU decisions.
      e_exact : the head's input before rounding, float64 [n, k] (the oracle's
                encoding, or for the TinyNeRF head the point and its encoding);
      e_err   : bound on the GPU input's fp32 error before rounding (a scalar,
                or one per input column);
      params  : [W1, b1, W2, b2, W3, b3];  cache, grads : the oracle's (fp32 sums).
    """
    W1, b1, W2, b2, W3, b3 = (np.asarray(p, dtype=np.float64) for p in params)
    A1, A2, A3 = np.abs(W1), np.abs(W2), np.abs(W3)
    n = e_exact.shape[0]
    e, z1, h1, z2, h2 = cache["e"], cache["z1"], cache["h1"], cache["z2"], cache["h2"]
    g33, g65, g5 = gamma(W1.shape[1]), gamma(64), gamma(4)
    # forward
    de_in = rounding_step(e_exact, e_err)
    dz1 = (de_in @ A1.T) * (1 + g33) + 2 * g33 * (np.abs(e) @ A1.T + np.abs(b1))
    dh1 = rounding_step(np.maximum(z1, 0.0), dz1)
    dz2 = (dh1 @ A2.T) * (1 + g65) + 2 * g65 * (np.abs(h1) @ A2.T + np.abs(b2))
    dh2 = rounding_step(np.maximum(z2, 0.0), dz2)
    dy_out = dh2 @ A3.T + g65 * ((np.abs(h2) + dh2) @ A3.T + np.abs(b3))
    # backward, in the scaled domain of the call's scale s (g3 is the same on both sides)
    s = grads["scale"]
    g3 = (np.asarray(dy, dtype=np.float64) * s).astype(np.float16).astype(np.float64)
    ag3 = np.abs(g3)
    unc2 = np.abs(z2) <= dz2
    unc1 = np.abs(z1) <= dz1
    u2 = _f32sum(g3, W3)
    du2 = 2 * g5 * (ag3 @ A3)
    v2 = u2 * (z2 > 0)
    ddz2 = np.where(unc2, np.abs(u2) + du2 + ulp16(np.abs(u2) + du2), rounding_step(v2, du2))
    dz2_or = v2.astype(np.float16).astype(np.float64)
    u1 = _f32sum(dz2_or, W2)
    du1 = (ddz2 @ A2) * (1 + g65) + 2 * g65 * (np.abs(dz2_or) @ A2)
    v1 = u1 * (z1 > 0)
    ddz1 = np.where(unc1, np.abs(u1) + du1 + ulp16(np.abs(u1) + du1), rounding_step(v1, du1))
    dz1_or = v1.astype(np.float16).astype(np.float64)
    dde = ((ddz1 @ A1) * (1 + g33) + g33 * (np.abs(dz1_or) @ A1)) / s
    dde = dde + U * (np.abs(grads["de"]) + dde)  # the fp32 value written
    acc = chain_steps(n) * U

    def wgrad(dg, g_mag, dact, act_mag):
        # sum_p g (x) act: perturbation of either factor plus the fp32 chain
        return (dg.T @ (act_mag + dact) + g_mag.T @ dact + acc * ((g_mag + dg).T @ (act_mag + dact))) / s

    ae, ah1, ah2 = np.abs(e), np.abs(h1), np.abs(h2)
    az2, az1 = np.abs(dz2_or), np.abs(dz1_or)
    return {
        "y": dy_out,
        "de": dde,
        "dW3": wgrad(np.zeros_like(ag3), ag3, dh2, ah2),
        "db3": acc * ag3.sum(0) / s,
        "dW2": wgrad(ddz2, az2, dh1, ah1),
        "db2": (ddz2.sum(0) + acc * (az2 + ddz2).sum(0)) / s,
        "dW1": wgrad(ddz1, az1, de_in, ae),
        "db1": (ddz1.sum(0) + acc * (az1 + ddz1).sum(0)) / s,
        "uncertain_relu": int(unc1.sum() + unc2.sum()),
    }


def table_bound(oracle, grid, x, de_ref, dde, ref_table):
    """Per-entry bound of the table gradient [L][T][F]: the oracle's table
    backward of the dL/de bound, the binned path's 20-bit products, and the
    1e-5 per-level bar of the table backward."""
    de_mag = np.abs(de_ref) + dde
    b = oracle.backward(grid, x, (dde + 2.0 ** -19 * de_mag).astype(np.float32))
    lvl = 1e-5 * np.max(np.abs(ref_table), axis=(1, 2), keepdims=True)
    return b * (1 + 1e-6) + lvl
