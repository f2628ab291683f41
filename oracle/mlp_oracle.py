"""CPU oracle of the tiny MLP that follows the encoder.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module; only the tests, the package's smoke check and the benchmark's
CPU baseline leg do.  It shares no code with the HIP library.

The network is the NeRFace head of "Speeding up NeRFace with Instant-NGP hash
encoding" (ipipp.com, section 3 listing): Linear(32, 64), ReLU, Linear(64, 64),
ReLU, Linear(64, 4), no output activation (its forward splits the 4 outputs
into density and colour afterwards).  nn.Linear carries a bias, so
    y = W3 relu(W2 relu(W1 e + b1) + b2) + b3,   W_i stored [out][in].
The 32 inputs are the encoding of L = 16 levels x F = 2 features (the page's
expression code is a separate, optional input and is not part of this head).

Precision: the GPU feeds its matrix cores binary16 operands with fp32
accumulation, so with ``round_fp16`` the oracle rounds to binary16 (nearest
even) exactly the tensors the GPU feeds them -- the encoding e and the hidden
activations h1, h2 in the forward; dL/dy and the pre-activation gradients
dz2, dz1 in the backward -- and does everything else in float64.  With
``round_fp16=False`` it is the plain float64 network.

Where a sum is rounded to binary16 (the pre-activations z1, z2 and, in the
backward, W3^T g and W2^T dz2), the oracle forms it as an fp32 sum of the
binary16 operands (``acc32``, on whenever ``round_fp16`` is), because the
configuration accumulates in fp32 and the rounding and the ReLU decision are
then taken from a value of the kernel's own precision; the two fp32 sums
differ only by their summation order.  Outputs (y, dL/de, the weight and bias
gradients) are float64 sums of the binary16 operands.

The backward's binary16 operands carry one power-of-two scale s per call
(``grad_scale``): dL/dy is multiplied by s before it is rounded, so that the
largest finite |dL/dy| lands in [1, 2) and small upstream gradients (a loss
averaged over millions of points gives ~1e-7) stay clear of binary16's
subnormal range; dz2 and dz1 inherit the scale, and dL/de and the weight and
bias gradients are divided by s.  Multiplying by a power of two is exact, so
without rounding the scale changes nothing.

Plain numpy: each layer is one matrix product (a library primitive), no
fusion or reordering.
"""
from __future__ import annotations

import numpy as np


def round_half(a) -> np.ndarray:
    """float64 -> binary16 (round to nearest even, subnormals kept) -> float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def _r(a, on: bool) -> np.ndarray:
    return round_half(a) if on else np.asarray(a, dtype=np.float64)


def _sum(a, W, b, acc32: bool) -> np.ndarray:
    """a @ W + b: an fp32 sum (library sgemm, then the fp32 bias) with acc32,
    else float64."""
    if acc32:
        r = np.asarray(a, dtype=np.float32) @ np.asarray(W, dtype=np.float32)
        if b is not None:
            r = r + np.asarray(b, dtype=np.float32)
        return r.astype(np.float64)
    r = np.asarray(a, dtype=np.float64) @ np.asarray(W, dtype=np.float64)
    return r if b is None else r + np.asarray(b, dtype=np.float64)


def forward(e, W1, b1, W2, b2, W3, b3, round_fp16: bool = True, acc32: bool | None = None):
    """e [n, 32] encoding -> (y [n, 4] float64, cache for backward)."""
    acc32 = round_fp16 if acc32 is None else acc32
    W1, W2, W3 = (np.asarray(w, dtype=np.float64) for w in (W1, W2, W3))
    b1, b2, b3 = (np.asarray(b, dtype=np.float64) for b in (b1, b2, b3))
    e16 = _r(e, round_fp16)
    z1 = _sum(e16, W1.T, b1, acc32)
    h1 = _r(np.maximum(z1, 0.0), round_fp16)
    z2 = _sum(h1, W2.T, b2, acc32)
    h2 = _r(np.maximum(z2, 0.0), round_fp16)
    y = h2 @ W3.T + b3
    return y, dict(e=e16, z1=z1, h1=h1, z2=z2, h2=h2, round=round_fp16, acc32=acc32)


def grad_scale(dy) -> float:
    """s = 2^(1 - e) where the largest finite |dy| lies in [2^(e-1), 2^e), so
    that max|dy| * s is in [1, 2); 1 when dy has no finite non-zero value."""
    a = np.abs(np.asarray(dy, dtype=np.float64)).ravel()
    a = a[np.isfinite(a)]
    m = float(a.max()) if a.size else 0.0
    if m == 0.0:
        return 1.0
    e = int(np.frexp(m)[1])
    return float(2.0 ** (1 - e))


def backward(cache, dy, W1, W2, W3):
    """Gradients of sum(dy * y): returns dict(de, dW1, db1, dW2, db2, dW3, db3,
    scale) (float64; the ReLU passes gradient where its input is > 0)."""
    on, acc32 = cache["round"], cache["acc32"]
    W1, W2, W3 = (np.asarray(w, dtype=np.float64) for w in (W1, W2, W3))
    s = grad_scale(dy)
    g3 = _r(np.asarray(dy, dtype=np.float64) * s, on)
    dz2 = _r(_sum(g3, W3, None, acc32) * (cache["z2"] > 0), on)
    dz1 = _r(_sum(dz2, W2, None, acc32) * (cache["z1"] > 0), on)
    de = (dz1 @ W1) / s
    return dict(de=de,
                dW3=(g3.T @ cache["h2"]) / s, db3=g3.sum(0) / s,
                dW2=(dz2.T @ cache["h1"]) / s, db2=dz2.sum(0) / s,
                dW1=(dz1.T @ cache["e"]) / s, db1=dz1.sum(0) / s,
                scale=s)
