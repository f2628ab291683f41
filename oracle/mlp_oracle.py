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


def forward(e, W1, b1, W2, b2, W3, b3, round_fp16: bool = True):
    """e [n, 32] encoding -> (y [n, 4] float64, cache for backward)."""
    W1, W2, W3 = (np.asarray(w, dtype=np.float64) for w in (W1, W2, W3))
    b1, b2, b3 = (np.asarray(b, dtype=np.float64) for b in (b1, b2, b3))
    e16 = _r(e, round_fp16)
    z1 = e16 @ W1.T + b1
    h1 = _r(np.maximum(z1, 0.0), round_fp16)
    z2 = h1 @ W2.T + b2
    h2 = _r(np.maximum(z2, 0.0), round_fp16)
    y = h2 @ W3.T + b3
    return y, dict(e=e16, z1=z1, h1=h1, z2=z2, h2=h2, round=round_fp16)


def backward(cache, dy, W1, W2, W3):
    """Gradients of sum(dy * y): returns dict(de, dW1, db1, dW2, db2, dW3, db3)
    (float64; the ReLU passes gradient where its input is > 0)."""
    on = cache["round"]
    W1, W2, W3 = (np.asarray(w, dtype=np.float64) for w in (W1, W2, W3))
    g3 = _r(dy, on)
    dz2 = _r((g3 @ W3) * (cache["z2"] > 0), on)
    dz1 = _r((dz2 @ W2) * (cache["z1"] > 0), on)
    de = dz1 @ W1
    return dict(de=de,
                dW3=g3.T @ cache["h2"], db3=g3.sum(0),
                dW2=dz2.T @ cache["h1"], db2=dz2.sum(0),
                dW1=dz1.T @ cache["e"], db1=dz1.sum(0))
