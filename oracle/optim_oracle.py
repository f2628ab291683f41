"""CPU oracle of the table optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this module; only the tests, the package's smoke check and the benchmark's
CPU baseline leg do.  It shares no code with the HIP library.

The pages train the hash tables with Adam and no weight decay on them
("Speeding up NeRFace with Instant-NGP hash encoding", ipipp.com, section 4;
the learning rate of the tables 5-10x that of the MLP, section 3), and show
the training loop with torch.optim.Adam (ijyty.com overview, section 4).
The pages do not restate Adam itself; the steps below are those of the
published algorithm (Kingma and Ba, "Adam: A Method for Stochastic
Optimization", ICLR 2015, Algorithm 1), applied to every table entry --
torch.optim.Adam, which the pages use, updates all entries of a parameter,
including those whose gradient in this step is zero.

Plain float64 numpy, one line per step of the algorithm, nothing fused.
"""
from __future__ import annotations

import numpy as np


def adam_step(param, m, v, grad, lr: float, beta1: float, beta2: float, eps: float, t: int):
    """One Adam update at 1-based step t.

    param, m, v, grad: arrays of one shape (any float dtype; computed in float64).
    Returns (param', m', v') as float64 arrays:
        m' = beta1 m + (1 - beta1) g
        v' = beta2 v + (1 - beta2) g^2
        m^ = m' / (1 - beta1^t),  v^ = v' / (1 - beta2^t)
        param' = param - lr m^ / (sqrt(v^) + eps)
    """
    if t < 1:
        raise ValueError("Adam steps are numbered from 1")
    g = np.asarray(grad, dtype=np.float64)
    m1 = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v1 = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * (g * g)
    m_hat = m1 / (1.0 - beta1 ** t)
    v_hat = v1 / (1.0 - beta2 ** t)
    p1 = np.asarray(param, dtype=np.float64) - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p1, m1, v1
