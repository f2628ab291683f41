"""GPU parity of the table Adam step (hashgrid_adam_step) against the float64
oracle (oracle/optim_oracle.py).

Bar: the fp32 kernel follows the oracle to within the rounding of fp32
arithmetic: per entry |p - p_ref| <= 2^-22 |p_ref| + 1e-6 lr + 1e-5 |p_ref - p_prev|
(a few ulps of the parameter plus the relative rounding of the update; the
moments round to ~1e-7 relative, which the 1e-6 lr term absorbs where they
cancel), and the moments to 1e-6 of their largest magnitude."""
import numpy as np
import pytest
import torch

import multiresolution_hash_grid_amd as hg
from oracle import optim_oracle as O

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def check_step(p_prev, got, ref, lr, g):
    p, m, v = (t.detach().cpu().double().numpy() for t in got)
    rp, rm, rv = ref
    tol = 2.0 ** -22 * np.abs(rp) + 1e-6 * lr + 1e-5 * np.abs(rp - p_prev)
    assert np.all(np.abs(p - rp) <= tol), float(np.max(np.abs(p - rp) - tol))
    assert np.max(np.abs(m - rm)) <= 1e-6 * max(np.max(np.abs(rm)), 1e-30)
    assert np.max(np.abs(v - rv)) <= 1e-6 * max(np.max(rv), 1e-30)


@pytest.mark.parametrize("count,offset,zero,half", [(3 << 16, 0, True, True), (3 << 16, 0, False, False),
                                                    (1001, 1, False, True), (4096 + 3, 0, True, False)])
def test_adam_matches_oracle(count, offset, zero, half):
    rng = np.random.default_rng(count + offset)
    # the ABI's hyperparameters are fp32: the oracle gets the same fp32 values
    lr, b1, b2, eps = (float(np.float32(a)) for a in (1e-2, 0.9, 0.99, 1e-15))
    base = torch.zeros(count + offset, device=DEV)
    p0 = (rng.uniform(-1e-4, 1e-4, count)).astype(np.float32)
    param = base[offset:]
    param.copy_(torch.from_numpy(p0))
    m = torch.zeros(count + offset, device=DEV)[offset:]
    v = torch.zeros(count + offset, device=DEV)[offset:]
    f16 = torch.zeros(count, device=DEV, dtype=torch.float16) if half else None
    ref = (p0.astype(np.float64), np.zeros(count), np.zeros(count))
    for t in range(1, 7):
        g = (rng.standard_normal(count) * 10.0 ** rng.integers(-6, 2)).astype(np.float32)
        g[rng.random(count) < 0.3] = 0.0            # entries no point touched
        grad = torch.zeros(count + offset, device=DEV)[offset:]
        grad.copy_(torch.from_numpy(g))
        p_prev = ref[0]
        hg.hashgrid_adam_step(param, m, v, grad, lr=lr, step=t, beta1=b1, beta2=b2, eps=eps,
                              param_f16=f16, zero_grad=zero)
        torch.cuda.synchronize()
        # the oracle starts each step from the kernel's fp32 state, so errors do not compound
        ref = O.adam_step(p_prev, ref[1], ref[2], g, lr, b1, b2, eps, t)
        check_step(p_prev, (param, m, v), ref, lr, g.astype(np.float64))
        ref = tuple(a.detach().cpu().double().numpy() for a in (param, m, v))
        if zero:
            assert int(torch.count_nonzero(grad)) == 0
        else:
            assert torch.equal(grad.cpu(), torch.from_numpy(g))
        if half:
            assert torch.equal(f16, param.to(torch.float16))


def test_adam_optimizer_class_matches_torch_adam():
    # The optimizer class against torch.optim.Adam (same fp32 arithmetic, other code).
    rng = np.random.default_rng(7)
    a = torch.nn.Parameter(torch.from_numpy(rng.standard_normal((4, 1024, 2)).astype(np.float32)).to(DEV))
    b = torch.nn.Parameter(a.detach().clone())
    oa = hg.HashGridAdam([a], lr=1e-2, betas=(0.9, 0.99), eps=1e-15)
    ob = torch.optim.Adam([b], lr=1e-2, betas=(0.9, 0.99), eps=1e-15)
    for _ in range(5):
        g = torch.from_numpy(rng.standard_normal((4, 1024, 2)).astype(np.float32)).to(DEV)
        a.grad, b.grad = g.clone(), g.clone()
        oa.step()
        ob.step()
    torch.cuda.synchronize()
    a, b = a.detach(), b.detach()
    assert float((a - b).abs().max()) <= 1e-6 * float(b.abs().max()) + 1e-7
