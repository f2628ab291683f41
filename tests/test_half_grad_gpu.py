"""GPU parity of the binary16 table gradient (grad_dtype "f16").

The binned backward sums each partition exactly in 64-bit fixed point.  With
an fp32 gradient it stores the fp32 sum of an entry's old value and the
partition's sum; with a binary16 gradient it rounds that same fp32 sum once
to binary16.  So from the same starting values (binary16 ones, widened
exactly for the fp32 run) the binary16 gradient is the fp32 gradient rounded
to binary16, bit for bit, wherever no contribution takes the direct atomics
(non-finite upstream values, corners whose pair straddles two partitions:
none in these batches).  Against the oracle the bar is the half-precision
one, 1e-3 of the level's largest value: the one rounding errs by at most
2^-11 of the entry, on top of the fp32 path's 1e-5.

Covered: the standard grid (in one group and in the smallest level groups),
binary16 tables, the large binary16 grid, the other shapes (D = 1, 2, 4;
F = 1, 4, 8), a 2-entry F = 1 table (a partition flush of fewer than four
values), starting values that are -0, subnormal or large, the
allocation-free entry point, the MLP head's backward, the autograd
functions of a binary16 table parameter, and non-finite upstream values,
which reach the entries through packed binary16 atomics as IEEE arithmetic
has them.  A binary16 gradient without the binned path is refused.
"""
import dataclasses
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import multiresolution_hash_grid_amd as hg  # noqa: E402
from multiresolution_hash_grid_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
HALF_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _threads(oracle):
    oracle.set_threads(min(16, os.cpu_count() or 1))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def half_cfg(cfg):
    return dataclasses.replace(cfg, grad_dtype="f16")


def start_values(shape, seed):
    """binary16 starting gradient: N(0, 0.5) with some -0, +0, subnormal
    (down to the smallest, 2^-24) and large values."""
    rng = np.random.default_rng(seed)
    g = rng.normal(0.0, 0.5, size=shape).astype(np.float16)
    pick = rng.random(shape)
    g[pick < 0.02] = np.float16(-0.0)
    g[(pick >= 0.02) & (pick < 0.03)] = np.float16(0.0)
    sub = (pick >= 0.03) & (pick < 0.05)
    g[sub] = (rng.integers(1, 1024, size=int(sub.sum())) * 2.0 ** -24).astype(np.float16)
    g[(pick >= 0.05) & (pick < 0.055)] = np.float16(3000.0)
    return g


def level_check(got, ref, L, tol):
    got = got.astype(np.float64)
    for l in range(L):
        scale = float(np.max(np.abs(ref[l])))
        err = float(np.max(np.abs(got[l] - ref[l])))
        assert err <= tol * scale, (l, err, scale)


def both(cfg, x, d, g0, workspace="auto"):
    """(fp32 gradient, binary16 gradient) after one backward from g0."""
    g32 = dev(g0.astype(np.float32))
    hg.hashgrid_backward(cfg, x, d, g32, workspace=workspace)
    g16 = dev(g0)
    hg.hashgrid_backward(half_cfg(cfg), x, d, g16, workspace=workspace)
    return g32.cpu().numpy(), g16.cpu().numpy()


CASES = [
    # name, points, overrides
    ("standard", 3 * 4096 + 77, {}),
    ("standard", 20000, {"table_dtype": "f16"}),
    ("large_f16", 6000, {}),
    ("standard", 5000, {"n_dims": 1, "n_features": 8, "log2_table_size": 12}),
    ("standard", 5000, {"n_dims": 2, "n_features": 1, "log2_table_size": 14}),
    ("standard", 5000, {"n_dims": 4, "n_features": 4, "log2_table_size": 14}),
    ("standard", 5000, {"n_features": 1, "log2_table_size": 1}),  # 2 entries x 1 feature
]


@pytest.mark.parametrize("name,n,kw", CASES)
def test_half_gradient_is_the_fp32_sum_rounded_once(oracle, name, n, kw):
    w = I.resized(I.WORKLOADS[name], n, **kw)
    print(f"binary16 gradient {name} n={n} {kw}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x_h, d_h = I.make_points(w), I.make_dout(w)
    g0 = start_values(cfg.table_shape, w.seed + 1)
    g32, g16 = both(cfg, dev(x_h), dev(d_h), g0)
    assert np.array_equal(g32.astype(np.float16).view(np.uint16), g16.view(np.uint16))
    ref = oracle.backward(oracle.grid_of(w), x_h, d_h) + g0.astype(np.float64)
    level_check(g16, ref, w.n_levels, HALF_TOL)


def test_half_gradient_in_level_groups_and_without_allocation():
    # The smallest workspace bins one level group at a time, the
    # allocation-free entry point bins in groups that fit its scratch: the
    # fixed-point sums, and so the binary16 roundings, are the same.
    w = I.resized(I.WORKLOADS["standard"], 1 << 16)
    cfg = half_cfg(hg.HashGridConfig.of(w))
    x, d = dev(I.make_points(w)), dev(I.make_dout(w))
    g0 = start_values(cfg.table_shape, 11)
    full, least = hg.hashgrid_backward_workspace_size(cfg, w.n_points)
    assert least < full
    outs = []
    for ws in (torch.empty(full, dtype=torch.uint8, device=DEV), torch.empty(least, dtype=torch.uint8, device=DEV)):
        g = dev(g0)
        hg.hashgrid_backward(cfg, x, d, g, workspace=ws)
        outs.append(g.cpu().numpy().view(np.uint16))
    g = dev(g0)
    hg.hashgrid_backward_noalloc(cfg, x, d, g)
    outs.append(g.cpu().numpy().view(np.uint16))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_mlp_backward_half_table_gradient():
    w = I.resized(I.WORKLOADS["fused_mlp"], 4096 + 5)
    cfg = hg.HashGridConfig.of(w)
    x, t = dev(I.make_points(w)), dev(I.make_table(w))
    P = [dev(a) for a in I.mlp_params(w.seed)]
    dy = dev(I.dout_normal(w.seed + 7, w.n_points, 4))
    y, stage = hg.hashgrid_mlp_forward(cfg, x, t, P)
    res = []
    for c in (cfg, half_cfg(cfg)):
        grads = [torch.zeros(hg.hashgrid.MLP_SHAPES[k], device=DEV) for k in ("w1", "b1", "w2", "b2", "w3", "b3")]
        dtable = torch.zeros(cfg.table_shape, device=DEV, dtype=c.torch_grad_dtype)
        hg.hashgrid_mlp_backward(c, x, stage, P, dy, grads, dtable)
        res.append((dtable.cpu().numpy(), [a.cpu().numpy() for a in grads]))
    assert np.array_equal(res[0][0].astype(np.float16).view(np.uint16), res[1][0].view(np.uint16))
    assert all(np.array_equal(a, b) for a, b in zip(res[0][1], res[1][1]))


@pytest.mark.parametrize("shape", [(3, 2), (2, 4), (4, 1)])
def test_half_gradient_with_nonfinite_upstream_values(oracle, shape):
    D, F = shape
    w = I.resized(I.WORKLOADS["standard"], 6000 + 17, n_dims=D, n_features=F, log2_table_size=14)
    print(f"binary16 gradient, non-finite dout D={D} F={F}", flush=True)
    cfg = half_cfg(hg.HashGridConfig.of(w))
    x, d = I.make_points(w), I.make_dout(w)
    rng = np.random.default_rng(37)
    rows = rng.choice(w.n_points, size=12, replace=False)
    cols = rng.integers(0, cfg.out_features, size=12)
    d[rows, cols] = np.array([np.nan, np.inf, -np.inf] * 4, dtype=np.float32)
    d[100, :] = np.nan
    ref = oracle.backward(oracle.grid_of(w), x, d)
    g = torch.zeros(cfg.table_shape, device=DEV, dtype=torch.float16)
    hg.hashgrid_backward(cfg, dev(x), dev(d), g, workspace="auto")
    got = g.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.array_equal(got[inf], ref[inf])
    fin = np.isfinite(ref)
    for l in range(w.n_levels):
        f = fin[l]
        scale = float(np.max(np.abs(ref[l][f])))
        assert float(np.max(np.abs(got[l][f] - ref[l][f]))) <= HALF_TOL * scale, l


def test_half_gradient_without_a_workspace_is_refused():
    w = I.resized(I.WORKLOADS["standard"], 1000)
    cfg = half_cfg(hg.HashGridConfig.of(w))
    g = torch.zeros(cfg.table_shape, device=DEV, dtype=torch.float16)
    with pytest.raises(hg.HashGridError, match="binned"):
        hg.hashgrid_backward(cfg, dev(I.make_points(w)), dev(I.make_dout(w)), g, workspace=None)
    assert not torch.any(g.view(torch.int16) != 0)


def test_half_parameter_autograd_gradient():
    # A binary16 table parameter (fp32_master=False) gets its gradient from a
    # binary16 buffer on the binned path: the same bits as the fp32 gradient
    # rounded to binary16, through the encoder and through the MLP head.
    w = I.resized(I.WORKLOADS["fused_mlp"], 3000)
    x, d = dev(I.make_points(w)), dev(I.make_dout(w))
    enc = hg.HashGridEncoder(table_dtype="f16", device=DEV, fp32_master=False)
    with torch.no_grad():
        enc.embeddings.copy_(dev(I.make_table(w)))
    enc(x).backward(d)
    got = enc.embeddings.grad
    assert got.dtype == torch.float16
    cfg = enc.cfg
    g32 = torch.zeros(cfg.table_shape, device=DEV)
    hg.hashgrid_backward(cfg, x, d, g32)
    assert torch.equal(got.view(torch.int16), g32.half().view(torch.int16))

    model = hg.HashGridMLP(device=DEV, fp32_master=False)
    with torch.no_grad():
        model.encoder.embeddings.copy_(enc.embeddings)
    dy = dev(I.dout_normal(w.seed + 7, w.n_points, 4))
    model(x).backward(dy)
    got = model.encoder.embeddings.grad
    assert got.dtype == torch.float16
    params = [model.w1.detach().half(), model.b1.detach(), model.w2.detach().half(), model.b2.detach(),
              model.w3.detach().half(), model.b3.detach()]
    y, stage = hg.hashgrid_mlp_forward(cfg, x, model.encoder.embeddings.detach(), params)
    grads = [torch.zeros(hg.hashgrid.MLP_SHAPES[k], device=DEV) for k in ("w1", "b1", "w2", "b2", "w3", "b3")]
    dt32 = torch.zeros(cfg.table_shape, device=DEV)
    hg.hashgrid_mlp_backward(cfg, x, stage, params, dy, grads, dt32)
    assert torch.equal(got.view(torch.int16), dt32.half().view(torch.int16))
