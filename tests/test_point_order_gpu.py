"""GPU parity of the staged forward's point order.

The staged forward of the D = 3, F = 2 grid may encode the points in the
order of a coarse cell (16^3 cells) and write each row back to its point's
position.  Every row is computed from its own point alone, so the output must
not change by a bit between the ordered path (HG_TUNE_FWD_ORDER = 2, taken at
any batch size) and the caller's order (0): over one and many groups of the
counting sort (4096 points each) with ragged last groups, binary16 tables,
tables gathered one half per pass (two stages), levels blended from LDS,
output rows with a stride, points outside the unit cube and non-finite
coordinates (which the sort puts in the nearest or first cell; the rows of
non-finite points are NaN on both paths, and as the pages leave such points
undefined only that is compared, not the NaNs' bits), a workspace
too small for the order (the caller's order then), and a forward captured in
a HIP graph and replayed.  One case is also held to the oracle.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import multiresolution_hash_grid_amd as hg  # noqa: E402
from multiresolution_hash_grid_amd import hashgrid as B  # noqa: E402
from multiresolution_hash_grid_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _threads(oracle):
    oracle.set_threads(min(16, os.cpu_count() or 1))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


class tuned:
    """Set tuning knobs for a block and restore them after."""

    def __init__(self, **kv):
        self.kv = {getattr(B, k): v for k, v in kv.items()}

    def __enter__(self):
        self.old = {k: hg.hashgrid_tune_get(k) for k in self.kv}
        for k, v in self.kv.items():
            hg.hashgrid_tune(k, v)

    def __exit__(self, *exc):
        for k, v in self.old.items():
            hg.hashgrid_tune(k, v)


def forward(cfg, x, t, order, stride=None, workspace="auto", **knobs):
    with tuned(HG_TUNE_FWD_ORDER=order, **knobs):
        n = x.shape[0]
        out = torch.full((n, stride or cfg.out_features), 7.0, device=DEV)
        hg.hashgrid_forward(cfg, dev(x), dev(t), out=out, workspace=workspace)
        return out.cpu().numpy()


def same_bits(a, b):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


def odd_points(w, seed=7):
    """The workload's points with some coordinates moved onto the faces of the
    cube, outside it and to non-finite values."""
    x = I.make_points(w).copy()
    rng = np.random.default_rng(seed)
    vals = np.array([0.0, 1.0, -0.0, -0.3, 1.7, -2.5, 3.25, np.inf, -np.inf, np.nan], dtype=np.float32)
    pick = rng.random(x.shape) < 0.02
    x[pick] = rng.choice(vals, size=int(pick.sum()))
    return x


CASES = [
    # name, points, overrides
    ("standard", 1, {}),
    ("standard", 4095, {}),
    ("standard", 4097, {}),
    ("standard", 3 * 4096 + 77, {}),
    ("standard", 70000, {"table_dtype": "f16"}),
    ("large_f16", 9000, {}),   # levels above 4 MiB gathered one half per pass: two stages
    ("ray", 4 * 256, {}),
]


@pytest.mark.parametrize("name,n,kw", CASES)
def test_ordered_forward_is_bit_identical(name, n, kw):
    w = I.replace(I.resized(I.WORKLOADS[name], n), **kw)
    print(f"point order {name} n={w.n_points} {kw}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x, t = I.make_points(w), I.make_table(w)
    ref = forward(cfg, x, t, 0)
    assert same_bits(forward(cfg, x, t, 2), ref)
    wide = forward(cfg, x, t, 2, stride=cfg.out_features + 5)
    assert same_bits(wide[:, :cfg.out_features], ref) and np.all(wide[:, cfg.out_features:] == 7.0)


def test_ordered_forward_with_lds_levels_and_odd_points(oracle):
    w = I.resized(I.WORKLOADS["standard"], 5 * 4096 + 3)
    cfg = hg.HashGridConfig.of(w)
    x, t = odd_points(w), I.make_table(w)
    fin = np.all(np.isfinite(x), axis=1)
    assert 0 < int(np.sum(~fin)) < len(x)
    ref = forward(cfg, x, t, 0, HG_TUNE_FWD_DENSE=0)
    assert np.all(np.isnan(ref[~fin]))
    for dense in (0, 2):
        got = forward(cfg, x, t, 2, HG_TUNE_FWD_DENSE=dense)
        assert same_bits(got[fin], ref[fin]), dense
        assert np.all(np.isnan(got[~fin])), dense
    want = oracle.forward(oracle.grid_of(w), x[fin], t)
    assert float(np.max(np.abs(ref[fin] - want))) <= 1e-6 * float(np.max(np.abs(t.astype(np.float64))))


def test_workspace_without_room_for_the_order():
    # A workspace sized with the order switched off holds the stage alone: the
    # forward then encodes the points in the caller's order.
    w = I.resized(I.WORKLOADS["standard"], 1 << 17)
    cfg = hg.HashGridConfig.of(w)
    x, t = I.make_points(w), I.make_table(w)
    with tuned(HG_TUNE_FWD_ORDER=0):
        small = hg.forward_workspace(cfg, w.n_points, DEV)
    with tuned(HG_TUNE_FWD_ORDER=2):
        big = hg.forward_workspace(cfg, w.n_points, DEV)
    assert big.numel() > small.numel()
    ref = forward(cfg, x, t, 0)
    for ws in (small, big):
        assert same_bits(forward(cfg, x, t, 2, workspace=ws), ref)


def test_ordered_forward_captured_in_a_graph():
    w = I.resized(I.WORKLOADS["standard"], 1 << 16)
    cfg = hg.HashGridConfig.of(w)
    n = w.n_points
    x, t = dev(I.make_points(w)), dev(I.make_table(w))
    out = torch.empty((n, cfg.out_features), device=DEV)
    with tuned(HG_TUNE_FWD_ORDER=2):
        ws = hg.forward_workspace(cfg, n, DEV)
        hg.hashgrid_forward(cfg, x, t, out=out, workspace=ws)
        torch.cuda.synchronize()
        ref = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            hg.hashgrid_forward(cfg, x, t, out=out, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            hg.hashgrid_forward(cfg, x, t, out=out, workspace=ws)
        for _ in range(3):
            out.fill_(-1.0)
            ws.fill_(0xFF)  # the order's tables and the stage are rebuilt by every replay
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
