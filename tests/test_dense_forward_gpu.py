"""GPU parity of the staged forward's LDS-blended levels.

Coarse levels whose vertex grids (N_l + 1)^3, or whole tables, fit the
kernel's LDS budget together are blended from a copy in LDS; the gather takes
the other levels.  The two kernels add the same fp32 terms in the same order,
so the forward must not change by a bit between the LDS path taken at any
batch size (HG_TUNE_FWD_DENSE = 2; by default it starts at 2^21 points) and
switched off (0), on every kind of level it takes: by vertex (fp32 and
binary16 tables), by table (tables smaller than the vertex grid), for points
on the far faces of the unit cube and outside it (their corners leave the
grid and are read from the table), with row strides, and through the MLP
head's binary16 stage.  Where tables above 4 MiB are gathered one half per
pass (whose two partial blends round differently from one pass), the LDS
levels equal the one-pass direct path bit for bit instead, and the whole
output stays within the forward bar of the all-gather result.  Each case is
also held to the oracle.
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
FWD_TOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _threads(oracle):
    oracle.set_threads(min(16, os.cpu_count() or 1))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def forward(cfg, x, t, dense, stride=None):
    old = hg.hashgrid_tune_get(B.HG_TUNE_FWD_DENSE)
    try:
        hg.hashgrid_tune(B.HG_TUNE_FWD_DENSE, dense)
        n = x.shape[0]
        out = torch.full((n, stride or cfg.out_features), 7.0, device=DEV)
        hg.hashgrid_forward(cfg, dev(x), dev(t), out=out, workspace="auto")
        return out.cpu().numpy()
    finally:
        hg.hashgrid_tune(B.HG_TUNE_FWD_DENSE, old)


def edge_points(w, seed=5):
    """The workload's points with some coordinates moved onto the far faces
    (x = 1: the voxel's upper corners lie past the grid), just below them,
    onto 0, and outside [0, 1)."""
    x = I.make_points(w).copy()
    rng = np.random.default_rng(seed)
    vals = np.array([1.0, np.nextafter(np.float32(1.0), np.float32(0.0)), 0.0, -0.3, 1.7, -2.5, 3.25],
                    dtype=np.float32)
    pick = rng.random(x.shape) < 0.05
    x[pick] = rng.choice(vals, size=int(pick.sum()))
    return x


CASES = [
    # name, points, overrides: by-vertex fp32 (levels 0 and 1), binary16 (levels 0 to 2),
    # by-table (T = 2^10 holds fewer entries than the vertex grids: levels 0 to 15), tables
    # gathered one half per pass next to LDS levels (binary16 T = 2^21), one point
    ("standard", 3 * 4096 + 77, {}),
    ("standard", 5000, {"table_dtype": "f16"}),
    ("tiny", 4096 + 5, {}),
    ("standard", 20000, {"log2_table_size": 10}),
    ("large_f16", 6000, {}),
    ("standard", 1, {}),
]


def lds_levels(cfg):
    """Levels the LDS path takes: from the coarsest up, vertex grids or tables
    whose entries fit 128 KiB together."""
    esize = 8 if cfg.table_dtype == "f32" else 4
    room, out = (128 << 10) // esize, []
    for l, r in enumerate(hg.hashgrid_resolutions(cfg)):
        entries = min(cfg.table_size, (r + 1) ** 3)
        if entries <= room:
            room -= entries
            out.append(l)
    return out


@pytest.mark.parametrize("name,n,kw", CASES)
def test_lds_levels_match_the_gather_bit_for_bit(oracle, name, n, kw):
    w = I.replace(I.resized(I.WORKLOADS[name], n), **kw)
    print(f"dense forward {name} n={n} {kw}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x, t = edge_points(w), I.make_table(w)
    got = forward(cfg, x, t, 2)
    dense = lds_levels(cfg)
    assert dense, "the case must exercise the LDS path"
    gathered = forward(cfg, x, t, 0)
    if cfg.table_size * (8 if cfg.table_dtype == "f32" else 4) > (4 << 20):  # halves per pass
        direct = hg.hashgrid_forward(cfg, dev(x), dev(t), workspace=None).cpu().numpy()
        cols = [2 * l + j for l in dense for j in range(2)]
        assert np.array_equal(got[:, cols], direct[:, cols])
        scale = float(np.max(np.abs(t.astype(np.float64))))
        assert float(np.max(np.abs(got - gathered))) <= FWD_TOL * scale
    else:
        assert np.array_equal(got, gathered)
    wide = forward(cfg, x, t, 2, stride=cfg.out_features + 5)
    assert np.array_equal(wide[:, :cfg.out_features], got) and np.all(wide[:, cfg.out_features:] == 7.0)
    ref = oracle.forward(oracle.grid_of(w), x, t)
    scale = float(np.max(np.abs(t.astype(np.float64))))
    assert float(np.max(np.abs(got - ref))) <= FWD_TOL * scale


@pytest.mark.parametrize("n", [4097, 1 << 16])
def test_mlp_stage_lds_levels_match_the_gather(n):
    w = I.resized(I.WORKLOADS["fused_mlp"], n)
    cfg = hg.HashGridConfig.of(w)
    x, t = dev(edge_points(w)), dev(I.make_table(w))
    P = [dev(a) for a in I.mlp_params(w.seed)]
    old = hg.hashgrid_tune_get(B.HG_TUNE_FWD_DENSE)
    res = []
    try:
        for dense in (2, 0):
            hg.hashgrid_tune(B.HG_TUNE_FWD_DENSE, dense)
            y, stage = hg.hashgrid_mlp_forward(cfg, x, t, P)
            res.append((y.cpu().numpy(), stage[: n * 64].cpu().numpy()))
    finally:
        hg.hashgrid_tune(B.HG_TUNE_FWD_DENSE, old)
    assert np.array_equal(res[0][1], res[1][1])
    assert np.array_equal(res[0][0], res[1][0])


def test_lds_levels_captured_in_a_graph_replay_like_eager():
    # The LDS path under HIP graph capture (its launcher sets the kernel's LDS
    # size attribute on every call): the staged forward and the MLP head's
    # stage, captured once and replayed with eager work in between, match the
    # eager results bit for bit.
    w = I.resized(I.WORKLOADS["fused_mlp"], 1 << 14)
    cfg = hg.HashGridConfig.of(w)
    n = w.n_points
    x, t = dev(I.make_points(w)), dev(I.make_table(w))
    P = [dev(a) for a in I.mlp_params(w.seed)]
    st_bytes, _ = hg.hashgrid_mlp_workspace_size(cfg, n)
    stage = torch.empty(st_bytes, dtype=torch.uint8, device=DEV)
    y = torch.empty((n, 4), device=DEV)
    out = torch.empty((n, cfg.out_features), device=DEV)
    fws = hg.forward_workspace(cfg, n, DEV)
    old = hg.hashgrid_tune_get(B.HG_TUNE_FWD_DENSE)
    try:
        hg.hashgrid_tune(B.HG_TUNE_FWD_DENSE, 2)

        def step():
            hg.hashgrid_forward(cfg, x, t, out=out, workspace=fws)
            hg.hashgrid_mlp_forward(cfg, x, t, P, y=y, stage=stage)

        step()
        torch.cuda.synchronize()
        ref_out, ref_y = out.clone(), y.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            out.fill_(-1.0)
            y.fill_(-1.0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out) and torch.equal(y, ref_y)
    finally:
        hg.hashgrid_tune(B.HG_TUNE_FWD_DENSE, old)
