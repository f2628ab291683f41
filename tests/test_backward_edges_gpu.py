"""GPU parity of the table backward at its edges, against the CPU oracle:

  - non-finite upstream values (NaN, +-Inf) reach the entries they touch on
    both paths as IEEE arithmetic has them, and leave the other entries and
    the fixed-point scale of the binned path alone;
  - tables of 2 to 8 entries (and a level of 8 vertices) under enough points
    that an entry receives 5 * 10^4 to 2 * 10^5 additions, through the
    allocation-free path (no workspace), whose levels of at most 16384 values
    are summed exactly in LDS per workgroup before the fp32 atomics;
  - the Python binding's buffers stay owned by an explicit side stream until
    its kernels are done.
Bars as the other parity tests: <= 1e-5 * max|oracle gradient| per level.
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


def compare_nonfinite(got, ref, L):
    """NaN exactly where the oracle has NaN, the same infinities, and the
    finite entries within 1e-5 of the level's largest finite gradient."""
    got = got.astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.array_equal(got[inf], ref[inf])
    fin = np.isfinite(ref)
    for l in range(L):
        f = fin[l]
        scale = float(np.max(np.abs(ref[l][f]))) if np.any(f) else 0.0
        err = float(np.max(np.abs(got[l][f] - ref[l][f]))) if np.any(f) else 0.0
        assert err <= 1e-5 * scale, (l, err, scale)


@pytest.mark.parametrize("shape", [(3, 2), (2, 4), (4, 1)])
@pytest.mark.parametrize("workspace", ["auto", None])
def test_backward_with_nonfinite_upstream_values(oracle, shape, workspace):
    D, F = shape
    w = I.resized(I.WORKLOADS["standard"], 6000 + 17, n_dims=D, n_features=F, log2_table_size=14)
    print(f"non-finite dout D={D} F={F} workspace={workspace}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x, d = I.make_points(w), I.make_dout(w)
    rng = np.random.default_rng(31)
    rows = rng.choice(w.n_points, size=12, replace=False)
    cols = rng.integers(0, cfg.out_features, size=12)
    vals = np.array([np.nan, np.inf, -np.inf] * 4, dtype=np.float32)
    d[rows, cols] = vals
    # an Inf on a level must not coarsen that level's finite sums: one more on
    # level 0 in every row block, and a whole row of NaN
    d[7, 0] = np.inf
    d[100, :] = np.nan
    ref = oracle.backward(oracle.grid_of(w), x, d)
    g = torch.zeros(cfg.table_shape, device=DEV)
    hg.hashgrid_backward(cfg, dev(x), dev(d), g, workspace=workspace)
    compare_nonfinite(g.cpu().numpy(), ref, w.n_levels)


def test_binned_scale_ignores_infinite_values(oracle):
    # A level whose only large |dL/dout| is infinite keeps the fixed-point step
    # of its finite values: gradients of ~1e-3 stay accurate to 1e-5.
    w = I.resized(I.WORKLOADS["standard"], 3000)
    cfg = hg.HashGridConfig.of(w)
    x = I.make_points(w)
    d = (I.make_dout(w) * np.float32(1e-3)).astype(np.float32)
    d[5, :] = np.inf
    ref = oracle.backward(oracle.grid_of(w), x, d)
    g = torch.zeros(cfg.table_shape, device=DEV)
    hg.hashgrid_backward(cfg, dev(x), dev(d), g)
    compare_nonfinite(g.cpu().numpy(), ref, w.n_levels)


# D, F, L, log2T, N_min, N_max, n: every entry of the small tables receives
# n * 2^D / (T) additions or more (a level of 8 vertices: n each).
SMALL = [
    (3, 2, 3, 1, 4, 32, 20000),     # 2 entries: 8 * 10^4 additions each
    (3, 2, 2, 3, 2, 16, 50000),     # 8 entries: 5 * 10^4
    (3, 1, 2, 2, 8, 8, 30000),      # 4 entries, one feature
    (2, 4, 2, 1, 3, 9, 50000),      # D = 2: 10^5
    (4, 8, 1, 3, 2, 2, 25000),      # D = 4, F = 8: 5 * 10^4
    (3, 2, 2, 19, 1, 40, 100000),   # level 0 has 8 vertices: 10^5 additions each, vertex-indexed
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_allocation_free_backward_on_small_tables(oracle, case):
    D, F, L, log2T, nmin, nmax, n = SMALL[case]
    w = I.Workload(f"small{case}", L, F, log2T, nmin, nmax, "f32", n, "uniform", seed=5000 + case, n_dims=D)
    print(f"small table case {case}: D={D} F={F} L={L} T=2^{log2T} n={n}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x, d = I.make_points(w), I.make_dout(w)
    ref = oracle.backward(oracle.grid_of(w), x, d)
    base = np.random.default_rng(case).uniform(-1, 1, cfg.table_shape).astype(np.float32)
    for workspace in (None, "auto"):
        g = dev(base)
        hg.hashgrid_backward(cfg, dev(x), dev(d), g, workspace=workspace)
        got = g.cpu().numpy().astype(np.float64) - base
        for l in range(L):
            scale = float(np.max(np.abs(ref[l])))
            err = float(np.max(np.abs(got[l] - ref[l])))
            # + the fp32 rounding of the base the gradient is added to
            assert err <= 1e-5 * scale + 4e-7 * (1 + scale), (workspace, l, err, scale)


def test_dense_levels_switch_is_result_equivalent(oracle):
    # With the LDS summation switched off every level is scattered directly;
    # both agree with the oracle on a grid where level 0 is vertex-indexed and
    # the others are scattered.
    w = I.resized(I.WORKLOADS["standard"], 9000)
    cfg = hg.HashGridConfig.of(w)
    x, d = I.make_points(w), I.make_dout(w)
    ref = oracle.backward(oracle.grid_of(w), x, d)
    old = hg.hashgrid_tune_get(B.HG_TUNE_BWD_DENSE)
    try:
        for v in (0, 1):
            hg.hashgrid_tune(B.HG_TUNE_BWD_DENSE, v)
            g = torch.zeros(cfg.table_shape, device=DEV)
            hg.hashgrid_backward(cfg, dev(x), dev(d), g, workspace=None)
            got = g.cpu().numpy().astype(np.float64)
            for l in range(w.n_levels):
                assert np.max(np.abs(got[l] - ref[l])) <= 1e-5 * np.max(np.abs(ref[l])), (v, l)
    finally:
        hg.hashgrid_tune(B.HG_TUNE_BWD_DENSE, old)


def test_auto_buffers_survive_a_busy_side_stream(oracle):
    # The kernels run on an explicit side stream kept busy first; the wrapper's
    # "auto" workspaces and outputs are freed to torch's allocator when it
    # returns, and the current stream allocates and scribbles on memory right
    # away.  The buffers must not be handed out before the side stream is done.
    w = I.resized(I.WORKLOADS["standard"], 1 << 16)
    cfg = hg.HashGridConfig.of(w)
    x_h, t_h, d_h = I.make_points(w), I.make_table(w), I.make_dout(w)
    x, t, d = dev(x_h), dev(t_h), dev(d_h)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    big = torch.randn((4096, 4096), device=DEV)
    with torch.cuda.stream(side):
        for _ in range(20):  # several ms of work ahead of the library's kernels
            big = (big @ big).clamp_(-1, 1)
    g = torch.zeros(cfg.table_shape, device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    out = hg.hashgrid_forward(cfg, x, t, workspace="auto", stream=side)
    hg.hashgrid_backward(cfg, x, d, g, workspace="auto", stream=side)
    dx = hg.hashgrid_input_grad(cfg, x, t, d, workspace="auto", stream=side)
    # the current stream reuses whatever the allocator offers, right now
    junk = [torch.full((s,), 7, dtype=torch.uint8, device=DEV)
            for s in (hg.hashgrid_backward_workspace_size(cfg, w.n_points)[0],
                      hg.hashgrid_forward_workspace_size(cfg, w.n_points),
                      hg.hashgrid_input_grad_workspace_size(cfg, w.n_points))]
    torch.cuda.synchronize()
    del junk
    og = oracle.grid_of(w)
    assert np.max(np.abs(out.cpu().numpy() - oracle.forward(og, x_h, t_h))) <= 1e-6 * np.max(np.abs(t_h))
    ref = oracle.backward(og, x_h, d_h)
    got = g.cpu().numpy()
    for l in range(w.n_levels):
        assert np.max(np.abs(got[l] - ref[l])) <= 1e-5 * np.max(np.abs(ref[l])), l
    dref = oracle.input_grad(og, x_h, t_h, d_h)
    assert np.max(np.abs(dx.cpu().numpy() - dref)) <= 1e-5 * np.max(np.abs(dref))
