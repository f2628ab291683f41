"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: corner indices bit-exact; forward fp32 max abs error <= 1e-6 * max|table|;
backward max abs error <= 1e-5 * max|oracle gradient| per level (fp32 atomics in
unspecified order); fp16-table grids <= 1e-3 relative (and, as expected from
fp32 arithmetic on exactly widened halves, within the fp32 bound as well).
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
BWD_TOL = 1e-5
F16_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _threads(oracle):
    oracle.set_threads(min(16, os.cpu_count() or 1))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def fwd_err(out, ref, table):
    return float(np.max(np.abs(out - ref))) / float(np.max(np.abs(table.astype(np.float64))))


def bwd_check(grad, ref, L):
    for l in range(L):
        scale = float(np.max(np.abs(ref[l])))
        err = float(np.max(np.abs(grad[l].astype(np.float64) - ref[l])))
        assert err <= BWD_TOL * scale, f"level {l}: backward err {err:.3g} > {BWD_TOL} * {scale:.3g}"


def run_forward(cfg, x, t, stride=None, workspace="auto"):
    n = x.shape[0]
    if stride is None:
        return hg.hashgrid_forward(cfg, dev(x), dev(t), workspace=workspace).cpu().numpy()
    buf = torch.full((n, stride), 7.0, device=DEV)
    hg.hashgrid_forward(cfg, dev(x), dev(t), out=buf, workspace=workspace)
    return buf.cpu().numpy()


def run_backward(cfg, x, d, init=None, workspace="auto"):
    g = torch.zeros(cfg.table_shape, device=DEV) if init is None else dev(init)
    hg.hashgrid_backward(cfg, dev(x), dev(d), g, workspace=workspace)
    return g.cpu().numpy()


# ----------------------------------------------------------------------------- corners

@pytest.mark.parametrize("name,n", [("tiny", 4096), ("standard", 3 * 1024 + 37), ("ray", 2 * 256),
                                    ("large_f16", 2000)])
def test_corner_indices_bit_exact(oracle, name, n):
    w = I.resized(I.WORKLOADS[name], n)
    cfg = hg.HashGridConfig.of(w)
    x = I.make_points(w)
    idx, wt = hg.hashgrid_debug_corners(cfg, dev(x))
    ridx, rw = oracle.corners(oracle.grid_of(w), x)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ridx)
    assert np.max(np.abs(wt.cpu().numpy() - rw)) <= 2.5e-7


def test_corner_indices_out_of_domain_points(oracle):
    w = I.WORKLOADS["standard"]
    cfg = hg.HashGridConfig.of(w)
    rng = np.random.default_rng(12)
    x = rng.uniform(-3.0, 4.0, size=(3000, 3)).astype(np.float32)
    x[:3] = [[1.0, 1.0, 1.0], [0.0, 0.0, 0.0], [-0.0, 1.0, 0.5]]
    idx, _ = hg.hashgrid_debug_corners(cfg, dev(x))
    ridx, _ = oracle.corners(oracle.grid_of(w), x)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ridx)


# ----------------------------------------------------------------------------- forward

@pytest.mark.parametrize("name,n", [("tiny", None), ("standard", 3 * 1024 + 37), ("standard", None),
                                    ("ray", None)])
def test_forward_matches_oracle(oracle, name, n):
    w = I.WORKLOADS[name] if n is None else I.resized(I.WORKLOADS[name], n)
    print(f"forward parity {name} n={w.n_points}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x, t = I.make_points(w), I.make_table(w)
    out = run_forward(cfg, x, t)
    ref = oracle.forward(oracle.grid_of(w), x, t)
    assert out.shape == ref.shape
    assert fwd_err(out, ref, t) <= FWD_TOL


def test_forward_half_tables_full_size_sampled(oracle):
    w = I.WORKLOADS["large_f16"]
    print(f"forward parity large_f16 n={w.n_points} (sampled)", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x, t = I.make_points(w), I.make_table(w)
    out = run_forward(cfg, x, t)
    rows = np.random.default_rng(13).choice(w.n_points, size=20000, replace=False)
    rows[:2] = [0, w.n_points - 1]
    ref = oracle.forward(oracle.grid_of(w), x[rows], t)
    err = np.max(np.abs(out[rows] - ref))
    assert err <= F16_TOL * np.max(np.abs(ref))
    assert fwd_err(out[rows], ref, t) <= FWD_TOL


def test_standard_grid_past_the_benchmarked_batch(oracle):
    # 2^24 + 77 points on the standard grid, 64 times the benchmarked batch:
    # 16385 bin tiles (the accumulate walks 17 chunks of tiles), level-major
    # stages past 2^31 bytes, a ragged last tile.  Sampled forward rows (the
    # first and last included) and every gradient entry against the oracle.
    w = I.resized(I.WORKLOADS["standard"], (1 << 24) + 77)
    print(f"standard grid n={w.n_points}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x, t, d = I.make_points(w), I.make_table(w), I.make_dout(w)
    g = oracle.grid_of(w)
    xd = dev(x)
    out = hg.hashgrid_forward(cfg, xd, dev(t), workspace="auto")
    rows = np.random.default_rng(17).choice(w.n_points, size=20000, replace=False)
    rows[:2] = [0, w.n_points - 1]
    assert fwd_err(out[torch.from_numpy(rows).to(DEV)].cpu().numpy(), oracle.forward(g, x[rows], t), t) <= FWD_TOL
    del out
    grad = torch.zeros(cfg.table_shape, device=DEV)
    hg.hashgrid_backward(cfg, xd, dev(d), grad, workspace="auto")
    bwd_check(grad.cpu().numpy(), oracle.backward(g, x, d), w.n_levels)


@pytest.mark.parametrize("workspace", ["auto", None])
def test_forward_writes_only_its_columns_of_a_wider_row(oracle, workspace):
    w = I.resized(I.WORKLOADS["standard"], 1000)
    cfg = hg.HashGridConfig.of(w)
    x, t = I.make_points(w), I.make_table(w)
    buf = run_forward(cfg, x, t, stride=cfg.out_features + 64, workspace=workspace)
    ref = oracle.forward(oracle.grid_of(w), x, t)
    assert fwd_err(buf[:, :cfg.out_features], ref, t) <= FWD_TOL
    assert np.all(buf[:, cfg.out_features:] == 7.0)


def test_forward_vertex_points_exact(oracle):
    # Points on vertices of power-of-two levels return the table entry exactly.
    w = I.WORKLOADS["tiny"]
    cfg = hg.HashGridConfig.of(w)
    t = I.make_table(w)
    v = np.random.default_rng(14).integers(0, 33, size=(2000, 3))
    x = (v / 32.0).astype(np.float32)
    out = run_forward(cfg, x, t)
    ref = oracle.forward(oracle.grid_of(w), x, t)
    assert np.array_equal(out[:, 6:8].astype(np.float64), ref[:, 6:8])


def test_forward_out_of_domain_points(oracle):
    w = I.WORKLOADS["standard"]
    cfg = hg.HashGridConfig.of(w)
    t = I.make_table(w)
    x = np.random.default_rng(15).uniform(-2.0, 3.0, size=(5000, 3)).astype(np.float32)
    assert fwd_err(run_forward(cfg, x, t), oracle.forward(oracle.grid_of(w), x, t), t) <= FWD_TOL


@pytest.mark.parametrize("n", [1, 63, 64, 65, 1023, 1025])
@pytest.mark.parametrize("workspace", ["auto", None])
def test_forward_ragged_sizes(oracle, n, workspace):
    w = I.resized(I.WORKLOADS["standard"], n)
    cfg = hg.HashGridConfig.of(w)
    x, t = I.make_points(w), I.make_table(w)
    out = run_forward(cfg, x, t, workspace=workspace)
    assert fwd_err(out, oracle.forward(oracle.grid_of(w), x, t), t) <= FWD_TOL


def split_levels(cfg):
    """Levels the staged gather takes one table half per pass: those whose
    rows of x-vertices ((N_l + 1)^2 rows, each in an aligned block of
    next_pow2(N_l + 1) entries) can touch more than 4 MiB of table lines."""
    per_line = 128 // (8 if cfg.table_dtype == "f32" else 4)
    out = []
    for l, r in enumerate(hg.hashgrid_resolutions(cfg)):
        R = r + 1
        block = 1 << (R - 1).bit_length()
        lines = min(R * R * -(-block // per_line), max(1, cfg.table_size // per_line))
        if lines * 128 > 4 << 20:
            out.append(l)
    return out


@pytest.mark.parametrize("name,log2T", [("standard", 19), ("standard", 20), ("large_f16", 21)])
def test_forward_staged_and_direct_are_identical(oracle, name, log2T):
    # Both output paths compute every value with the same instructions, except
    # at levels whose gathers can touch more than 4 MiB of table lines (the
    # finer levels of fp32 T = 2^20 and binary16 T = 2^21 tables): the staged
    # path gathers those one table half per launch and adds the two partial
    # blends, so the paths agree to fp32 rounding there and bit for bit at the
    # other levels, and both match the oracle.
    w = I.replace(I.resized(I.WORKLOADS[name], 7777), log2_table_size=log2T)
    cfg = hg.HashGridConfig.of(w)
    x, t = I.make_points(w), I.make_table(w)
    staged = run_forward(cfg, x, t, workspace="auto")
    direct = run_forward(cfg, x, t, workspace=None)
    split = split_levels(cfg)
    whole = [c for l in range(cfg.n_levels) if l not in split for c in (2 * l, 2 * l + 1)]
    assert np.array_equal(staged[:, whole], direct[:, whole])
    assert fwd_err(staged, direct, t) <= FWD_TOL
    if log2T > 19:  # the coarse levels touch at most a few MB of the large tables and go in one pass
        assert split and min(split) >= 5
    assert np.array_equal(staged, run_forward(cfg, x, t, stride=cfg.out_features + 3)[:, :cfg.out_features])
    ref = oracle.forward(oracle.grid_of(w), x, t)
    assert fwd_err(staged, ref, t) <= FWD_TOL and fwd_err(direct, ref, t) <= FWD_TOL
    # A workspace of one stage: the second half adds into the first half's
    # stage in place instead of writing a second one; the same sums.
    one = torch.empty(cfg.table_shape[0] * x.shape[0] * 2 * 4, dtype=torch.uint8, device=DEV)
    assert np.array_equal(staged, run_forward(cfg, x, t, workspace=one))
    # Non-temporal point and output traffic (the second half's read of the first
    # half's partial blend included) does not change a bit.
    old = hg.hashgrid_tune_get(B.HG_TUNE_FWD_NT)
    try:
        hg.hashgrid_tune(B.HG_TUNE_FWD_NT, 1)
        assert np.array_equal(staged, run_forward(cfg, x, t, workspace="auto"))
        assert np.array_equal(direct, run_forward(cfg, x, t, workspace=None))
    finally:
        hg.hashgrid_tune(B.HG_TUNE_FWD_NT, old)


# ----------------------------------------------------------------------------- backward

@pytest.mark.parametrize("name,n", [("tiny", None), ("standard", 3 * 1024 + 37), ("standard", None),
                                    ("ray", None), ("large_f16", 1 << 16)])
def test_backward_matches_oracle(oracle, name, n):
    w = I.WORKLOADS[name] if n is None else I.resized(I.WORKLOADS[name], n)
    print(f"backward parity {name} n={w.n_points}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x, d = I.make_points(w), I.make_dout(w)
    grad = run_backward(cfg, x, d)
    ref = oracle.backward(oracle.grid_of(w), x, d)
    bwd_check(grad, ref, w.n_levels)


def test_backward_half_grid_full_size(oracle):
    # The large binary16 grid at its full size (2^21 points, 32 levels, 2^21
    # entries per level), in the launch configuration the benchmark times:
    # every entry of every level against the oracle, and the per-level sums
    # against the upstream column sums (a point's weights sum to one).
    w = I.WORKLOADS["large_f16"]
    print(f"backward parity large_f16 n={w.n_points} (every entry)", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x_h, d_h = I.make_points(w), I.make_dout(w)
    x, d = dev(x_h), dev(d_h)
    g = torch.zeros(cfg.table_shape, device=DEV)
    hg.hashgrid_backward(cfg, x, d, g, workspace=hg.backward_workspace(cfg, w.n_points, DEV))
    got = g.double().sum(dim=1)
    want = d.double().reshape(-1, w.n_levels, 2).sum(dim=0)
    scale = d.double().abs().reshape(-1, w.n_levels, 2).sum(dim=0)
    assert float(((got - want).abs() / scale).max()) < 1e-6
    grad = g.cpu().numpy()
    del g, x, d
    bwd_check(grad, oracle.backward(oracle.grid_of(w), x_h, d_h), w.n_levels)


def test_backward_exact_dyadic_case(oracle):
    # Dyadic points on power-of-two levels and dout in {-1, 0, 1}: every partial
    # sum is exact in fp32, so the atomic order cannot matter and the result is
    # bit-exact.
    w = I.WORKLOADS["tiny"]
    cfg = hg.HashGridConfig.of(w)
    rng = np.random.default_rng(16)
    x = (rng.integers(0, 128, size=(4096, 3)) / 128.0).astype(np.float32)
    d = rng.integers(-1, 2, size=(4096, 8)).astype(np.float32)
    grad = run_backward(cfg, x, d)
    ref = oracle.backward(oracle.grid_of(w), x, d)
    assert np.array_equal(grad.astype(np.float64), ref)


def runs_of_points(seed, n, max_run=100, jitter=2e-4):
    # Consecutive points that share a voxel at the coarse levels, as ray samples
    # do: runs of 1..max_run points around one base point each, and one run of
    # 200 identical points in the middle.
    rng = np.random.default_rng(seed)
    x = np.empty((n, 3), dtype=np.float64)
    i = 0
    while i < n:
        m = min(int(rng.integers(1, max_run + 1)), n - i)
        x[i:i + m] = rng.uniform(0.01, 0.99, 3) + rng.uniform(-jitter, jitter, (m, 3))
        i += m
    mid = n // 2
    x[mid:mid + 200] = x[mid]
    return np.clip(x, 0.0, 0.999).astype(np.float32)


@pytest.mark.parametrize("name,n", [("standard", 3 * 1024 + 37), ("standard", 4096), ("tiny", 2 * 512 + 63)])
def test_backward_runs_of_points_in_one_voxel(oracle, name, n):
    # Runs of consecutive points in one voxel are summed inside the wave before
    # they become records: runs crossing wave and tile boundaries and the ragged
    # end, runs of identical points whose sums exceed max|dL/dout| many times,
    # and the one-partition table of the tiny grid.
    w = I.resized(I.WORKLOADS[name], n)
    print(f"backward runs {name} n={n}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    x, d = runs_of_points(n, n), I.make_dout(w)
    ref = oracle.backward(oracle.grid_of(w), x, d)
    bwd_check(run_backward(cfg, x, d), ref, w.n_levels)
    old = hg.hashgrid_tune_get(B.HG_TUNE_BWD_LANES)
    try:
        for lanes in (1, 2, 4):  # the atomic kernels; one lane per point pre-reduces the runs
            hg.hashgrid_tune(B.HG_TUNE_BWD_LANES, lanes)
            bwd_check(run_backward(cfg, x, d, workspace=None), ref, w.n_levels)
    finally:
        hg.hashgrid_tune(B.HG_TUNE_BWD_LANES, old)


@pytest.mark.parametrize("name,kw", [
    # the largest table the binned backward takes: 2^25 / 2^13 = 4096 partitions, resolution 2^20
    ("max_binned_table", dict(n_levels=1, log2_table_size=25, base_resolution=1 << 20, finest_resolution=1 << 20)),
    # the same 4096 partitions for F = 4 and F = 8 (2^11- and 2^10-entry partitions), whose
    # 48 and 40 KB record stages sit next to 32 KB of run counters
    ("max_binned_table_f4", dict(n_levels=1, n_dims=2, n_features=4, log2_table_size=23, base_resolution=1 << 12,
                                 finest_resolution=1 << 12)),
    ("max_binned_table_f8", dict(n_levels=1, n_dims=4, n_features=8, log2_table_size=22, base_resolution=64,
                                 finest_resolution=64)),
    # past it (8192 partitions): the atomic path only
    ("beyond_binned_table", dict(n_levels=1, log2_table_size=26, base_resolution=1 << 12, finest_resolution=1 << 12)),
    # the most levels, up to resolution 2^23
    ("max_levels", dict(n_levels=64, log2_table_size=10, base_resolution=2, finest_resolution=1 << 23)),
])
def test_limit_configurations_match_oracle(oracle, name, kw):
    w = I.resized(I.WORKLOADS["standard"], 2000 + 37, **kw)
    print(f"limits {name}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    g = oracle.grid_of(w)
    x, t, d = I.make_points(w), I.make_table(w), I.make_dout(w)
    assert fwd_err(run_forward(cfg, x, t), oracle.forward(g, x, t), t) <= FWD_TOL
    full, _ = hg.hashgrid_backward_workspace_size(cfg, w.n_points)
    assert (full > 0) == (name != "beyond_binned_table")
    ref = oracle.backward(g, x, d)
    bwd_check(run_backward(cfg, x, d), ref, w.n_levels)
    bwd_check(run_backward(cfg, x, d, workspace=None), ref, w.n_levels)
    idx, _ = hg.hashgrid_debug_corners(cfg, dev(x))
    ridx, _ = oracle.corners(g, x)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ridx)


@pytest.mark.parametrize("name", ["standard", "ray"])
def test_backward_binned_is_reproducible(name):
    # Fixed-point accumulation: the binned gradient does not depend on the
    # order in which workgroups add their records, so two runs agree bit for bit.
    w = I.WORKLOADS[name]
    cfg = hg.HashGridConfig.of(w)
    x, d = dev(I.make_points(w)), dev(I.make_dout(w))
    ws = hg.backward_workspace(cfg, w.n_points, DEV)
    runs = []
    for _ in range(2):
        g = torch.zeros(cfg.table_shape, device=DEV)
        hg.hashgrid_backward(cfg, x, d, g, workspace=ws)
        runs.append(g.cpu().numpy())
    assert np.array_equal(runs[0], runs[1])


def test_backward_accumulates_and_reads_strided_rows(oracle):
    w = I.resized(I.WORKLOADS["standard"], 2000)
    cfg = hg.HashGridConfig.of(w)
    x, d = I.make_points(w), I.make_dout(w)
    wide = np.concatenate([d, np.full((2000, 3), 1e30, dtype=np.float32)], axis=1)
    base = np.random.default_rng(17).standard_normal(cfg.table_shape).astype(np.float32)
    grad = run_backward(cfg, x, wide, init=base)
    ref = oracle.backward(oracle.grid_of(w), x, d, base.astype(np.float64))
    delta = oracle.backward(oracle.grid_of(w), x, d)
    for l in range(w.n_levels):
        err = np.max(np.abs(grad[l] - ref[l]))
        assert err <= BWD_TOL * np.max(np.abs(delta[l])) + 4e-7 * np.max(np.abs(base[l]))


@pytest.mark.parametrize("name,n", [("standard", 3 * 1024 + 37), ("tiny", None)])
def test_backward_atomic_path_matches_oracle(oracle, name, n):
    # No workspace: the fp32 global-atomic scatter.
    w = I.WORKLOADS[name] if n is None else I.resized(I.WORKLOADS[name], n)
    cfg = hg.HashGridConfig.of(w)
    x, d = I.make_points(w), I.make_dout(w)
    bwd_check(run_backward(cfg, x, d, workspace=None), oracle.backward(oracle.grid_of(w), x, d), w.n_levels)


@pytest.mark.parametrize("levels_per_pass", [1, 3, 16])
def test_backward_binned_in_level_groups(oracle, levels_per_pass):
    # A workspace for fewer levels than L: the library processes level groups.
    w = I.resized(I.WORKLOADS["standard"], 4 * 512 + 300)
    cfg = hg.HashGridConfig.of(w)
    x, d = I.make_points(w), I.make_dout(w)
    full, least = hg.hashgrid_backward_workspace_size(cfg, w.n_points)
    ws = torch.empty(least * levels_per_pass + 100, dtype=torch.uint8, device=DEV)
    grad = run_backward(cfg, x, d, workspace=ws)
    bwd_check(grad, oracle.backward(oracle.grid_of(w), x, d), w.n_levels)


def test_backward_binned_split_corner_pairs(oracle):
    # Negative coordinates make x = -1 corners whose x+1 neighbour lies in another
    # table partition: those pairs take the split path.
    w = I.WORKLOADS["standard"]
    cfg = hg.HashGridConfig.of(w)
    rng = np.random.default_rng(18)
    x = rng.uniform(-0.02, 0.02, size=(6000, 3)).astype(np.float32)
    d = rng.standard_normal((6000, 32)).astype(np.float32)
    bwd_check(run_backward(cfg, x, d), oracle.backward(oracle.grid_of(w), x, d), w.n_levels)


def test_backward_binned_reused_workspace_and_dirty_contents(oracle):
    w = I.resized(I.WORKLOADS["standard"], 5000)
    cfg = hg.HashGridConfig.of(w)
    x, d = I.make_points(w), I.make_dout(w)
    full, _ = hg.hashgrid_backward_workspace_size(cfg, w.n_points)
    ws = torch.full((full,), 0xA5, dtype=torch.uint8, device=DEV)
    g1 = run_backward(cfg, x, d, workspace=ws)
    x2 = x[:3001].copy()
    d2 = d[:3001].copy()
    g2 = run_backward(cfg, x2, d2, workspace=ws)
    ref1 = oracle.backward(oracle.grid_of(w), x, d)
    ref2 = oracle.backward(oracle.grid_of(w), x2, d2)
    bwd_check(g1, ref1, w.n_levels)
    bwd_check(g2, ref2, w.n_levels)


# ----------------------------------------------------------------------------- launch shapes

@pytest.mark.parametrize("key,value", [(B.HG_TUNE_FWD_LANES, 1), (B.HG_TUNE_BWD_LANES, 1),
                                       (B.HG_TUNE_BWD_LANES, 2), (B.HG_TUNE_XCD_MAP, 0),
                                       (B.HG_TUNE_CHUNK_POINTS, 64), (B.HG_TUNE_CHUNK_POINTS, 8192),
                                       (B.HG_TUNE_BWD_BINNED, 0), (B.HG_TUNE_FWD_UNROLL, 2),
                                       (B.HG_TUNE_FWD_UNROLL, 4), (B.HG_TUNE_FWD_NT, 1),
                                       (B.HG_TUNE_BWD_PART_LOG2, 11), (B.HG_TUNE_BWD_PART_LOG2, 12),
                                       (B.HG_TUNE_BWD_GROUP_MIB, 0), (B.HG_TUNE_BWD_GROUP_MIB, 3)])
def test_launch_variants_match_oracle(oracle, key, value):
    # (GROUP_MIB, 3): 270 KB of records per level at this n, so 3 MiB holds 11
    # levels (1408 accumulate workgroups): two groups of 8; 0: one group.
    w = I.resized(I.WORKLOADS["standard"], 5 * 1024 + 77)
    cfg = hg.HashGridConfig.of(w)
    x, t, d = I.make_points(w), I.make_table(w), I.make_dout(w)
    old = hg.hashgrid_tune_get(key)
    try:
        hg.hashgrid_tune(key, value)
        out = run_forward(cfg, x, t)
        grad = run_backward(cfg, x, d)
    finally:
        hg.hashgrid_tune(key, old)
    g = oracle.grid_of(w)
    assert fwd_err(out, oracle.forward(g, x, t), t) <= FWD_TOL
    bwd_check(grad, oracle.backward(g, x, d), w.n_levels)


@pytest.mark.parametrize("key,value", [(B.HG_TUNE_CHUNK_POINTS, 64), (B.HG_TUNE_CHUNK_POINTS, 8192),
                                       (B.HG_TUNE_XCD_MAP, 0), (B.HG_TUNE_FWD_UNROLL, 1), (B.HG_TUNE_FWD_NT, 1),
                                       (B.HG_TUNE_FWD_STAGED, 0), (B.HG_TUNE_BWD_PART_LOG2, 11),
                                       (B.HG_TUNE_BWD_PART_LOG2, 13), (B.HG_TUNE_BWD_GROUP_MIB, 0),
                                       (B.HG_TUNE_BWD_GROUP_MIB, 3), (B.HG_TUNE_FWD_DENSE, 2),
                                       (B.HG_TUNE_FWD_ORDER, 2)])
def test_result_neutral_knobs_give_identical_results(key, value):
    # The launch shapes that the header documents as result-neutral reproduce
    # the default's forward and binned backward bit for bit.
    w = I.resized(I.WORKLOADS["standard"], 5 * 1024 + 77)
    cfg = hg.HashGridConfig.of(w)
    x, t, d = I.make_points(w), I.make_table(w), I.make_dout(w)
    ref_out, ref_grad = run_forward(cfg, x, t), run_backward(cfg, x, d)
    old = hg.hashgrid_tune_get(key)
    try:
        hg.hashgrid_tune(key, value)
        out, grad = run_forward(cfg, x, t), run_backward(cfg, x, d)
    finally:
        hg.hashgrid_tune(key, old)
    assert np.array_equal(out, ref_out) and np.array_equal(grad, ref_grad)


# ----------------------------------------------------------------------------- graph capture

@pytest.mark.parametrize("workspace", ["binned", "atomic"])
def test_step_captured_in_a_graph_replays_like_eager(workspace):
    # The library allocates nothing, never synchronises and issues no memsets,
    # so a forward + backward can be captured in a HIP graph.  Every replay,
    # with eager work and synchronisations in between, matches the eager result:
    # bit for bit on the binned path (fixed-point sums), to fp32 rounding on the
    # atomic path (its additions happen in an unspecified order).
    w = I.resized(I.WORKLOADS["standard"], 1 << 16)
    cfg = hg.HashGridConfig.of(w)
    x, t, d = dev(I.make_points(w)), dev(I.make_table(w)), dev(I.make_dout(w))
    out = torch.empty((w.n_points, cfg.out_features), device=DEV)
    grad = torch.zeros(cfg.table_shape, device=DEV)
    ws = hg.backward_workspace(cfg, w.n_points, DEV) if workspace == "binned" else None
    fws = hg.forward_workspace(cfg, w.n_points, DEV)

    def step():
        hg.hashgrid_forward(cfg, x, t, out=out, workspace=fws)
        hg.hashgrid_backward(cfg, x, d, grad, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_grad = out.clone(), grad.clone()
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
        grad.zero_()
        out.fill_(-1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        if workspace == "binned":
            assert torch.equal(grad, ref_grad)
        else:
            scale = float(ref_grad.abs().max())
            assert float((grad - ref_grad).abs().max()) <= 1e-6 * scale


@pytest.mark.parametrize("coords", [0, 3])
def test_head_input_grad_and_adam_captured_in_a_graph_replay_like_eager(coords):
    # The other entry points under graph capture: encoder + MLP head forward and
    # backward (the NeRFace head, or with coords = 3 the TinyNeRF head), dL/dx
    # and the Adam step, with every buffer (stages, workspaces) allocated
    # before capture.  Each replay starts from the same state, set by eager
    # copies between replays, and matches the eager step bit for bit: the
    # binned table sums are exact and the weight gradients are reduced in a
    # fixed order.
    w = I.resized(I.WORKLOADS["fused_mlp"], 1 << 14)
    cfg = hg.HashGridConfig.of(w)
    n = w.n_points
    x, t = dev(I.make_points(w)), dev(I.make_table(w))
    P = [dev(a) for a in I.mlp_params(w.seed, sizes=(32 + coords, 64, 64, 4))]
    dy = dev(I.dout_normal(w.seed + 7, n, 4))
    st_bytes, bw_bytes = hg.hashgrid_mlp_workspace_size(cfg, n)
    stage = torch.empty(st_bytes, dtype=torch.uint8, device=DEV)
    mws = torch.empty(bw_bytes, dtype=torch.uint8, device=DEV)
    y = torch.empty((n, 4), device=DEV)
    grads = [torch.zeros(a.shape, device=DEV) for a in P]
    dtable = torch.zeros(cfg.table_shape, device=DEV)
    ws = I.resized(I.WORKLOADS["standard"], n)
    scfg = hg.HashGridConfig.of(ws)
    st, sd = dev(I.make_table(ws)), dev(I.make_dout(ws))
    iws = torch.empty(hg.hashgrid_input_grad_workspace_size(scfg, n), dtype=torch.uint8, device=DEV)
    dx = torch.empty((n, 3), device=DEV)
    p0 = torch.from_numpy(np.random.default_rng(3).uniform(-1, 1, 1 << 16).astype(np.float32)).to(DEV)
    g0 = torch.from_numpy(np.random.default_rng(4).normal(size=1 << 16).astype(np.float32)).to(DEV)
    param, m, v, gr = p0.clone(), torch.zeros_like(p0), torch.zeros_like(p0), g0.clone()

    def reset():
        for a in grads:
            a.zero_()
        dtable.zero_()
        y.fill_(-1.0)
        dx.fill_(-1.0)
        param.copy_(p0)
        m.zero_()
        v.zero_()
        gr.copy_(g0)

    def step():
        hg.hashgrid_mlp_forward(cfg, x, t, P, y=y, stage=stage)
        hg.hashgrid_mlp_backward(cfg, x, stage, P, dy, grads, dtable, workspace=mws)
        hg.hashgrid_input_grad(scfg, x, st, sd, dx=dx, workspace=iws)
        hg.hashgrid_adam_step(param, m, v, gr, lr=1e-2, step=1)

    reset()
    step()
    torch.cuda.synchronize()
    ref = [y.clone(), dtable.clone(), dx.clone(), param.clone(), m.clone(), v.clone()] + [a.clone() for a in grads]
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
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [y, dtable, dx, param, m, v] + grads
        for name, a, b in zip(("y", "dtable", "dx", "param", "m", "v", "dw1", "db1", "dw2", "db2", "dw3", "db3"),
                              got, ref):
            assert torch.equal(a, b), name


def test_concurrent_calls_from_host_threads_on_their_own_streams():
    # The library keeps no per-call state (the last error is thread-local), so
    # host threads may call it at once, each on its own stream with its own
    # buffers and workspaces: every thread's forward and binned backward equal
    # the single-threaded results bit for bit.
    import threading
    w = I.resized(I.WORKLOADS["standard"], 20000 + 13)
    cfg = hg.HashGridConfig.of(w)
    x, t, d = dev(I.make_points(w)), dev(I.make_table(w)), dev(I.make_dout(w))
    ref_out = hg.hashgrid_forward(cfg, x, t)
    ref_grad = torch.zeros(cfg.table_shape, device=DEV)
    hg.hashgrid_backward(cfg, x, d, ref_grad)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(k):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                out = torch.empty_like(ref_out)
                grad = torch.zeros_like(ref_grad)
                fws = hg.forward_workspace(cfg, w.n_points, DEV)
                bws = hg.backward_workspace(cfg, w.n_points, DEV)
                for _ in range(5):
                    grad.zero_()
                    hg.hashgrid_forward(cfg, x, t, out=out, workspace=fws)
                    hg.hashgrid_backward(cfg, x, d, grad, workspace=bws)
            stream.synchronize()
            results[k] = (out, grad)
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for k in range(4):
        out, grad = results[k]
        assert torch.equal(out, ref_out), k
        assert torch.equal(grad, ref_grad), k


# ----------------------------------------------------------------------------- module

def test_encoder_module_autograd(oracle):
    w = I.resized(I.WORKLOADS["standard"], 3000)
    enc = hg.HashGridEncoder(device=DEV)
    t = I.make_table(w)
    with torch.no_grad():
        enc.embeddings.copy_(dev(t))
    x = I.make_points(w)
    d = I.make_dout(w)
    out = enc(dev(x))
    out.backward(dev(d))
    g = oracle.grid_of(w)
    assert fwd_err(out.detach().cpu().numpy(), oracle.forward(g, x, t), t) <= FWD_TOL
    bwd_check(enc.embeddings.grad.cpu().numpy(), oracle.backward(g, x, d), w.n_levels)


def test_half_table_module_keeps_fp32_gradients(oracle):
    # A binary16-table encoder keeps an fp32 master parameter by default: the
    # kernels read its binary16 copy, and gradients far below binary16's range
    # (upstream values of 1e-6) reach the parameter unrounded.
    w = I.resized(I.WORKLOADS["large_f16"], 3000, n_levels=4, log2_table_size=14)
    enc = hg.HashGridEncoder(n_levels=4, log2_hashmap_size=14, finest_resolution=4096, table_dtype="f16",
                             device=DEV)
    assert enc.embeddings.dtype == torch.float32
    t16 = I.make_table(w)  # binary16 values
    with torch.no_grad():
        enc.embeddings.copy_(dev(t16.astype(np.float32)))
    x = I.make_points(w)
    d = (I.make_dout(w) * np.float32(1e-6)).astype(np.float32)
    out = enc(dev(x))
    out.backward(dev(d))
    g = oracle.grid_of(w)
    assert fwd_err(out.detach().cpu().numpy(), oracle.forward(g, x, t16), t16) <= FWD_TOL
    got = enc.embeddings.grad
    assert got.dtype == torch.float32
    bwd_check(got.cpu().numpy(), oracle.backward(g, x, d), w.n_levels)
