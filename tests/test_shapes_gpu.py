"""GPU parity of the other grid shapes (input dimension D in 1..4, F in
{1, 2, 4, 8} features per entry; jsqmd.com HashEncoding sections 3 and 4)
and of the gradient with respect to the points, against the CPU oracle.

Bars as for the standard grid: corner indices bit-exact; forward
<= 1e-6 * max|table| (fp32; fp16 tables are widened exactly, so the same bar
holds and the 1e-3 relative bound with it); backward <= 1e-5 * max|oracle
gradient| per level.  dL/dx (not bounded on the pages): its fp32 sum of
2^D signed products per level rounds to ~1e-7 of the sum of their
magnitudes, which for these tables is within a few times |dL/dx|, so the
bar is <= 1e-5 * max|oracle dL/dx| per coordinate."""
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


def shape_workload(D, F, dtype, n=3 * 1024 + 77, L=8, log2T=14, nmin=4, nmax=128):
    return I.Workload(f"d{D}f{F}{dtype}", L, F, log2T, nmin, nmax, dtype, n, "uniform",
                      seed=2000 + 10 * D + F, n_dims=D)


SHAPES = [(1, 2, "f32"), (2, 1, "f32"), (2, 2, "f16"), (2, 4, "f32"), (3, 1, "f32"), (3, 4, "f32"),
          (3, 8, "f16"), (3, 8, "f32"), (4, 2, "f32"), (4, 4, "f16"), (4, 8, "f32")]


def input_grad_check(dx, ref):
    for d in range(ref.shape[1]):
        scale = float(np.max(np.abs(ref[:, d])))
        err = float(np.max(np.abs(dx[:, d].astype(np.float64) - ref[:, d])))
        assert err <= 1e-5 * scale, f"coordinate {d}: dL/dx err {err:.3g} > 1e-5 * {scale:.3g}"


@pytest.mark.parametrize("D,F,dtype", SHAPES)
def test_shape_forward_backward_corners(oracle, D, F, dtype):
    w = shape_workload(D, F, dtype)
    cfg = hg.HashGridConfig.of(w)
    g = oracle.grid_of(w)
    x, t, d = I.make_points(w), I.make_table(w), I.make_dout(w)
    # forward
    out = hg.hashgrid_forward(cfg, dev(x), dev(t)).cpu().numpy()
    ref = oracle.forward(g, x, t)
    tmax = float(np.max(np.abs(t.astype(np.float64))))
    assert float(np.max(np.abs(out - ref))) <= 1e-6 * tmax
    # backward (accumulates into a non-zero buffer)
    base = np.random.default_rng(D * 10 + F).uniform(-1, 1, cfg.table_shape).astype(np.float32)
    grad = dev(base)
    hg.hashgrid_backward(cfg, dev(x), dev(d), grad)
    gref = oracle.backward(g, x, d)
    got = grad.cpu().numpy().astype(np.float64) - base
    for l in range(w.n_levels):
        assert np.max(np.abs(got[l] - gref[l])) <= 1e-5 * np.max(np.abs(gref[l])) + 4e-7
    # corners
    idx, wt = hg.hashgrid_debug_corners(cfg, dev(x))
    ridx, rw = oracle.corners(g, x)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ridx)
    assert np.max(np.abs(wt.cpu().numpy() - rw)) <= 2.5e-7


@pytest.mark.parametrize("D,F,dtype", SHAPES)
def test_shape_forward_one_lane_per_point(oracle, D, F, dtype):
    # The default forward of these shapes uses lane pairs (one lane per x
    # offset); one thread per (point, level) is the other launch shape.
    w = shape_workload(D, F, dtype)
    cfg = hg.HashGridConfig.of(w)
    x, t = I.make_points(w), I.make_table(w)
    ref = oracle.forward(oracle.grid_of(w), x, t)
    tmax = float(np.max(np.abs(t.astype(np.float64))))
    old = hg.hashgrid_tune_get(B.HG_TUNE_FWD_LANES)
    try:
        hg.hashgrid_tune(B.HG_TUNE_FWD_LANES, 1)
        one = hg.hashgrid_forward(cfg, dev(x), dev(t)).cpu().numpy()
    finally:
        hg.hashgrid_tune(B.HG_TUNE_FWD_LANES, old)
    assert one.shape == ref.shape and float(np.max(np.abs(one - ref))) <= 1e-6 * tmax


@pytest.mark.parametrize("D,F,dtype", SHAPES)
def test_shape_forward_staged_equals_direct(D, F, dtype):
    # With a workspace the levels are written level-major and transposed into
    # the rows (16-byte moves when F n and F L are multiples of 4, 4-byte moves
    # for a wide output buffer or an odd n); the same arithmetic either way.
    for n in (3 * 1024 + 77, 4096):
        w = shape_workload(D, F, dtype, n=n)
        cfg = hg.HashGridConfig.of(w)
        x, t = dev(I.make_points(w)), dev(I.make_table(w))
        direct = hg.hashgrid_forward(cfg, x, t, workspace=None).cpu().numpy()
        staged = hg.hashgrid_forward(cfg, x, t, workspace="auto").cpu().numpy()
        wide = torch.full((n, cfg.out_features + 3), 7.0, device=DEV)
        hg.hashgrid_forward(cfg, x, t, out=wide, workspace="auto")
        wide = wide.cpu().numpy()
        assert np.array_equal(direct, staged) and np.array_equal(direct, wide[:, :cfg.out_features])
        assert np.all(wide[:, cfg.out_features:] == 7.0)


@pytest.mark.parametrize("D,F,dtype", SHAPES + [(3, 2, "f32"), (3, 2, "f16")])
def test_shape_input_grad(oracle, D, F, dtype):
    w = shape_workload(D, F, dtype)
    cfg = hg.HashGridConfig.of(w)
    x, t, d = I.make_points(w), I.make_table(w), I.make_dout(w)
    ref = oracle.input_grad(oracle.grid_of(w), x, t, d)
    staged = hg.hashgrid_input_grad(cfg, dev(x), dev(t), dev(d)).cpu().numpy()
    direct = hg.hashgrid_input_grad(cfg, dev(x), dev(t), dev(d), workspace=None).cpu().numpy()
    input_grad_check(staged, ref)
    assert np.array_equal(staged, direct)  # same fp32 terms in the same level order


@pytest.mark.parametrize("name,n", [("standard", None), ("ray", 1 << 18), ("large_f16", 1 << 16)])
def test_input_grad_workloads(oracle, name, n):
    w = I.WORKLOADS[name] if n is None else I.resized(I.WORKLOADS[name], n)
    cfg = hg.HashGridConfig.of(w)
    x, t, d = I.make_points(w), I.make_table(w), I.make_dout(w)
    ref = oracle.input_grad(oracle.grid_of(w), x, t, d)
    input_grad_check(hg.hashgrid_input_grad(cfg, dev(x), dev(t), dev(d)).cpu().numpy(), ref)


def test_input_grad_strided_upstream_and_ragged(oracle):
    w = I.resized(I.WORKLOADS["standard"], 1000 + 3)
    cfg = hg.HashGridConfig.of(w)
    x, t = I.make_points(w), I.make_table(w)
    wide = I.dout_normal(77, w.n_points, 40)          # rows of 40 values, the first 32 used
    ref = oracle.input_grad(oracle.grid_of(w), x, t, wide)
    got = hg.hashgrid_input_grad(cfg, dev(x), dev(t), dev(wide)).cpu().numpy()
    input_grad_check(got, ref)
    empty = torch.empty((0, 3), device=DEV)
    assert hg.hashgrid_input_grad(cfg, empty, dev(t), torch.empty((0, 32), device=DEV)).shape == (0, 3)


def test_autograd_gives_point_and_table_gradients(oracle):
    w = I.resized(I.WORKLOADS["standard"], 2000)
    enc = hg.HashGridEncoder(device=DEV)
    t = I.make_table(w)
    with torch.no_grad():
        enc.embeddings.copy_(dev(t))
    x = dev(I.make_points(w)).requires_grad_(True)
    d = I.make_dout(w)
    enc(x).backward(dev(d))
    g = oracle.grid_of(w)
    input_grad_check(x.grad.cpu().numpy(), oracle.input_grad(g, I.make_points(w), t, d))
    ref = oracle.backward(g, I.make_points(w), d)
    got = enc.embeddings.grad.cpu().numpy()
    for l in range(w.n_levels):
        assert np.max(np.abs(got[l] - ref[l])) <= 1e-5 * np.max(np.abs(ref[l]))


@pytest.mark.parametrize("D,F,log2T", [(2, 1, 10), (4, 8, 10), (1, 4, 12), (3, 8, 16), (2, 2, 13)])
def test_shape_binned_backward_edge_cases(oracle, D, F, log2T):
    # The binned path of the other shapes against the oracle: points partly
    # outside [0,1) (negative voxel coordinates have all-ones low bits, so
    # their x+1 corner leaves its partition and takes the atomic side path),
    # one-partition tables (log2 T below the partition size), the smallest
    # workspace (one level per group) and an accumulating, non-zero buffer.
    w = shape_workload(D, F, "f32", n=2 * 4096 + 5, log2T=log2T)
    cfg = hg.HashGridConfig.of(w)
    g = oracle.grid_of(w)
    x = (I.make_points(w).astype(np.float64) * 1.5 - 0.25).astype(np.float32)
    d = I.make_dout(w)
    full, least = hg.hashgrid_backward_workspace_size(cfg, w.n_points)
    assert full > 0 and least > 0
    base = np.random.default_rng(D + F).uniform(-1, 1, cfg.table_shape).astype(np.float32)
    ref = oracle.backward(g, x, d)
    for ws in (torch.empty(full, dtype=torch.uint8, device=DEV), torch.empty(least, dtype=torch.uint8, device=DEV)):
        grad = dev(base)
        hg.hashgrid_backward(cfg, dev(x), dev(d), grad, workspace=ws)
        got = grad.cpu().numpy().astype(np.float64) - base
        for l in range(w.n_levels):
            assert np.max(np.abs(got[l] - ref[l])) <= 1e-5 * np.max(np.abs(ref[l])) + 4e-7, (l, ws.numel())
    atomic = torch.zeros(cfg.table_shape, device=DEV)
    hg.hashgrid_backward(cfg, dev(x), dev(d), atomic, workspace=None)
    for l in range(w.n_levels):
        assert np.max(np.abs(atomic.cpu().numpy()[l] - ref[l])) <= 1e-5 * np.max(np.abs(ref[l]))


@pytest.mark.parametrize("D,F,log2T,res", [(2, 2, 24, 1 << 20), (4, 8, 22, 1 << 10), (1, 1, 25, 1 << 22),
                                          (3, 4, 23, 1 << 16)])
def test_shape_limits_match_oracle(oracle, D, F, log2T, res):
    # 4096 partitions of 8192 / F entries, the largest tables the binned
    # backward takes (its counters and record stage pass 64 KB of LDS for F = 2),
    # at high resolutions.
    w = shape_workload(D, F, "f32", n=2000 + 37, L=1, log2T=log2T, nmin=res, nmax=res)
    print(f"shape limits D{D} F{F} T=2^{log2T} N={res}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    g = oracle.grid_of(w)
    x, t, d = I.make_points(w), I.make_table(w), I.make_dout(w)
    tmax = float(np.max(np.abs(t.astype(np.float64))))
    assert float(np.max(np.abs(hg.hashgrid_forward(cfg, dev(x), dev(t)).cpu().numpy() - oracle.forward(g, x, t)))) \
        <= 1e-6 * tmax
    full, _ = hg.hashgrid_backward_workspace_size(cfg, w.n_points)
    assert full > 0
    ref = oracle.backward(g, x, d)
    for ws in ("auto", None):
        grad = torch.zeros(cfg.table_shape, device=DEV)
        hg.hashgrid_backward(cfg, dev(x), dev(d), grad, workspace=ws)
        assert np.max(np.abs(grad.cpu().numpy()[0] - ref[0])) <= 1e-5 * np.max(np.abs(ref[0])), ws
    idx, _ = hg.hashgrid_debug_corners(cfg, dev(x))
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), oracle.corners(g, x)[0])
    input_grad_check(hg.hashgrid_input_grad(cfg, dev(x), dev(t), dev(d)).cpu().numpy(), oracle.input_grad(g, x, t, d))


@pytest.mark.parametrize("n", [4096 + 2, 1001])
def test_input_grad_workspace_variants_agree(oracle, n):
    # Full workspace (stage + level-major copy of the upstream rows), stage only
    # (the level pass reads the rows), none (point-major): the same fp32 terms
    # in the same order, so the same bits; even and odd n take the 16-byte and
    # the 4-byte copy kernels.
    w = I.resized(I.WORKLOADS["standard"], n)
    cfg = hg.HashGridConfig.of(w)
    x, t, d = dev(I.make_points(w)), dev(I.make_table(w)), dev(I.make_dout(w))
    full = hg.hashgrid_input_grad_workspace_size(cfg, n)
    stage_only = (n * cfg.n_levels * 3 * 4 + 255) // 256 * 256
    assert full > stage_only
    outs = [hg.hashgrid_input_grad(cfg, x, t, d, workspace=ws).cpu().numpy()
            for ws in (torch.empty(full, dtype=torch.uint8, device=DEV),
                       torch.empty(stage_only, dtype=torch.uint8, device=DEV), None)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    input_grad_check(outs[0], oracle.input_grad(oracle.grid_of(w), I.make_points(w), I.make_table(w),
                                                I.make_dout(w)))


@pytest.mark.parametrize("D,F", [(2, 2), (4, 2), (3, 1), (3, 4), (3, 8)])
def test_benchmarked_shape_at_full_size(oracle, D, F):
    # The shapes the benchmark times, at its size: the standard grid's L = 16,
    # T = 2^19 and resolutions 16..512 over 2^18 uniform points, with the
    # workspaces the benchmark passes (staged forward, binned backward in level
    # groups, level-major dL/dx).  The binned backward walks every tile chunk
    # and run-map window of the accumulate kernel; every output, gradient entry
    # and dL/dx value is compared.
    w = I.resized(I.WORKLOADS["standard"], 1 << 18, n_dims=D, n_features=F)
    print(f"full-size shape D={D} F={F} n={w.n_points}", flush=True)
    cfg = hg.HashGridConfig.of(w)
    g = oracle.grid_of(w)
    x, t, d = I.make_points(w), I.make_table(w), I.make_dout(w)
    xd, td, dd = dev(x), dev(t), dev(d)
    n = w.n_points
    out = hg.hashgrid_forward(cfg, xd, td, workspace=hg.forward_workspace(cfg, n, DEV)).cpu().numpy()
    tmax = float(np.max(np.abs(t.astype(np.float64))))
    assert float(np.max(np.abs(out - oracle.forward(g, x, t)))) <= 1e-6 * tmax
    del out
    grad = torch.zeros(cfg.table_shape, device=DEV)
    hg.hashgrid_backward(cfg, xd, dd, grad, workspace=hg.backward_workspace(cfg, n, DEV))
    got = grad.cpu().numpy()
    del grad
    gref = oracle.backward(g, x, d)
    for l in range(w.n_levels):
        assert np.max(np.abs(got[l] - gref[l])) <= 1e-5 * np.max(np.abs(gref[l])), l
    del got, gref
    isz = hg.hashgrid_input_grad_workspace_size(cfg, n)
    iws = torch.empty(isz, dtype=torch.uint8, device=DEV) if isz else None
    dx = hg.hashgrid_input_grad(cfg, xd, td, dd, workspace=iws).cpu().numpy()
    input_grad_check(dx, oracle.input_grad(g, x, t, d))
