"""The allocation-free backward (hashgrid_backward_noalloc, the library's own
fixed device scratch in place of a caller workspace) against the existing
entry point hashgrid_backward with a full workspace, through the C ABI: two
calls in a row on each grid, the second with fewer points, so the second
finds the first call's records in the scratch.  Bar: <= 1e-5 * max|gradient|
per level (in fact both take the binned path, whose fixed-point sums make
them agree bit for bit), and the oracle's gradient for the smaller call."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import multiresolution_hash_grid_amd as hg  # noqa: E402
from multiresolution_hash_grid_amd import inputs as I  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def level_check(got, ref, L):
    for l in range(L):
        scale = float(np.max(np.abs(ref[l])))
        err = float(np.max(np.abs(got[l].astype(np.float64) - ref[l].astype(np.float64))))
        assert err <= 1e-5 * scale, (l, err, scale)


@pytest.mark.parametrize("name,D,F,sizes", [("standard", 3, 2, (1 << 18, 5000 + 13)),
                                            ("standard", 2, 4, (3 * 4096 + 5, 2000 + 1)),
                                            ("tiny", 3, 2, (4096, 1000 + 3))])
def test_noalloc_backward_matches_workspace_backward(oracle, name, D, F, sizes):
    oracle.set_threads(min(16, os.cpu_count() or 1))
    base = I.resized(I.WORKLOADS[name], max(sizes), n_dims=D, n_features=F)
    cfg = hg.HashGridConfig.of(base)
    x_all, d_all = I.make_points(base), I.make_dout(base)
    for n in sizes:
        print(f"no-alloc backward {name} D={D} F={F} n={n}", flush=True)
        x, d = dev(x_all[:n]), dev(d_all[:n])
        ref = torch.zeros(cfg.table_shape, device=DEV)
        hg.hashgrid_backward(cfg, x, d, ref, workspace=hg.backward_workspace(cfg, n, DEV))
        got = torch.zeros(cfg.table_shape, device=DEV)
        hg.hashgrid_backward_noalloc(cfg, x, d, got)
        torch.cuda.synchronize()
        g, r = got.cpu().numpy(), ref.cpu().numpy()
        level_check(g, r, cfg.n_levels)
        assert np.array_equal(g, r)
    w = I.resized(base, sizes[-1])
    level_check(g, oracle.backward(oracle.grid_of(w), x_all[:sizes[-1]], d_all[:sizes[-1]]), cfg.n_levels)
