"""Workload driver for rocprofv3 counter runs: one configuration's forward and
backward, called a fixed number of times, after a calibration copy.

    python -m multiresolution_hash_grid_amd.profile_workloads NAME [--calls K]

NAME is a workload of ``inputs.WORKLOADS`` (standard, ray, large_f16,
fused_mlp) or one of the other grid shapes at the standard grid's sizes
(D2F2, D4F2, D3F1, D3F4, D3F8).  The run first copies 256 MiB on the device
five times (the calibration the traffic summary scales the FETCH_SIZE and
WRITE_SIZE counters by), then makes K forward and K backward calls with the
workspaces the benchmark passes: the forward and backward of the encoder, or
for fused_mlp the encoder + MLP head's.  profile_summary's ``workload``
subcommand turns the counter and kernel-trace output of such runs into
per-pass figures.
"""
from __future__ import annotations

import argparse
import os
import sys

COPY_BYTES = 256 << 20
SHAPES = {"D2F2": (2, 2), "D4F2": (4, 2), "D3F1": (3, 1), "D3F4": (3, 4), "D3F8": (3, 8)}
NAMES = ("standard", "ray", "large_f16", "fused_mlp") + tuple(SHAPES)


def workload(name: str):
    from multiresolution_hash_grid_amd import inputs
    if name in SHAPES:
        D, F = SHAPES[name]
        return inputs.resized(inputs.WORKLOADS["standard"], 1 << 18, n_dims=D, n_features=F)
    return inputs.WORKLOADS[name]


def algorithmic_bytes(w) -> dict:
    """Bytes per point the method moves (as the benchmark counts them): forward
    = the point, 2^D L F table values, the L F outputs (fp32; the MLP head's
    forward: binary16 corners and the 4 outputs); backward = the point, the L F
    upstream values, 2^D L F fp32 gradient additions (the MLP head's: the point,
    dL/dy, the binary16 stage and the gradient additions)."""
    D, L, F = getattr(w, "n_dims", 3), w.n_levels, w.n_features
    esize = 2 if w.table_dtype == "f16" else 4
    corners = (1 << D) * L * F
    if w.mlp:
        return {"forward": 12 + corners * esize + 16, "backward": 12 + 16 + 2 * L * F + corners * 4}
    return {"forward": 4 * D + corners * esize + 4 * L * F, "backward": 4 * D + 4 * L * F + corners * 4}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("name", choices=NAMES)
    ap.add_argument("--calls", type=int, default=5)
    args = ap.parse_args()
    import torch
    import multiresolution_hash_grid_amd as hg
    from multiresolution_hash_grid_amd import inputs

    dev = torch.device("cuda:0")
    a = torch.ones(COPY_BYTES // 4, device=dev)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    print(f"[profile] calibration copy of {COPY_BYTES} bytes x5 done", flush=True)
    w = workload(args.name)
    cfg = hg.HashGridConfig.of(w)
    n = w.n_points
    x = torch.from_numpy(inputs.make_points(w)).to(dev)
    t = torch.from_numpy(inputs.make_table(w)).to(dev)
    g = torch.zeros(cfg.table_shape, device=dev)
    if w.mlp:
        P = [torch.from_numpy(p).to(dev) for p in inputs.mlp_params(w.seed)]
        dy = torch.from_numpy(inputs.dout_normal(w.seed + 7, n, 4)).to(dev)
        st_bytes, bw_bytes = hg.hashgrid_mlp_workspace_size(cfg, n)
        stage = torch.empty(st_bytes, dtype=torch.uint8, device=dev)
        ws = torch.empty(bw_bytes, dtype=torch.uint8, device=dev)
        y = torch.empty((n, 4), device=dev)
        grads = [torch.zeros(hg.hashgrid.MLP_SHAPES[k], device=dev) for k in ("w1", "b1", "w2", "b2", "w3", "b3")]

        def fwd():
            hg.hashgrid_mlp_forward(cfg, x, t, P, y=y, stage=stage)

        def bwd():
            hg.hashgrid_mlp_backward(cfg, x, stage, P, dy, grads, g, workspace=ws)
    else:
        d = torch.from_numpy(inputs.make_dout(w)).to(dev)
        out = torch.empty((n, cfg.out_features), device=dev)
        fws = hg.forward_workspace(cfg, n, dev)
        bws = hg.backward_workspace(cfg, n, dev)

        def fwd():
            hg.hashgrid_forward(cfg, x, t, out=out, workspace=fws)

        def bwd():
            hg.hashgrid_backward(cfg, x, d, g, workspace=bws)
    torch.cuda.synchronize()
    print(f"[profile] {args.name}: n={n}, {args.calls} forward and backward calls", flush=True)
    for _ in range(args.calls):
        fwd()
    torch.cuda.synchronize()
    for _ in range(args.calls):
        bwd()
    torch.cuda.synchronize()
    print(f"[profile] {args.name}: done", flush=True)
    return 0


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    sys.exit(main())
