#!/usr/bin/env python3
"""Throughput of the hash-grid encoder on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one forward encoding plus one backward table-gradient scatter of the
standard Instant-NGP grid (L=16, F=2, T=2^19, N_min=16, N_max=512, fp32
tables) over 2^18 uniform points in [0,1)^3, all inputs resident in HBM.
Prints one JSON line with points/s for fwd+bwd, the roofline of the dominant
kernel (HIP events on the launch stream) and the CPU oracle's throughput on
the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
# L2 request peak: 8 XCDs x 16 L2 channels, each serving one 128-byte request
# per clock, at 2.4 GHz.
L2_REQ_PEAK_PER_S = 8 * 16 * 2.4e9
PROFILES = os.path.join(ROOT, "profiles")
PASS_KERNELS = {"forward": "fwd_f2_pair_kernel + transpose_kernel",
                "backward": "bin_kernel + accumulate_kernel per level group"}


def load_counters(name: str):
    """The committed rocprofv3 counter summary of one configuration
    (profiles/counters_<name>.json: per-pass HBM traffic, L2 hit and request
    rates, MFMA utilisation), or None when it is missing or was taken on other
    library sources."""
    from multiresolution_hash_grid_amd import profile_summary as ps
    try:
        with open(os.path.join(PROFILES, f"counters_{name}.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("source_sha256") == ps.source_digest() else None


def counter_summary(rec) -> dict | None:
    """Per pass of a configuration: counter HBM bytes and their rate against
    the HBM peak, L2 hit rate and request rate against the L2 request peak
    (and MFMA utilisation of the kernels that use the matrix cores)."""
    if not rec:
        return None
    out = {}
    for p, v in rec["passes"].items():
        out[p] = {"hbm_bytes": v["hbm_bytes"], "hbm_GBps": v["hbm_GBps"], "hbm_frac": v["hbm_frac"],
                  "traffic_over_algorithmic": v["traffic_over_algorithmic"], "l2_hit_rate": v["l2_hit_rate"],
                  "l2_requests_per_s": v["l2_requests_per_s"], "l2_request_peak_per_s": L2_REQ_PEAK_PER_S,
                  "l2_request_frac": v["l2_request_frac"], "profiled_time_us": v["time_us"]}
        mf = {k: {"util_pct": kv["mfma_util_pct"], "tflops": kv.get("mfma_fp16_tflops"), "peak_tflops": 2500.0}
              for k, kv in rec["kernels"].items() if kv["pass"] == p and kv.get("mfma_util_pct") is not None}
        if mf:
            out[p]["mfma"] = mf
    return out


def algorithmic_bytes_per_point(w, table_esize: int) -> dict:
    """Bytes the method itself moves per point: the point once, 2^D corners x L
    levels x F features of table, the L*F outputs (forward); the point, the L*F
    upstream values and 2^D x L x F fp32 gradient additions (backward)."""
    D, L, F = 3, w.n_levels, w.n_features
    corners = (1 << D) * L * F
    return {"fwd": 4 * D + corners * table_esize + 4 * L * F,
            "bwd": 4 * D + 4 * L * F + corners * 4}


def load_traffic(pass_name: str, name: str = "standard"):
    """HBM bytes per call of a pass from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other sources."""
    rec = load_counters(name)
    if rec is None:
        return None
    p = rec.get("passes", {}).get(pass_name)
    return None if p is None else p.get("hbm_bytes")


def time_calls(fn, iters: int) -> float:
    """Mean milliseconds of fn() over iters calls, HIP events on the current stream."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def measure_adam(cfg, dev, iters: int) -> dict:
    """Adam update of the standard tables (L*T*F fp32 entries): reads param, m,
    v, grad and writes param, m, v -- 28 algorithmic bytes per entry."""
    import torch
    import multiresolution_hash_grid_amd as hg
    count = cfg.n_levels * cfg.table_size * cfg.n_features
    g = torch.Generator(device=dev).manual_seed(5)
    p = torch.empty(count, device=dev).uniform_(-1e-4, 1e-4, generator=g)
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    grad = torch.randn(count, device=dev, generator=g)
    step = [0]

    def call():
        step[0] += 1
        hg.hashgrid_adam_step(p, m, v, grad, lr=1e-2, step=step[0], beta1=0.9, beta2=0.99, eps=1e-15)

    ms = time_calls(call, iters)
    gbs = 28 * count / (ms * 1e-3) / 1e9
    return {"entries": count, "us_per_call": ms * 1e3, "algorithmic_bytes_per_entry": 28,
            "achieved_GBps": gbs, "frac": gbs / HBM_PEAK_GBS}


def measure_input_grad(cfg, x, t, d, iters: int) -> dict:
    """dL/dx of the standard workload (level-major with its stage): reads the
    point, its L*F upstream values and 2^D x L x F table values, writes D
    values -- 4D + 4LF + 2^D*4LF + 4D algorithmic bytes per point."""
    import torch
    import multiresolution_hash_grid_amd as hg
    n = x.shape[0]
    D, L, F = cfg.n_dims, cfg.n_levels, cfg.n_features
    dx = torch.empty((n, D), device=x.device)
    ws = torch.empty(hg.hashgrid_input_grad_workspace_size(cfg, n), dtype=torch.uint8, device=x.device)
    ms = time_calls(lambda: hg.hashgrid_input_grad(cfg, x, t, d, dx=dx, workspace=ws), iters)
    bpp = 4 * D + 4 * L * F + (1 << D) * 4 * L * F + 4 * D
    gbs = bpp * n / (ms * 1e-3) / 1e9
    return {"points": n, "us_per_call": ms * 1e3, "points_per_s": n / (ms * 1e-3),
            "algorithmic_bytes_per_point": bpp, "achieved_GBps": gbs, "frac": gbs / HBM_PEAK_GBS}


def measure_half_grad(cfg, x, d, iters: int) -> dict:
    """The standard workload's backward into a binary16 gradient buffer
    (grad_dtype "f16", binned path: each entry rounded once), with the fp32
    buffer's time beside it.  Algorithmic bytes as the fp32 backward's, the
    gradient additions priced at 2 bytes."""
    import dataclasses
    import torch
    import multiresolution_hash_grid_amd as hg
    n = x.shape[0]
    D, L, F = cfg.n_dims, cfg.n_levels, cfg.n_features
    ws = hg.backward_workspace(cfg, n, x.device)
    res = {}
    for name, c in (("f32", cfg), ("f16", dataclasses.replace(cfg, grad_dtype="f16"))):
        g = torch.zeros(cfg.table_shape, device=x.device, dtype=c.torch_grad_dtype)
        res[name] = time_calls(lambda: hg.hashgrid_backward(c, x, d, g, workspace=ws), iters)
    bpp = 4 * D + 4 * L * F + (1 << D) * L * F * 2
    gbs = bpp * n / (res["f16"] * 1e-3) / 1e9
    return {"points": n, "us_per_call": res["f16"] * 1e3, "f32_grad_us_per_call": res["f32"] * 1e3,
            "points_per_s": n / (res["f16"] * 1e-3), "algorithmic_bytes_per_point": bpp,
            "achieved_GBps": gbs, "frac": gbs / HBM_PEAK_GBS}


def measure_shapes(dev, n: int, iters: int) -> dict:
    """Forward (lane-pair kernel, staged for F <= 4), backward (generic binned
    path) and dL/dx (lane pairs level-major for D >= 3) of other grid shapes at
    the standard L, T and resolutions, n uniform points."""
    import torch
    import multiresolution_hash_grid_amd as hg
    from multiresolution_hash_grid_amd import inputs
    out = {}
    for D, F in ((2, 2), (4, 2), (3, 1), (3, 4), (3, 8)):
        w = inputs.resized(inputs.WORKLOADS["standard"], n, n_dims=D, n_features=F)
        cfg = hg.HashGridConfig.of(w)
        x = torch.from_numpy(inputs.make_points(w)).to(dev)
        t = torch.from_numpy(inputs.make_table(w)).to(dev)
        d = torch.from_numpy(inputs.make_dout(w)).to(dev)
        o = torch.empty((n, cfg.out_features), device=dev)
        g = torch.zeros(cfg.table_shape, device=dev)
        ws = hg.backward_workspace(cfg, n, dev)
        fws = hg.forward_workspace(cfg, n, dev)
        isz = hg.hashgrid_input_grad_workspace_size(cfg, n)
        iws = torch.empty(isz, dtype=torch.uint8, device=dev) if isz else None
        dx = torch.empty((n, D), device=dev)
        fms = time_calls(lambda: hg.hashgrid_forward(cfg, x, t, out=o, workspace=fws), iters)
        bms = time_calls(lambda: hg.hashgrid_backward(cfg, x, d, g, workspace=ws), iters)
        ims = time_calls(lambda: hg.hashgrid_input_grad(cfg, x, t, d, dx=dx, workspace=iws), iters)
        L, K = cfg.n_levels, 1 << D
        fb = 4 * D + K * 4 * L * F + 4 * L * F
        bb = 4 * D + 4 * L * F + K * 4 * L * F
        ib = 4 * D + 4 * L * F + K * 4 * L * F + 4 * D  # x, dout, corner gathers, dx
        out[f"D{D}_F{F}"] = {"fwd_points_per_s": n / (fms * 1e-3), "bwd_points_per_s": n / (bms * 1e-3),
                             "input_grad_points_per_s": n / (ims * 1e-3),
                             "fwd_frac": fb * n / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "bwd_frac": bb * n / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "input_grad_frac": ib * n / (ims * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "counters": counter_summary(load_counters(f"D{D}F{F}"))}
        del x, t, d, o, g, ws, fws, iws, dx
    return out


def measure_fused_mlp(dev, iters: int) -> dict:
    """Encoder + MLP head (2^22 uniform points, standard grid with binary16
    tables, 32-64-64-4, and beside it the TinyNeRF head [x, e] -> 64 -> 64 -> 4):
    forward = binary16 encoding stage + head, backward =
    head backward + weight-gradient reduction + table backward.  Algorithmic
    bytes per point: forward 12 (x) + 8 L F 2 (binary16 corners) + 16 (y);
    backward 12 (x) + 16 (dL/dy) + 2 L F (the stage) + 8 L F 4 (table
    gradient additions)."""
    import torch
    import multiresolution_hash_grid_amd as hg
    from multiresolution_hash_grid_amd import inputs
    w = inputs.WORKLOADS["fused_mlp"]
    cfg = hg.HashGridConfig.of(w)
    n = w.n_points
    x = torch.from_numpy(inputs.make_points(w)).to(dev)
    t = torch.from_numpy(inputs.make_table(w)).to(dev)
    P = [torch.from_numpy(a).to(dev) for a in inputs.mlp_params(w.seed)]
    dy = torch.from_numpy(inputs.dout_normal(w.seed + 7, n, 4)).to(dev)
    st_bytes, bw_bytes = hg.hashgrid_mlp_workspace_size(cfg, n)
    stage = torch.empty(st_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(bw_bytes, dtype=torch.uint8, device=dev)
    y = torch.empty((n, 4), device=dev)
    grads = [torch.zeros(hg.hashgrid.MLP_SHAPES[k], device=dev) for k in ("w1", "b1", "w2", "b2", "w3", "b3")]
    dtable = torch.zeros(cfg.table_shape, device=dev)
    fms = time_calls(lambda: hg.hashgrid_mlp_forward(cfg, x, t, P, y=y, stage=stage), iters)
    bms = time_calls(lambda: hg.hashgrid_mlp_backward(cfg, x, stage, P, dy, grads, dtable, workspace=ws), iters)
    # The TinyNeRF head ([x, e] -> Linear(35, 64), ...) on the same grid and points.
    P3 = [torch.from_numpy(a).to(dev) for a in inputs.mlp_params(w.seed, sizes=(35, 64, 64, 4))]
    grads3 = [torch.zeros(a.shape, device=dev) for a in P3]
    tfms = time_calls(lambda: hg.hashgrid_mlp_forward(cfg, x, t, P3, y=y, stage=stage), iters)
    tbms = time_calls(lambda: hg.hashgrid_mlp_backward(cfg, x, stage, P3, dy, grads3, dtable, workspace=ws), iters)
    L, F = cfg.n_levels, cfg.n_features
    fb = 12 + 8 * L * F * 2 + 16
    bb = 12 + 16 + 2 * L * F + 8 * L * F * 4
    return {"points": n, "fwd_points_per_s": n / (fms * 1e-3), "bwd_points_per_s": n / (bms * 1e-3),
            "step_points_per_s": n / ((fms + bms) * 1e-3), "fwd_us": fms * 1e3, "bwd_us": bms * 1e3,
            "algorithmic_bytes_per_point": {"fwd": fb, "bwd": bb},
            "fwd_frac": fb * n / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bwd_frac": bb * n / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "step_frac": (fb + bb) * n / ((fms + bms) * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tinynerf": {"fwd_us": tfms * 1e3, "bwd_us": tbms * 1e3,
                         "step_points_per_s": n / ((tfms + tbms) * 1e-3)},
            # committed rocprofv3 summary: HBM traffic, L2 rates, MfmaUtil and fp16 MFMA throughput of the head
            "counters": counter_summary(load_counters("fused_mlp"))}


def measure_other_configs(dev, iters: int) -> dict:
    """Forward and backward (with workspaces) of the other full-size grids the
    parity tests run: the ray batch (ray-major samples, whose coarse levels the
    wave pre-reduction folds) and the large binary16 grid."""
    import torch
    import multiresolution_hash_grid_amd as hg
    from multiresolution_hash_grid_amd import inputs
    out = {}
    for name in ("ray", "large_f16"):
        w = inputs.WORKLOADS[name]
        cfg = hg.HashGridConfig.of(w)
        n = w.n_points
        x = torch.from_numpy(inputs.make_points(w)).to(dev)
        t = torch.from_numpy(inputs.make_table(w)).to(dev)
        d = torch.from_numpy(inputs.make_dout(w)).to(dev)
        o = torch.empty((n, cfg.out_features), device=dev)
        g = torch.zeros(cfg.table_shape, device=dev)
        ws = hg.backward_workspace(cfg, n, dev)
        fws = hg.forward_workspace(cfg, n, dev)
        fms = time_calls(lambda: hg.hashgrid_forward(cfg, x, t, out=o, workspace=fws), iters)
        bms = time_calls(lambda: hg.hashgrid_backward(cfg, x, d, g, workspace=ws), iters)
        bpp = algorithmic_bytes_per_point(w, 2 if w.table_dtype == "f16" else 4)
        out[name] = {"points": n, "fwd_us": fms * 1e3, "bwd_us": bms * 1e3,
                     "fwd_points_per_s": n / (fms * 1e-3), "bwd_points_per_s": n / (bms * 1e-3),
                     "fwd_frac": bpp["fwd"] * n / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "bwd_frac": bpp["bwd"] * n / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "counters": counter_summary(load_counters(name))}
        del x, t, d, o, g, ws, fws
    return out


def cpu_model() -> str:
    """The host CPU's model name, with family/model/stepping when the name is
    generic."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    info.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    name = info.get("model name", "unknown")
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return f"{name} ({', '.join(ids)})" if ids else name


def cpu_baseline(w, x, t, d, budget_s: float) -> dict:
    """The CPU oracle, as it stands, on the same workload.  Multi-threaded
    (OpenMP over the levels, all host threads up to the level count): three
    runs, each timing the forward and the backward of every point, repeated
    to about budget_s / 3 seconds of work; the median run's rates are
    reported.  Single-threaded: the first 2^14 points, median of 3."""
    import statistics
    from oracle import hashgrid_oracle as oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    g = oracle.grid_of(w)

    def run(xs, ds, per_run_s):
        fwd, bwd = [], []
        for _ in range(3):
            f_s = b_s = 0.0
            reps = 0
            while f_s + b_s < per_run_s or reps == 0:
                t0 = time.perf_counter()
                oracle.forward(g, xs, t)
                t1 = time.perf_counter()
                oracle.backward(g, xs, ds)
                t2 = time.perf_counter()
                f_s += t1 - t0
                b_s += t2 - t1
                reps += 1
                if reps >= 400:
                    break
            fwd.append(len(xs) * reps / f_s)
            bwd.append(len(xs) * reps / b_s)
        f, b = statistics.median(fwd), statistics.median(bwd)
        return f, b, 1.0 / (1.0 / f + 1.0 / b)

    oracle.set_threads(threads)
    f, b, fb = run(x, d, budget_s / 3)
    oracle.set_threads(1)
    m = min(len(x), 1 << 14)
    f1, b1, fb1 = run(x[:m], d[:m], 0.0)
    oracle.set_threads(threads)
    used = min(threads, w.n_levels)
    return {"value": fb, "unit": "points/s", "cores": used, "kind": "oracle",
            "sample": f"full workload ({w.n_points} points), forward and backward timed separately, repeated to "
                      f"~{budget_s / 3:.0f} s per run, median of 3 runs; OpenMP over the {w.n_levels} levels",
            "fwd_points_per_s": f, "bwd_points_per_s": b,
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(), "omp_threads": threads,
            "single_thread": {"value": fb1, "unit": "points/s", "fwd_points_per_s": f1, "bwd_points_per_s": b1,
                              "sample": f"first {m} points, forward and backward, median of 3"}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="standard")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--section", choices=("all", "main", "next", "mlp"), default="all",
                    help="main: the standard fwd+bwd step only; next: only the figures of the "
                         "optimizer, input-gradient, shape and MLP-head paths; mlp: the MLP head "
                         "only (for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the encoder shards by points; see the design notes)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import multiresolution_hash_grid_amd as hg
    from multiresolution_hash_grid_amd import inputs

    w = inputs.WORKLOADS[args.workload]
    if w.mlp:
        raise SystemExit("the fused encode+MLP workload is measured by its own entry point")
    cfg = hg.HashGridConfig.of(w)
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    x_h, t_h, d_h = inputs.make_points(w), inputs.make_table(w), inputs.make_dout(w)
    x = torch.from_numpy(x_h).to(dev)
    t = torch.from_numpy(t_h).to(dev)
    d = torch.from_numpy(d_h).to(dev)
    out = torch.empty((w.n_points, cfg.out_features), device=dev)
    grad = torch.zeros(cfg.table_shape, device=dev)
    ws = hg.backward_workspace(cfg, w.n_points, dev)
    fws = hg.forward_workspace(cfg, w.n_points, dev)
    torch.cuda.synchronize()

    def step():
        hg.hashgrid_forward(cfg, x, t, out=out, workspace=fws)
        hg.hashgrid_backward(cfg, x, d, grad, workspace=ws)

    if args.section == "mlp":
        print(json.dumps({"next": {"fused_mlp": measure_fused_mlp(dev, 5)}}), flush=True)
        return 0
    if args.section == "next":
        print(json.dumps({"next": {"adam": measure_adam(cfg, dev, 50),
                                   "input_grad": measure_input_grad(cfg, x, t, d, 20),
                                   "half_grad": measure_half_grad(cfg, x, d, 20),
                                   "shapes": measure_shapes(dev, w.n_points, 10),
                                   "fused_mlp": measure_fused_mlp(dev, 5),
                                   "other_configs": measure_other_configs(dev, 5)}}), flush=True)
        return 0

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Pass durations for the roofline: HIP events on the launch stream around
    # each library call, over K more steps run right after the timed region
    # (recorded inside it, the events would add their own cost, ~4 %, to it).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for k in range(K):
        ev[k][0].record()
        hg.hashgrid_forward(cfg, x, t, out=out, workspace=fws)
        ev[k][1].record()
        hg.hashgrid_backward(cfg, x, d, grad, workspace=ws)
        ev[k][2].record()
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))

    esize = 2 if w.table_dtype == "f16" else 4
    bpp = algorithmic_bytes_per_point(w, esize)
    dom = "backward" if bwd_ms >= fwd_ms else "forward"
    dom_ms = bwd_ms if dom == "backward" else fwd_ms
    dom_bytes = bpp["bwd"] if dom == "backward" else bpp["fwd"]
    achieved = dom_bytes * w.n_points / (dom_ms * 1e-3) / 1e9
    traffic = load_traffic(dom, w.name)

    result = {
        "metric": "points/sec hash-grid encode fwd & fwd+bwd (L16,T2^19,F2); % HBM roofline",
        "value": w.n_points * K / elapsed,
        "unit": "points/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        # how the f32 backward rounds on its default (binned) path
        "dtype_note": "fp32 tables, blends and gradient buffer; the binned backward stores each corner pair's "
                      "w_y*w_z*dL/dout products with 20 significant bits and sums the contributions to an entry "
                      "exactly in 64-bit fixed point with a step below 2^-29 max|dL/dout| of the level, then adds "
                      "the sum to the fp32 gradient",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: L={w.n_levels} F={w.n_features} T=2^{w.log2_table_size} "
                        f"N_min={w.base_resolution} N_max={w.finest_resolution} {w.table_dtype} tables, "
                        f"N={w.n_points} {w.structure} points, forward+backward per step",
            "points_per_step": w.n_points,
        },
        "fwd_points_per_s": w.n_points / (fwd_ms * 1e-3),
        "bwd_points_per_s": w.n_points / (bwd_ms * 1e-3),
        "fwd_kernel_ms": fwd_ms,
        "bwd_kernel_ms": bwd_ms,
        "algorithmic_bytes_per_point": bpp,
        "roofline": {
            "bound": "hbm",
            "kernel": f"{dom} pass ({PASS_KERNELS[dom]}), one library call",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
        },
        # HBM traffic, L2 hit and request rates per pass (committed rocprofv3 counter summary)
        "cache": counter_summary(load_counters(w.name)),
        "roofline_fwd_frac": bpp["fwd"] * w.n_points / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline_fwd_bwd_frac": (bpp["fwd"] + bpp["bwd"]) * w.n_points * K / elapsed / 1e9 / HBM_PEAK_GBS,
    }
    # The paths after the encoder's own step: Adam over the tables, dL/dx,
    # the binary16 gradient buffer, other grid shapes, the MLP head.
    if args.section in ("all", "next"):
        print("[bench] optimizer, input gradient, shapes, MLP head", file=sys.stderr, flush=True)
        result["next"] = {"adam": measure_adam(cfg, dev, 50),
                          "input_grad": measure_input_grad(cfg, x, t, d, 20),
                          "half_grad": measure_half_grad(cfg, x, d, 20),
                          "shapes": measure_shapes(dev, w.n_points, 10),
                          "fused_mlp": measure_fused_mlp(dev, 5),
                          "other_configs": measure_other_configs(dev, 5)}
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, x_h, t_h, d_h, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
