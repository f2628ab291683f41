"""Summaries of rocprofv3 output for the encoder's passes.

    # kernel durations of a --kernel-trace --stats -f csv run that made PASSES
    # calls of each library entry point (e.g. the benchmark itself)
    python -m multiresolution_hash_grid_amd.profile_summary stats DIR --passes P --command "..." --out FILE.md

    # per-pass HBM traffic, L2 hit and request rates, MFMA utilisation and
    # roofline fractions of one configuration, from three runs of
    # ``python -m multiresolution_hash_grid_amd.profile_workloads NAME --calls K``:
    #   --stats: rocprofv3 --kernel-trace --stats -f csv
    #   --pmc1 : rocprofv3 --pmc FETCH_SIZE TCC_REQ_sum -f csv
    #   --pmc2 : rocprofv3 --pmc WRITE_SIZE TCC_HIT_sum TCC_MISS_sum -f csv
    #   --mfma : (optional) rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_F16 -f csv
    python -m multiresolution_hash_grid_amd.profile_summary workload NAME --stats D1 --pmc1 D2 --pmc2 D3 \
        --calls K --command "..." --out profiles/counters_NAME.json

A pass is the group of kernels one library call launches: the forward is the
gather (plus the level-major transpose, or the MLP head), the backward the
binned path's bin and accumulate kernels, once per level group (plus the MLP
head's backward and its reductions).  Per-pass figures weight each kernel by
its launches per call.  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are
scaled by the factors that make them read the known 256 MiB of the device
copy each run starts with.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

PASSES = {
    "forward": ("fwd_f2_kernel", "fwd_f2_pair_kernel", "fwd_dense_kernel", "transpose_kernel", "fwd_generic_kernel",
                "fwd_generic_pair_kernel", "mlp_fwd_kernel", "order_count_kernel", "order_prefix_kernel",
                "order_scatter_kernel"),
    "backward": ("bin_kernel", "accumulate_kernel", "bwd_f2_kernel", "bwd_f2_quad_kernel", "bin_generic_kernel",
                 "bwd_generic_kernel", "bwd_dense_kernel", "mlp_bwd_kernel", "mlp_dy_max_kernel",
                 "mlp_reduce1_kernel", "mlp_reduce2_kernel"),
}
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "multiresolution_hash_grid_amd", "csrc")
HBM_PEAK_BPS = 8000e9                 # MI355X HBM3E, AMD published peak
L2_REQ_PEAK_PER_S = 8 * 16 * 2.4e9    # 8 XCDs x 16 L2 channels x one request per clock at 2.4 GHz
COPY_BYTES = 256 << 20


def all_sources() -> tuple:
    """Every file of the library's sources: kernels, their headers and the host
    code that sizes and launches them."""
    return tuple(sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp"))))


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace runs collapsed: edits
    to comments or layout do not change the code the figures belong to."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(files=None) -> str:
    """sha256 over the code of the library sources (counter figures are only valid for it)."""
    h = hashlib.sha256()
    for f in files if files is not None else all_sources():
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(f.encode())
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def _unmangle(name: str) -> str:
    """Kernel name and template arguments of a mangled hg:: kernel symbol that
    the profiler left mangled (e.g. ones with _Float16 arguments)."""
    m = re.match(r"_ZN2hg12_GLOBAL__N_1(\d+)", name)
    if not m:
        return name
    k = int(m.group(1))
    rest = name[m.end():]
    ident, rest = rest[:k], rest[k:]
    if not rest.startswith("I"):
        return ident
    args = []
    for tok in re.finditer(r"Li(-?\d+)E|Lb([01])E|DF16_|f(?=[EL])", rest[1:rest.find("EE") + 1]):
        if tok.group(1) is not None:
            args.append(tok.group(1))
        elif tok.group(2) is not None:
            args.append("true" if tok.group(2) == "1" else "false")
        elif tok.group(0) == "DF16_":
            args.append("_Float16")
        else:
            args.append("float")
    return f"{ident}<{', '.join(args)}>"


def short_name(name: str) -> str:
    if name.startswith("_ZN"):
        return _unmangle(name)
    name = re.sub(r"hg::(\(anonymous namespace\)::|binned::)+", "", name).replace("void ", "")
    return re.sub(r"\(.*", "", name)


def pass_of(name: str):
    base = re.sub(r"<.*", "", short_name(name))
    for p, kernels in PASSES.items():
        if base in kernels:
            return p
    return None


def _find(d: str, suffix: str) -> str:
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def stats(args) -> None:
    rows = list(csv.DictReader(open(_find(args.dir, "kernel_stats.csv"))))
    lines = [f"# Kernel durations: {args.title}", "", "Command:", "", "```", args.command, "```", "",
             "| kernel | pass | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|---|"]
    per_pass = collections.defaultdict(float)
    for r in rows:
        p = pass_of(r["Name"])
        avg = float(r["AverageNs"]) / 1e3
        lines.append(f"| `{short_name(r['Name'])}` | {p or '-'} | {r['Calls']} | {avg:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
        if p and args.passes > 0:
            per_pass[p] += avg * int(r["Calls"]) / args.passes
    if args.passes > 0:
        lines += ["", f"Kernel time per call of each entry point ({args.passes} calls each, us): " +
                  ", ".join(f"{p} {v:.1f}" for p, v in sorted(per_pass.items()))]
    lines.append("")
    text = "\n".join(lines)
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


def _counter_per_dispatch(d: str, counter: str):
    """{kernel short name: [per-dispatch value summed over dimensions]}"""
    per = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for did in sorted(per, key=int):
        out[names[did]].append(per[did])
    return out


def _avg(vals):
    vals = vals[2:] if len(vals) > 4 else vals   # drop the first (cold) dispatches
    return sum(vals) / len(vals)


def _durations_us(d: str) -> dict:
    """{kernel short name: average duration in us} of a --kernel-trace --stats run."""
    return {short_name(r["Name"]): float(r["AverageNs"]) / 1e3
            for r in csv.DictReader(open(_find(d, "kernel_stats.csv")))}


def _find_copy(per: dict) -> tuple:
    """(name, KiB per dispatch) of the calibration copy: the largest dispatch
    of a kernel that is not one of the library's."""
    best = None
    for name, vals in per.items():
        if pass_of(name) is None and not short_name(name).startswith(("fwd_", "bin", "acc", "mlp", "bwd")):
            v = max(vals)
            if best is None or v > best[1]:
                best = (name, v)
    if best is None:
        raise ValueError("no calibration copy in the counter run")
    return best


def workload(args) -> None:
    from multiresolution_hash_grid_amd import profile_workloads as pw
    w = pw.workload(args.name)
    alg = pw.algorithmic_bytes(w)
    dur = _durations_us(args.stats)
    calls = {short_name(r["Name"]): int(r["Calls"])
             for r in csv.DictReader(open(_find(args.stats, "kernel_stats.csv")))}
    fetch = _counter_per_dispatch(args.pmc1, "FETCH_SIZE")
    req = _counter_per_dispatch(args.pmc1, "TCC_REQ_sum")
    write = _counter_per_dispatch(args.pmc2, "WRITE_SIZE")
    hit = _counter_per_dispatch(args.pmc2, "TCC_HIT_sum")
    miss = _counter_per_dispatch(args.pmc2, "TCC_MISS_sum")
    mdir = getattr(args, "mfma", None) or args.pmc2
    util = _counter_per_dispatch(mdir, "MfmaUtil")
    mops = _counter_per_dispatch(mdir, "SQ_INSTS_VALU_MFMA_MOPS_F16")
    copy_name, copy_fetch_kib = _find_copy(fetch)
    if copy_name not in write:
        raise ValueError(f"the calibration copy {copy_name} is missing from the WRITE_SIZE run")
    copy_write_kib = max(write[copy_name])
    f_scale = COPY_BYTES / (copy_fetch_kib * 1024.0)
    w_scale = COPY_BYTES / (copy_write_kib * 1024.0)
    kernels = {}
    passes = {p: collections.defaultdict(float) for p in PASSES}
    for name in set(fetch) | set(write):
        p = pass_of(name)
        if p is None:
            continue
        sn = short_name(name)
        per_call = calls.get(sn, len(fetch.get(name, write.get(name)))) / args.calls
        k = {"pass": p, "launches_per_call": per_call, "duration_us": dur.get(sn),
             "fetch_bytes": _avg(fetch[name]) * 1024.0 * f_scale if name in fetch else None,
             "write_bytes": _avg(write[name]) * 1024.0 * w_scale if name in write else None,
             "l2_requests": _avg(req[name]) if name in req else None}
        if name in hit and name in miss:
            h, m = _avg(hit[name]), _avg(miss[name])
            k["l2_hit_rate"] = h / (h + m) if h + m else None
        if name in mops and _avg(mops[name]) > 0:
            flops = _avg(mops[name]) * 512.0  # the counter counts fp16 MFMA work in units of 512 flops
            k["mfma_util_pct"] = _avg(util[name]) if name in util else None
            k["mfma_fp16_tflops"] = flops / (k["duration_us"] * 1e-6) / 1e12 if k["duration_us"] else None
        kernels[sn] = k
        acc = passes[p]
        acc["time_us"] += per_call * (k["duration_us"] or 0.0)
        acc["hbm_bytes"] += per_call * ((k["fetch_bytes"] or 0.0) + (k["write_bytes"] or 0.0))
        acc["fetch_bytes"] += per_call * (k["fetch_bytes"] or 0.0)
        acc["write_bytes"] += per_call * (k["write_bytes"] or 0.0)
        acc["l2_requests"] += per_call * (k["l2_requests"] or 0.0)
        if "l2_hit_rate" in k and k["l2_hit_rate"] is not None:
            acc["_hits"] += per_call * k["l2_hit_rate"] * (k["l2_requests"] or 0.0)
    out_passes = {}
    for p, acc in passes.items():
        if not acc["time_us"]:
            continue
        t = acc["time_us"] * 1e-6
        a = alg[p] * w.n_points
        out_passes[p] = {
            "time_us": acc["time_us"], "points_per_s": w.n_points / t,
            "algorithmic_bytes_per_point": alg[p], "algorithmic_GBps": a / t / 1e9, "frac": a / t / HBM_PEAK_BPS,
            "hbm_bytes": acc["hbm_bytes"], "fetch_bytes": acc["fetch_bytes"], "write_bytes": acc["write_bytes"],
            "hbm_GBps": acc["hbm_bytes"] / t / 1e9, "hbm_frac": acc["hbm_bytes"] / t / HBM_PEAK_BPS,
            "traffic_over_algorithmic": acc["hbm_bytes"] / a,
            "l2_requests": acc["l2_requests"], "l2_requests_per_s": acc["l2_requests"] / t,
            "l2_request_frac": acc["l2_requests"] / t / L2_REQ_PEAK_PER_S,
            "l2_hit_rate": acc["_hits"] / acc["l2_requests"] if acc["l2_requests"] else None}
    rec = {
        "about": "Per-pass figures of one configuration from rocprofv3: kernel-trace durations, FETCH_SIZE and "
                 "WRITE_SIZE (scaled by a 256 MiB device copy in the same run), L2 (TCC) requests and hit rate, "
                 "MFMA utilisation; algorithmic bytes as the benchmark counts them; peaks: HBM 8 TB/s, L2 "
                 "307 G requests/s.",
        "workload": args.name, "points": w.n_points, "calls": args.calls, "command": args.command,
        "source_sha256": source_digest(),
        "calibration": {"kernel": short_name(copy_name), "copy_bytes": COPY_BYTES, "fetch_scale": f_scale,
                        "write_scale": w_scale},
        "passes": out_passes, "kernels": kernels,
    }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# Counters: {args.name} ({w.n_points} points, {args.calls} calls of each pass)", "",
             "Commands:", "", "```", args.command, "```", "",
             "| pass | time (us) | points/s | algorithmic GB/s | frac of 8 TB/s | HBM bytes | HBM / algorithmic "
             "| L2 hit | L2 requests/s | frac of L2 request peak |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for p, v in out_passes.items():
        hr = "-" if v["l2_hit_rate"] is None else f"{v['l2_hit_rate']:.2f}"
        lines.append(f"| {p} | {v['time_us']:.1f} | {v['points_per_s']:.3g} | {v['algorithmic_GBps']:.0f} | "
                     f"{v['frac']:.3f} | {v['hbm_bytes'] / 1e6:.1f} MB | {v['traffic_over_algorithmic']:.2f} | {hr} | "
                     f"{v['l2_requests_per_s'] / 1e9:.0f} G | {v['l2_request_frac']:.2f} |")
    lines += ["", "| kernel | pass | launches per call | us | fetch MB | write MB | L2 hit | MFMA busy % |",
              "|---|---|---|---|---|---|---|---|"]
    for sn, k in sorted(kernels.items(), key=lambda kv: (kv[1]["pass"], kv[0])):
        f = "-" if k["fetch_bytes"] is None else f"{k['fetch_bytes'] / 1e6:.1f}"
        wr = "-" if k["write_bytes"] is None else f"{k['write_bytes'] / 1e6:.1f}"
        hr = "-" if k.get("l2_hit_rate") is None else f"{k['l2_hit_rate']:.2f}"
        mu = "-" if k.get("mfma_util_pct") is None else f"{k['mfma_util_pct']:.1f}"
        d = "-" if k["duration_us"] is None else f"{k['duration_us']:.1f}"
        lines.append(f"| `{sn}` | {k['pass']} | {k['launches_per_call']:.2f} | {d} | {f} | {wr} | {hr} | {mu} |")
    lines.append("")
    with open(os.path.splitext(args.out)[0] + ".md", "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--out", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="rocprofv3 --kernel-trace --stats")
    s.add_argument("--passes", type=int, required=True,
                   help="calls of each entry point in the run (0: list the kernels only)")
    k = sub.add_parser("workload")
    k.add_argument("name")
    for a in ("stats", "pmc1", "pmc2", "out", "command"):
        k.add_argument("--" + a, dest=a, required=True)
    k.add_argument("--calls", type=int, required=True)
    k.add_argument("--mfma", default=None, help="run with --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_F16")
    args = ap.parse_args()
    {"stats": stats, "workload": workload}[args.cmd](args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
