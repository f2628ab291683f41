"""Summaries of rocprofv3 output for the encoder's passes.

    # kernel durations of a --kernel-trace --stats -f csv run that made PASSES
    # calls of each library entry point
    python -m multiresolution_hash_grid_amd.profile_summary stats DIR --passes P --command "..." --out FILE.md

    # HBM traffic per pass from --pmc FETCH_SIZE / --pmc WRITE_SIZE runs of the
    # benchmark and of a plain device copy (the calibration)
    python -m multiresolution_hash_grid_amd.profile_summary traffic --fetch D1 --write D2 \\
        --copy-fetch D3 --copy-write D4 --copy-bytes B --passes P --out FILE.json

    # the calibration workload itself: a device-to-device copy of B bytes
    python -m multiresolution_hash_grid_amd.profile_summary copy --bytes B

    # L2 (TCC) hit rate and request rate per kernel from a --pmc TCC_HIT_sum
    # TCC_MISS_sum TCC_REQ_sum run, MFMA utilisation from a --pmc MfmaUtil
    # SQ_INSTS_VALU_MFMA_MOPS_F16 run; durations from kernel-trace --stats runs
    python -m multiresolution_hash_grid_amd.profile_summary counters --l2 D1 --l2-stats S1 \
        --mfma D2 --mfma-stats S2 --out FILE.json

A pass is the group of kernels one library call launches: the forward is the
gather plus the level-major transpose, the backward the binned path's bin and
accumulate kernels, once per level group (or the atomic scatter).  Per-pass
figures weight each kernel by its launches per call.
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
    "forward": ("fwd_f2_kernel", "fwd_f2_pair_kernel", "transpose_kernel"),
    "backward": ("bin_kernel", "accumulate_kernel", "bwd_f2_kernel"),
}
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ("device_common.h", "hashgrid_internal.h", "encode_kernels.hip", "binned_common.h",
           "binned_backward.hip")
MLP_SOURCES = SOURCES + ("mlp_kernels.hip",)


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace runs collapsed: edits
    to comments or layout do not change the code the figures belong to."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(files=SOURCES) -> str:
    """sha256 over the code of the kernel sources (counter figures are only valid for it)."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "multiresolution_hash_grid_amd", "csrc", f), encoding="utf-8") as fh:
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


def traffic(args) -> None:
    fetch = _counter_per_dispatch(args.fetch, "FETCH_SIZE")
    write = _counter_per_dispatch(args.write, "WRITE_SIZE")
    cf = _counter_per_dispatch(args.copy_fetch, "FETCH_SIZE")
    cw = _counter_per_dispatch(args.copy_write, "WRITE_SIZE")
    # The copy moves copy_bytes in and copy_bytes out; counters are in KiB.
    copy_read_kib = max(max(v) for v in cf.values())
    copy_write_kib = max(max(v) for v in cw.values())
    f_scale = args.copy_bytes / (copy_read_kib * 1024.0)
    w_scale = args.copy_bytes / (copy_write_kib * 1024.0)
    kernels = {}
    passes = collections.defaultdict(lambda: {"fetch_bytes": 0.0, "write_bytes": 0.0})
    for name in set(fetch) | set(write):
        p = pass_of(name)
        fv, wv = fetch.get(name, [0.0]), write.get(name, [0.0])
        fb = _avg(fv) * 1024.0 * f_scale
        wb = _avg(wv) * 1024.0 * w_scale
        per_call = len(fv) / args.passes  # launches of this kernel per library call
        kernels[short_name(name)] = {"pass": p, "fetch_bytes": fb, "write_bytes": wb,
                                     "launches_per_call": per_call}
        if p:
            passes[p]["fetch_bytes"] += fb * per_call
            passes[p]["write_bytes"] += wb * per_call
    for p in passes.values():
        p["hbm_bytes_per_launch"] = p["fetch_bytes"] + p["write_bytes"]
    rec = {
        "about": "HBM bytes per call of each entry point from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB "
                 "per dispatch, times dispatches per call), each scaled by the factor that makes the same "
                 "counter read the known size of a plain device copy.",
        "calls_per_run": args.passes,
        "command_fetch": args.command_fetch, "command_write": args.command_write,
        "copy_bytes": args.copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
        "source_sha256": source_digest(), "passes": dict(passes), "kernels": kernels,
    }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def _durations_us(d: str) -> dict:
    """{kernel short name: average duration in us} of a --kernel-trace --stats run."""
    return {short_name(r["Name"]): float(r["AverageNs"]) / 1e3
            for r in csv.DictReader(open(_find(d, "kernel_stats.csv")))}


def counters(args) -> None:
    hit = _counter_per_dispatch(args.l2, "TCC_HIT_sum")
    miss = _counter_per_dispatch(args.l2, "TCC_MISS_sum")
    req = _counter_per_dispatch(args.l2, "TCC_REQ_sum")
    dur = _durations_us(args.l2_stats)
    l2 = {}
    for name in hit:
        sn = short_name(name)
        h, m, r = _avg(hit[name]), _avg(miss.get(name, [0.0])), _avg(req.get(name, [0.0]))
        us = dur.get(sn)
        l2[sn] = {"pass": pass_of(name), "hit_rate": h / (h + m) if h + m else None, "requests": r,
                  "hits": h, "misses": m, "duration_us": us,
                  "requests_per_s": r / (us * 1e-6) if us else None}
    util = _counter_per_dispatch(args.mfma, "MfmaUtil")
    mops = _counter_per_dispatch(args.mfma, "SQ_INSTS_VALU_MFMA_MOPS_F16")
    mdur = _durations_us(args.mfma_stats)
    mfma = {}
    for name in mops:
        sn = short_name(name)
        ops = _avg(mops[name])
        if ops <= 0:
            continue
        us = mdur.get(sn)
        flops = ops * 512.0  # the counter counts fp16 MFMA work in units of 512 flops
        mfma[sn] = {"mfma_util_pct": _avg(util[name]) if name in util else None, "fp16_flops": flops,
                    "duration_us": us, "tflops": flops / (us * 1e-6) / 1e12 if us else None}
    rec = {
        "about": "Per-kernel L2 (TCC) hit rate, requests per dispatch and request rate of the standard "
                 "workload's kernels; MFMA utilisation (busy cycles over SIMD cycles) and fp16 MFMA "
                 "throughput of the MLP head's kernels. Durations are the kernel-trace averages of "
                 "runs without counters.",
        "command_l2": args.command_l2, "command_mfma": args.command_mfma,
        "source_sha256": source_digest(), "mlp_source_sha256": source_digest(MLP_SOURCES),
        "l2": l2, "mfma": mfma,
    }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def copy(args) -> None:
    import torch
    n = args.bytes // 4
    a = torch.ones(n, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied", args.bytes, "bytes x5", flush=True)


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
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write", "out"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--passes", type=int, required=True, help="calls of each entry point in the run")
    t.add_argument("--command-fetch", default="")
    t.add_argument("--command-write", default="")
    k = sub.add_parser("counters")
    for a in ("l2", "l2_stats", "mfma", "mfma_stats", "out"):
        k.add_argument("--" + a.replace("_", "-"), dest=a, required=True)
    k.add_argument("--command-l2", default="")
    k.add_argument("--command-mfma", default="")
    c = sub.add_parser("copy")
    c.add_argument("--bytes", type=int, default=256 << 20)
    args = ap.parse_args()
    {"stats": stats, "traffic": traffic, "counters": counters, "copy": copy}[args.cmd](args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
