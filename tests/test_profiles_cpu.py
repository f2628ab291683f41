"""Host logic of the rocprofv3 summaries: kernel-name normalisation, pass
attribution, and the counters summary on synthetic profiler CSVs; the
committed summaries parse."""
import csv
import json
import os
import types

from multiresolution_hash_grid_amd import profile_summary as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_names_and_passes():
    acc = "void hg::binned::accumulate_kernel<512, hg::(anonymous namespace)::StdPolicy>(hg::BinParams, int)"
    assert ps.short_name(acc) == "accumulate_kernel<512, StdPolicy>"
    assert ps.pass_of(acc) == "backward"
    assert ps.short_name("hg::(anonymous namespace)::bin_kernel(float const*, long)") == "bin_kernel"
    assert ps.pass_of("hg::(anonymous namespace)::transpose_kernel<2, true>(float const*)") == "forward"
    assert ps.short_name("_ZN2hg12_GLOBAL__N_114mlp_bwd_kernelEPKDF16_lNS_9MlpParamsEP") == "mlp_bwd_kernel"
    assert ps.pass_of("void at::native::vectorized_elementwise_kernel<4>(int)") is None
    assert ps.pass_of("hg::(anonymous namespace)::mlp_dy_max_kernel(float4 const*)") == "backward"
    assert ps.pass_of("hg::(anonymous namespace)::fwd_generic_pair_kernel<3, 4, 0>(float const*)") == "forward"
    assert ps.pass_of("void hg::(anonymous namespace)::fwd_dense_kernel<1, _Float16>(float const*, long)") == "forward"
    assert ps.pass_of("hg::(anonymous namespace)::order_scatter_kernel(hg::(anonymous namespace)::Point3 const*)") == "forward"


def _write(path, rows, fields):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_" + ("counter_collection.csv" if "Counter_Name" in fields
                                          else "kernel_stats.csv")), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_workload_summary(tmp_path):
    # A synthetic run of the standard workload with K = 2 calls of each pass:
    # the calibration copy (256 MiB read and written; the counters read half of
    # it for FETCH_SIZE, all of it for WRITE_SIZE), one gather and one
    # transpose per forward, two bin and two accumulate launches per backward.
    K = 2
    copy = "void at::native::copy_kernel(float*)"
    ks = {"hg::(anonymous namespace)::fwd_f2_pair_kernel<0, 4, false, float, false>(float const*)": (1, 100e3),
          "hg::(anonymous namespace)::transpose_kernel<2, true>(float const*)": (1, 10e3),
          "hg::(anonymous namespace)::bin_kernel(float const*, long)": (2, 30e3),
          "void hg::binned::accumulate_kernel<1024, hg::(anonymous namespace)::StdPolicy>(hg::BinParams)": (2, 50e3)}
    cf = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    r1, r2, did = [], [], 0
    did += 1
    r1 += [{"Dispatch_Id": did, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 131072.0}]
    r2 += [{"Dispatch_Id": did, "Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 262144.0}]
    for name, (per, _) in ks.items():
        for _ in range(per * K):
            did += 1
            r1 += [{"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1024.0},
                   {"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": "TCC_REQ_sum", "Counter_Value": 1e6}]
            r2 += [{"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": "WRITE_SIZE", "Counter_Value": 2048.0},
                   {"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": "TCC_HIT_sum", "Counter_Value": 9e5},
                   {"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": "TCC_MISS_sum", "Counter_Value": 1e5}]
    _write(str(tmp_path / "p1"), r1, cf)
    _write(str(tmp_path / "p2"), r2, cf)
    sf = ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"]
    _write(str(tmp_path / "st"), [{"Name": n, "Calls": per * K, "AverageNs": ns, "MinNs": 1, "MaxNs": 1}
                                  for n, (per, ns) in ks.items()], sf)
    out = str(tmp_path / "counters_standard.json")
    ps.workload(types.SimpleNamespace(name="standard", stats=str(tmp_path / "st"), pmc1=str(tmp_path / "p1"),
                                      pmc2=str(tmp_path / "p2"), calls=K, command="cmd", out=out))
    rec = json.load(open(out))
    assert rec["calibration"]["fetch_scale"] == 2.0 and rec["calibration"]["write_scale"] == 1.0
    f, b = rec["passes"]["forward"], rec["passes"]["backward"]
    assert f["time_us"] == 110.0 and b["time_us"] == 160.0
    # per launch 1024 KiB fetched (x2 calibration) and 2048 KiB written: 4 MiB per launch
    assert f["hbm_bytes"] == 2 * (4 << 20) and b["hbm_bytes"] == 4 * (4 << 20)
    n = 1 << 18
    assert abs(f["frac"] - 1164 * n / 110e-6 / 8e12) < 1e-12
    assert abs(b["l2_hit_rate"] - 0.9) < 1e-12 and b["l2_requests"] == 4e6
    assert os.path.exists(str(tmp_path / "counters_standard.md"))


def test_committed_summaries_parse():
    names = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.startswith("counters_") and
             f.endswith(".json")]
    for fn in names:
        rec = json.load(open(os.path.join(ROOT, "profiles", fn)))
        assert set(rec["passes"]) <= {"forward", "backward"} and rec["passes"]
        for p in rec["passes"].values():
            assert p["time_us"] > 0 and p["hbm_bytes"] > 0 and 0 < p["frac"] < 1.5


def test_source_digest_ignores_comments_and_layout():
    a = "int f(int x) {  // twice\n    return 2 * x; /* the result */\n}\n"
    b = "int f(int x)\n{\n  return 2 * x;\n}  // another comment\n"
    c = "int f(int x) { return 3 * x; }"
    assert ps._code_only(a) == ps._code_only(b)
    assert ps._code_only(a) != ps._code_only(c)
