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


def _write(path, rows, fields):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_" + ("counter_collection.csv" if "Counter_Name" in fields
                                          else "kernel_stats.csv")), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_counters_summary(tmp_path):
    k = "hg::(anonymous namespace)::bin_kernel(float const*, long)"
    m = "_ZN2hg12_GLOBAL__N_114mlp_fwd_kernelEPKDF16_lNS_9MlpParamsEP"
    cfields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    for did in range(1, 7):   # six dispatches; the summary drops the first two as cold
        hit = 900.0 if did > 2 else 0.0
        rows += [{"Dispatch_Id": did, "Kernel_Name": k, "Counter_Name": "TCC_HIT_sum", "Counter_Value": hit},
                 {"Dispatch_Id": did, "Kernel_Name": k, "Counter_Name": "TCC_MISS_sum", "Counter_Value": 100.0},
                 {"Dispatch_Id": did, "Kernel_Name": k, "Counter_Name": "TCC_REQ_sum", "Counter_Value": 1000.0}]
    _write(str(tmp_path / "l2"), rows, cfields)
    mrows = [{"Dispatch_Id": d, "Kernel_Name": m, "Counter_Name": c, "Counter_Value": v}
             for d in range(1, 4) for c, v in (("MfmaUtil", 40.0), ("SQ_INSTS_VALU_MFMA_MOPS_F16", 1e6))]
    _write(str(tmp_path / "mfma"), mrows, cfields)
    sfields = ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"]
    _write(str(tmp_path / "s1"), [{"Name": k, "Calls": 6, "AverageNs": 1000.0, "MinNs": 1, "MaxNs": 1}], sfields)
    _write(str(tmp_path / "s2"), [{"Name": m, "Calls": 3, "AverageNs": 2000.0, "MinNs": 1, "MaxNs": 1}], sfields)
    out = str(tmp_path / "c.json")
    ps.counters(types.SimpleNamespace(l2=str(tmp_path / "l2"), l2_stats=str(tmp_path / "s1"),
                                      mfma=str(tmp_path / "mfma"), mfma_stats=str(tmp_path / "s2"), out=out,
                                      command_l2="", command_mfma=""))
    rec = json.load(open(out))
    b = rec["l2"]["bin_kernel"]
    assert b["pass"] == "backward" and abs(b["hit_rate"] - 0.9) < 1e-12
    assert b["requests"] == 1000.0 and abs(b["requests_per_s"] - 1e9) < 1e-3   # 1000 in 1 us
    f = rec["mfma"]["mlp_fwd_kernel"]
    assert f["mfma_util_pct"] == 40.0 and f["fp16_flops"] == 512e6
    assert abs(f["tflops"] - 512e6 / 2e-6 / 1e12) < 1e-9


def test_committed_summaries_parse():
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic_standard.json")))
    assert {"forward", "backward"} <= set(t["passes"])
    c = json.load(open(os.path.join(ROOT, "profiles", "counters_standard_mlp.json")))
    gather = [k for k in c["l2"] if k.startswith("fwd_f2_pair_kernel<0, 4, false, float")]
    assert len(gather) == 1 and 0.0 <= c["l2"][gather[0]]["hit_rate"] <= 1.0
    assert set(c["mfma"]) >= {"mlp_fwd_kernel", "mlp_bwd_kernel"}


def test_source_digest_ignores_comments_and_layout():
    a = "int f(int x) {  // twice\n    return 2 * x; /* the result */\n}\n"
    b = "int f(int x)\n{\n  return 2 * x;\n}  // another comment\n"
    c = "int f(int x) { return 3 * x; }"
    assert ps._code_only(a) == ps._code_only(b)
    assert ps._code_only(a) != ps._code_only(c)
