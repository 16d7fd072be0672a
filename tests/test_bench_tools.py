"""CPU tests of the benchmark's host-side accounting and profile tooling.

No GPU: the algorithmic flop counts of the workloads against the step's
structure (three times the forward products plus the prescribed recompute),
the kernel-name shortener used by the profile summaries, the calibration of
the FETCH_SIZE / WRITE_SIZE counters, and the one-GPU guard.
"""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from rank_bottleneck_online_amd import synth  # noqa: E402

SWIGLU_BWD = ("_ZN3rbo11gemm_kernelINS_3CfgIDF16bLi256ELi128ELi4ELi2ELb1ELb1ELi3EEENS_12EpiSwigluBwdELi0EEEvNS_8"
              "GemmGeomENS_7GemmOpsENT0_4ArgsE")
DOWN1 = ("_ZN3rbo11gemm_kernelINS_3CfgIDF16bLi256ELi256ELi2ELi4ELb1ELb1ELi1EEENS_7EpiDownILb1ELb0EEELi0EEEvNS_8"
         "GemmGeomENS_7GemmOpsENT0_4ArgsE")
WGRAD = ("_ZN3rbo11gemm_kernelINS_3CfgIDF16bLi128ELi128ELi2ELi4ELb0ELb0ELi1EEENS_8EpiStoreILb1EEELi4EEEvNS_8"
         "GemmGeomENS_7GemmOpsENT0_4ArgsE")


def test_mlp_step_flops_are_three_forwards_plus_the_recompute():
    w = synth.WORKLOADS["llama2_7b_mlp"]
    k = bench.mlp_kernel_flops(w["T"], w["d"], w["r"], w["ffn"])
    fwd = sum(k[n] for n in ("mlp_down1", "mlp_up1_swiglu", "mlp_down2", "mlp_up2"))
    rec = bench.recompute_flops("lrmlp", w)
    assert sum(k.values()) == 3 * fwd + rec
    assert round(sum(k.values()) / 1e9, 1) == 2650.0


def test_btp_share_flops_are_three_forwards_plus_the_recompute():
    w = synth.WORKLOADS["llama2_13b_btp_share_tp4"]
    ds = w["d_global"] // w["P"]
    k = bench.btp_kernel_flops(w["T"], w["r"], ds)
    fwd = k["btp_u"] + k["btp_p"]
    assert sum(k.values()) == 3 * fwd + bench.recompute_flops("btp", w)
    # the u recompute and e = dp A_s^T are one product each
    assert k["btp_u_re"] == k["btp_u_bwd"] == k["btp_u"]


def test_lrblock_backward_is_twice_the_forward():
    k = bench.lrblock_kernel_flops(300, 512, 128, 3, 320, bwd=True)
    fwd = k["lrblock_down"] + k["lrblock_up"]
    assert sum(k.values()) == 3 * fwd


def test_short_kernel_names():
    assert bench.short_kernel_name(SWIGLU_BWD) == "gemm bf16 256x128 waves 4x2 KC/KC nacc=3 EpiSwigluBwd"
    assert bench.short_kernel_name(DOWN1) == "gemm bf16 256x256 waves 2x4 KC/KC nacc=1 EpiDown<1,0>"
    assert bench.short_kernel_name(WGRAD) == "gemm bf16 128x128 waves 2x4 MC/NC nacc=1 EpiStore<1> tag 4"
    assert bench.short_kernel_name("void rbo::colsum_kernel(float const*)") == "rbo::colsum_kernel"


def test_each_mlp_label_names_one_kernel():
    """Every launch label of the MLP step maps to exactly one of the step's
    kernel instantiations (the weight-gradient products carry a launch tag)."""
    names = [SWIGLU_BWD, DOWN1, WGRAD]
    for tag in (1, 2, 3):
        names.append(WGRAD.replace("EELi4EEEv", f"EELi{tag}EEEv"))
    for lab in ("mlp1_dB", "mlp1_dA", "mlp_dB2", "mlp_dA2", "mlp_recompute_swiglu_bwd", "mlp_down1"):
        hits = [n for n in names if bench.MLP_LABEL_PATTERNS[lab] in n]
        assert len(hits) == 1, (lab, hits)


def _gemm_name(cfg, epi, tag=0):
    return f"_ZN3rbo11gemm_kernelINS_3CfgIDF16b{cfg}EEENS_{epi}ELi{tag}EEEvNS_8GemmGeomENS_7GemmOpsENT0_4ArgsE"


def test_each_btp_label_names_one_kernel():
    """The tensor-parallel share's seven launches run seven distinct kernel
    instantiations, and each label pattern picks out exactly its own."""
    kcnc, kckc, mcnc = "Li192ELi256ELi2ELi4ELb1ELb0ELi1", "Li192ELi256ELi2ELi4ELb1ELb1ELi1", "Li128ELi128ELi2ELi4ELb0ELb0ELi1"
    step = {"btp_u": _gemm_name(kcnc, "7EpiBtpU"), "btp_p": _gemm_name(kcnc, "7EpiBtpP"),
            "btp_u_re": _gemm_name(kcnc, "8EpiStoreILb1EE"), "btp_u_bwd": _gemm_name(kckc, "10EpiBtpEBwd"),
            "btp_dz": _gemm_name(kckc, "8EpiStoreILb0EE"), "btp_dA": _gemm_name(mcnc, "8EpiStoreILb1EE", 5),
            "btp_dB": _gemm_name(mcnc, "8EpiStoreILb1EE", 6)}
    assert set(bench.BTP_LABEL_PATTERNS) == set(step)
    for lab, pat in bench.BTP_LABEL_PATTERNS.items():
        hits = [k for k, n in step.items() if pat in n]
        assert hits == [lab], (lab, hits)
    patterns, flops, rw = bench.counter_workload("llama2_13b_btp_share_tp4")
    assert set(flops) == set(rw) == set(patterns)
    # e.g. dz = du B_s^T reads du [T, S] and B_s [r, S] in bf16, writes dz [T, r]
    w = synth.WORKLOADS["llama2_13b_btp_share_tp4"]
    T, r, S = w["T"], w["r"], w["d_global"] // w["P"]
    assert rw["btp_dz"] == (2 * (T * S + r * S), 2 * T * r)


def test_shared_instantiations_are_summarised_per_kernel(tmp_path):
    """The chained layer's weight-gradient instantiation serves several
    launches: the MFMA table lists it once, with its dispatch count and
    per-dispatch means."""
    assert bench.counter_workload("llama2_40b_layer_chained")[0] is None
    path = str(tmp_path / "m.csv")
    rows = []
    for util, mops in ((40.0, 1e9), (60.0, 3e9)):
        rows += [(WGRAD, "MfmaUtil", util), (WGRAD, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops)]
    rows += [(DOWN1, "MfmaUtil", 50.0), (DOWN1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2e9),
             ("rbo::colsum_kernel", "MfmaUtil", 0.0)]
    _counter_csv(path, rows)
    table = bench.mfma_summary(path, "t", "c", "llama2_40b_layer_chained")
    body = [ln for ln in table.splitlines() if ln.startswith("| gemm")]
    assert len(body) == 2
    wg = [c.strip() for c in [ln for ln in body if "tag 4" in ln][0].strip("|").split("|")]
    assert wg[1] == "2" and wg[2] == "50.0" and wg[3] == f"{2e9 * 512 / 1e9:.1f}"


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, counter, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_calibration(tmp_path):
    # A 1 GiB copy that FETCH_SIZE reports as half its size and WRITE_SIZE
    # as its size: fetched bytes are scaled by 2, written bytes by 1; two
    # dispatches of a kernel are averaged.
    fetch, write = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    _counter_csv(fetch, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0),
                         (SWIGLU_BWD, "FETCH_SIZE", 1000.0), (SWIGLU_BWD, "FETCH_SIZE", 3000.0)])
    _counter_csv(write, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0),
                         (SWIGLU_BWD, "WRITE_SIZE", 500.0), (SWIGLU_BWD, "WRITE_SIZE", 500.0)])
    tj = bench.traffic_json(fetch, write, "llama2_7b_mlp", 1024)
    assert tj["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert tj["calibration"]["write_scale"] == pytest.approx(1.0)
    k = tj["kernels"]["mlp_recompute_swiglu_bwd"]
    assert k["dispatches"] == 2
    assert k["fetch_bytes"] == 2000 * 1024 * 2
    assert k["write_bytes"] == 500 * 1024
    assert tj["source_digest"] == bench.source_digest()


def test_traffic_rates_from_dispatch_times(tmp_path):
    # Two dispatches of 100 and 300 us in each counter run: the launch
    # averages 200 us, and the table turns (fetched + written) bytes into
    # GB/s against the HBM peak.
    fetch, write = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    for path, cnt, cal in ((fetch, "FETCH_SIZE", 1048576.0), (write, "WRITE_SIZE", 1048576.0)):
        with open(path, "w", newline="") as f:
            wr = csv.DictWriter(f, fieldnames=cols)
            wr.writeheader()
            wr.writerow(dict(zip(cols, (1, "__amd_rocclr_copyBuffer", cnt, cal, 0, 10))))
            wr.writerow(dict(zip(cols, (2, SWIGLU_BWD, cnt, 390625.0, 1000, 101000))))
            wr.writerow(dict(zip(cols, (3, SWIGLU_BWD, cnt, 390625.0, 200000, 500000))))
    tj = bench.traffic_json(fetch, write, "llama2_7b_mlp", 1024)
    k = tj["kernels"]["mlp_recompute_swiglu_bwd"]
    assert k["avg_ms_profiled"] == pytest.approx(0.2)
    assert k["fetch_bytes"] == k["write_bytes"] == 400_000_000
    jp = tmp_path / "t.json"
    jp.write_text(json.dumps(tj))
    row = [ln for ln in bench.traffic_table(str(jp), "t", "c").splitlines() if ln.startswith("| mlp_recompute")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[7] == "200.0" and cells[8] == "4000" and cells[9] == "50.0"


def test_traffic_needs_the_calibration_copy(tmp_path):
    fetch, write = str(tmp_path / "f.csv"), str(tmp_path / "w.csv")
    _counter_csv(fetch, [(SWIGLU_BWD, "FETCH_SIZE", 1000.0)])
    _counter_csv(write, [(SWIGLU_BWD, "WRITE_SIZE", 500.0)])
    with pytest.raises(SystemExit):
        bench.traffic_json(fetch, write, "llama2_7b_mlp", 1024)


def test_code_text_drops_comments_only():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* the\n  answer */ }\n"
    b = "int f(int x) {\n  return 2 * x;\n}\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(b.replace("2 *", "3 *"))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
