"""Host logic of bench.py, no GPU: the reductions of rocprofv3 counter files into
the committed summaries, the digest that ties a summary to the kernel sources, and
the refusal of a multi-GPU run."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
        "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
        "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
DQ = "void hga::(anonymous namespace)::attend_bwd_dq_bf16_kernel<128, 4, 4>(hga::(anonymous namespace)::BwdArgs)"
FWD = "void hga::(anonymous namespace)::attend_fwd_bf16_kernel<128, 4, 4>(hga::(anonymous namespace)::FwdArgs)"
SUM = "void hga::(anonymous namespace)::summaries_kernel<unsigned short, 128>(unsigned short const*)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float>>(int)"


def _write(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=COLS)
        wr.writeheader()
        for i, (name, grid, counter, value) in enumerate(rows):
            r = {c: 0 for c in COLS}
            r.update(Dispatch_Id=i + 1, Kernel_Name=name, Grid_Size=grid, Counter_Name=counter,
                     Counter_Value=value)
            wr.writerow(r)


def test_traffic_summary_scales_by_the_copy_kernel(tmp_path):
    mib = 8
    n = mib << 20
    # the copy kernel reports half its bytes read and all its bytes written (KiB)
    fetch = [(COPY, 1, "FETCH_SIZE", n / 2 / 1024), (DQ, 131072, "FETCH_SIZE", 1000.0),
             (DQ, 131072, "FETCH_SIZE", 1200.0), (SUM, 458752, "FETCH_SIZE", 5.0),
             (SUM, 65536, "FETCH_SIZE", 7.0), (SUM, 65536, "FETCH_SIZE", 9.0)]
    write = [(COPY, 1, "WRITE_SIZE", n / 1024), (DQ, 131072, "WRITE_SIZE", 64.0), (DQ, 131072, "WRITE_SIZE", 64.0),
             (SUM, 458752, "WRITE_SIZE", 1.0), (SUM, 65536, "WRITE_SIZE", 2.0), (SUM, 65536, "WRITE_SIZE", 2.0)]
    _write(tmp_path / "f.csv", fetch)
    _write(tmp_path / "w.csv", write)
    s = bench.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), mib, "qwen3_8b_layer_ctx16k")
    assert s["fetch_factor"] == pytest.approx(2.0) and s["write_factor"] == pytest.approx(1.0)
    dq = s["kernels"]["attend_bwd_dq"]
    assert dq["fetch_bytes_per_launch"] == round(2.0 * 1100.0 * 1024)
    assert dq["write_bytes_per_launch"] == 64 * 1024
    assert dq["hbm_bytes_per_launch"] == dq["fetch_bytes_per_launch"] + dq["write_bytes_per_launch"]
    # the most frequent grid of a kernel is the step's (the one-off history build is dropped)
    sm = s["kernels"]["summaries"]
    assert sm["launches"] == 2 and sm["fetch_bytes_per_launch"] == round(2.0 * 8.0 * 1024)
    assert s["source_sha256"] == bench.kernel_source_digest("qwen3_8b_layer_ctx16k")


def test_traffic_summary_needs_one_calibration_dispatch(tmp_path):
    _write(tmp_path / "f.csv", [(DQ, 131072, "FETCH_SIZE", 1.0)])
    _write(tmp_path / "w.csv", [(DQ, 131072, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 8, "qwen3_8b_layer_ctx16k")


def test_mfma_summary_averages_each_kernel(tmp_path):
    rows = [(DQ, 131072, "MfmaUtil", 30.0), (DQ, 131072, "MfmaFlopsBF16", 1.0e9),
            (DQ, 131072, "MfmaUtil", 34.0), (DQ, 131072, "MfmaFlopsBF16", 1.2e9),
            (FWD, 131072, "MfmaUtil", 25.0), (FWD, 131072, "MfmaFlopsBF16", 5.0e8),
            (SUM, 65536, "MfmaUtil", 0.0), (SUM, 65536, "MfmaFlopsBF16", 0.0)]
    _write(tmp_path / "m.csv", rows)
    s = bench.mfma_summary(str(tmp_path / "m.csv"), "qwen3_8b_layer_ctx16k")
    assert s["kernels"]["attend_bwd_dq"] == {"launches": 2, "mfma_util_pct": 32.0,
                                             "mfma_bf16_flops_per_launch": 1.1e9}
    assert s["kernels"]["attend_fwd"]["mfma_util_pct"] == 25.0
    assert s["kernels"]["summaries"]["mfma_bf16_flops_per_launch"] == 0


def test_stall_summary_gives_fractions_of_wave_cycles(tmp_path):
    a = [(DQ, 131072, "SQ_WAVE_CYCLES", 1000.0), (DQ, 131072, "SQ_WAIT_ANY", 400.0),
         (DQ, 131072, "SQ_WAIT_INST_ANY", 300.0), (DQ, 131072, "SQ_ACTIVE_INST_ANY", 300.0),
         (DQ, 131072, "SQ_WAVE_CYCLES", 3000.0), (DQ, 131072, "SQ_WAIT_ANY", 1200.0),
         (DQ, 131072, "SQ_WAIT_INST_ANY", 900.0), (DQ, 131072, "SQ_ACTIVE_INST_ANY", 900.0),
         (SUM, 458752, "SQ_WAVE_CYCLES", 50.0), (SUM, 65536, "SQ_WAVE_CYCLES", 10.0),
         (SUM, 65536, "SQ_WAIT_ANY", 8.0), (SUM, 65536, "SQ_WAVE_CYCLES", 10.0), (SUM, 65536, "SQ_WAIT_ANY", 8.0)]
    b = [(DQ, 131072, "SQ_VALU_MFMA_BUSY_CYCLES", 800.0), (DQ, 131072, "SQ_VALU_MFMA_COEXEC_CYCLES", 200.0),
         (DQ, 131072, "SQ_LDS_IDX_ACTIVE", 100.0), (DQ, 131072, "SQ_LDS_BANK_CONFLICT", 5.0)]
    _write(tmp_path / "a.csv", a)
    _write(tmp_path / "b.csv", b)
    s = bench.stall_summary([str(tmp_path / "a.csv"), str(tmp_path / "b.csv")], "qwen3_8b_layer_ctx16k")
    dq = s["kernels"]["attend_bwd_dq"]
    assert dq["launches"] == 2
    assert dq["counters_per_launch"]["SQ_WAVE_CYCLES"] == 2000
    assert (dq["wait_dependency_frac"], dq["wait_issue_frac"], dq["active_any_frac"]) == (0.4, 0.3, 0.3)
    assert dq["valu_coissue_frac_of_mfma_busy"] == 0.25
    assert dq["lds_bank_conflict_frac"] == 0.05
    # the step's summaries launches (the most frequent grid), not the one-off history build
    assert s["kernels"]["summaries"]["launches"] == 2
    assert s["kernels"]["summaries"]["wait_dependency_frac"] == 0.8


def test_summaries_are_tied_to_the_kernel_sources(tmp_path, monkeypatch):
    summ = {"workload": "qwen3_8b_layer_ctx16k", "source_sha256": bench.kernel_source_digest("qwen3_8b_layer_ctx16k"),
            "kernels": {"attend_bwd_dq": {"hbm_bytes_per_launch": 123, "mfma_util_pct": 40.0,
                                          "mfma_bf16_flops_per_launch": 2.0e9}}}
    path = tmp_path / "s.json"
    path.write_text(json.dumps(summ))
    monkeypatch.setitem(bench.PMC_SUMMARIES, "qwen3_8b_layer_ctx16k", str(path))
    monkeypatch.setitem(bench.MFMA_SUMMARIES, "qwen3_8b_layer_ctx16k", str(path))
    assert bench.measured_traffic("attend_bwd_dq", "qwen3_8b_layer_ctx16k") == 123
    mc = bench.measured_mfma("attend_bwd_dq", "qwen3_8b_layer_ctx16k", 0.040)
    assert mc == {"util_pct": 40.0, "hw_bf16_tflops": 50.0, "frac_of_peak": 0.02}
    # any other digest (the kernels changed since the counters were taken): no figure
    summ["source_sha256"] = "0" * 64
    path.write_text(json.dumps(summ))
    assert bench.measured_traffic("attend_bwd_dq", "qwen3_8b_layer_ctx16k") is None
    assert bench.measured_mfma("attend_bwd_dq", "qwen3_8b_layer_ctx16k", 0.040) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_digest_ignores_comments_only(tmp_path, monkeypatch):
    import shutil
    for name in bench.WORKLOAD_SOURCES["decode_b8_ctx32k"]:
        shutil.copy(os.path.join(bench.CSRC, name), tmp_path / name)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    d0 = bench.kernel_source_digest("decode_b8_ctx32k")
    p = tmp_path / "decode.hip"
    src = p.read_text()
    p.write_text("// a new comment line\n" + src.replace("\n", "\n\n", 3) + "\n/* trailing */\n")
    assert bench.kernel_source_digest("decode_b8_ctx32k") == d0
    p.write_text(src + "\nstatic int unused_for_test = 1;\n")
    assert bench.kernel_source_digest("decode_b8_ctx32k") != d0
    assert bench._code_only('x = "a // b"; // tail\ny /* z */ = 1;') == 'x = "a // b"; y = 1;'
