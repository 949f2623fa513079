"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the
algorithmic work per stage, the kernel-selection rule it names, the input
rotation count and the fractions of the measured peaks."""
import json
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_touching_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_stage_work_of_the_skewed_layer():
    w = workloads.WORKLOADS["skewed"]
    N, active = 32768.0, 56.0
    work = bench.stage_work(w, N, active, 2, gathers=True)
    d, F, T, E, k = w.d, w.F, w.T, w.E, w.k
    assert work["expert_up"]["flops"] == 2 * N * d * F
    assert work["expert_down"]["flops"] == 2 * N * F * d
    # active experts' weights once, the pairs' input rows and output rows once: 7 784 628 224 bytes
    assert work["expert_up"]["bytes"] == 56 * F * d * 2 + 32768 * d * 2 + 32768 * F * 2 == 7784628224
    assert work["route"]["bytes"] == T * d * 2 + d * E * 2 + T * k * 8
    assert work["combine"]["bytes"] == N * d * 2 + T * k * 8 + T * d * 2
    # gathering: the dispatch moves indices only; with the row copy it reads X and writes the rows
    assert work["dispatch"]["bytes"] == T * k * 12
    assert bench.stage_work(w, N, active, 2, gathers=False)["dispatch"]["bytes"] == T * d * 2 + N * d * 2 + T * k * 12


@pytest.mark.parametrize("name,stage,want", [
    ("skewed", "expert_up", "grouped_gemm_bf16_256<true, true, 8>"),
    ("skewed", "expert_down", "grouped_gemm_bf16_256<false, false, 8>"),
    ("capacity", "expert_down", "grouped_gemm_bf16_256<false, false, 8>"),
    ("decode", "expert_up", "grouped_gemm_bf16_gemv<true, 2, true>"),
    ("decode", "expert_down", "grouped_gemm_bf16_gemv<false, 2, false>"),
    ("tiny", "expert_up", "grouped_gemm_kernel<float, 64, 64, 2, 2, true>"),
])
def test_kernel_named_for_each_workload(name, stage, want):
    w = workloads.WORKLOADS[name]
    cap = -1 if name != "capacity" else -(-w.T // w.E) * w.k
    assert bench.gemm_kernel_name(w, cap, stage, gathers=w.dtype == "bf16") == want


def test_kernel_name_follows_the_decode_kernel_rule():
    """Few rows per expert: the decode kernel up to a bound of 16, or up to 64
    while the batch averages at most 16 rows per expert; else the 16-row-tile
    kernel up to 64, the 256x256 kernel beyond."""
    base = workloads.WORKLOADS["decode"]
    mk = lambda T: workloads.Workload("t", T=T, d=base.d, E=base.E, k=base.k, F=base.F, dtype="bf16", seed=0)  # noqa
    assert bench.gemm_kernel_name(mk(64), -1, "expert_up", True) == "grouped_gemm_bf16_gemv<true, 4, true>"
    assert bench.gemm_kernel_name(mk(128), -1, "expert_up", True) == "grouped_gemm_bf16_256<true, true, 8>"
    few = workloads.Workload("t", T=64, d=base.d, E=4, k=2, F=base.F, dtype="bf16", seed=0)  # 128 rows > 16 * 4
    assert bench.gemm_kernel_name(few, -1, "expert_down", False) == "grouped_gemm_bf16_skinny<false, 4>"


def test_rotation_sets_exceed_the_last_level_cache():
    for name, want in (("skewed", 8), ("prefill", 32), ("capacity", 8)):
        w = workloads.WORKLOADS[name]
        n = bench.rotation_sets(w, w.T, w.d, w.F, w.k, 2)
        assert n == want and n * w.T * w.d * 2 >= (1 << 30)


def test_fractions_of_the_measured_peaks():
    ach = {"hbm_gbs": 5000.0, "bf16_gemm_tflops": 1200.0}
    mfma = {"bound": "mfma", "achieved": 1000.0, "peak": bench.PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    hbm = {"bound": "hbm", "achieved": 6000.0, "peak": bench.PEAK_HBM_GBS, "unit": "GB/s"}
    f32 = {"bound": "mfma", "achieved": 10.0, "peak": bench.PEAK_F32_TFLOPS, "unit": "TFLOP/s"}
    for r in (mfma, hbm, f32):
        bench.add_achievable(r, ach)
    assert mfma["frac_of_achievable"] == pytest.approx(1000.0 / 1200.0, abs=1e-4)
    assert hbm["frac_of_achievable"] == pytest.approx(1.2)
    assert "frac_of_achievable" not in f32  # the fp32 layer has no measured fp32 reference


def test_gemm_code_hash_ignores_comments(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("// a comment line\nint f(int x) {\n\n  return x + 1;   // another comment\n}\n")
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.gemm_code_sha1(a) == bench.gemm_code_sha1(b) != bench.gemm_code_sha1(c)
