"""Host logic of bench.py (no GPU): the per-kernel roofline figures, the
source hash that ties a committed profile to the kernel sources, the readers
of committed profiles, the rocprofv3 summaries, the memory-controller
activity average, and the one-GPU guard."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refresh_windows_leave_out_the_window_before_the_first_refresh():
    # busy 49% for 3 windows of 1 s after the first refresh; what came before it
    # (another phase at 90%) must not count
    refreshes = [(5_000_000_000, 1_000_000)]
    for i in range(1, 4):
        refreshes.append((5_000_000_000 + i * 1_000_000_000, 1_000_000 + 49_000 * i))
    pct, windows, span = bench.refresh_window_activity(refreshes)
    assert windows == 3 and span == pytest.approx(3000.0)
    assert pct == pytest.approx(49.0)


def test_refresh_windows_weight_by_length():
    # 1 s at 10% then 3 s at 30%: 25% overall, not the mean of the two windows
    r = [(0, 0), (1_000_000_000, 10_000), (4_000_000_000, 10_000 + 90_000)]
    pct, windows, span = bench.refresh_window_activity(r)
    assert windows == 2 and span == pytest.approx(4000.0)
    assert pct == pytest.approx(25.0)


@pytest.mark.parametrize("refreshes", [[], [(7, 8)]])
def test_refresh_windows_need_two_refreshes(refreshes):
    assert bench.refresh_window_activity(refreshes) == (None, 0, 0.0)


def test_kernel_figures_per_launch_flops_and_fraction():
    N, H, V, kept = 8192, 4096, 128256, 16384
    steps = 2
    log = []
    for _ in range(steps):
        log.append(("fused_fwd_kernel<unsigned short, true, true, true>", 0.8))
        log.append(("fwd_lse_kernel<unsigned short, true, true, true>", 4.0))
        log += [("bwd_dz_kernel<unsigned short, true, true>", 0.7)] * 7
        log += [("bwd_dx_kernel<unsigned short, 1, false>", 0.7)] * 8
        log += [("bwd_dw_kernel<unsigned short, false>", 0.7)] * 8
        log.append(("fwd_combine_kernel", 0.01))
    k = bench.kernel_figures(log, steps, N, H, V, kept, 2500.0)
    assert k["bwd_dz_kernel"]["launches_per_step"] == 7
    assert k["bwd_dz_kernel"]["flops_per_launch"] == pytest.approx(2.0 * N * H * (V - kept) / 7)
    assert k["bwd_dw_kernel"]["flops_per_launch"] == pytest.approx(2.0 * N * H * V / 8)
    assert k["fused_fwd_kernel"]["flops_per_launch"] == pytest.approx(2.0 * N * H * kept)
    fl = 2.0 * N * H * (V - kept)
    assert k["fwd_lse_kernel"]["tflops"] == pytest.approx(fl / 4.0e-3 / 1e12)
    assert k["fwd_lse_kernel"]["frac"] == pytest.approx(fl / 4.0e-3 / 1e12 / 2500.0)
    assert "tflops" not in k["fwd_combine_kernel"]
    assert k["fwd_combine_kernel"]["avg_us"] == pytest.approx(10.0)
    # the whole vocabulary recomputed: no kept-value kernel flops
    k2 = bench.kernel_figures(log, steps, N, H, V, 0, 2500.0)
    assert k2["fused_fwd_kernel"]["avg_us"] == pytest.approx(800.0)
    assert "tflops" not in k2["fused_fwd_kernel"]


def test_source_hash_ignores_comments_and_whitespace():
    a = {"k.hip": "int f(int x) { return x + 1; } // one\n"}
    b = {"k.hip": "/* header */\nint f(int x)\n{\n    return x + 1;   // other words\n}\n"}
    c = {"k.hip": "int f(int x) { return x + 2; }"}
    assert bench.kernel_source_hash(a) == bench.kernel_source_hash(b)
    assert bench.kernel_source_hash(a) != bench.kernel_source_hash(c)
    # the file name is part of it
    assert bench.kernel_source_hash(a) != bench.kernel_source_hash({"j.hip": a["k.hip"]})


def _fake_root(tmp_path, monkeypatch, kernel_code="int k() { return 1; }"):
    csrc = tmp_path / "lm_head_cross_flce_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text(kernel_code)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return bench.kernel_source_hash()


def test_recorded_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    h = _fake_root(tmp_path, monkeypatch)
    p = tmp_path / "profiles" / "fwd_lse_kernel_wl_traffic.md"
    p.write_text(f"source hash: `{h}`\n\ntraffic_bytes_per_launch: 1.25e+10\n")
    assert bench.recorded_traffic("fwd_lse_kernel", "wl") == pytest.approx(1.25e10)
    assert bench.recorded_traffic("bwd_dw_kernel", "wl") is None
    p.write_text("source hash: `0123456789abcdef`\n\ntraffic_bytes_per_launch: 1.25e+10\n")
    assert bench.recorded_traffic("fwd_lse_kernel", "wl") is None


def test_recorded_trace_sums_a_kernel_pair(tmp_path, monkeypatch):
    h = _fake_root(tmp_path, monkeypatch)
    p = tmp_path / "profiles" / "flce_step_wl_kernel_trace.md"
    p.write_text(f"Source hash `{h}`\n\nkernel_avg_us: bwd_dw_kernel 700.00 over 8 launches\n"
                 "kernel_avg_us: bwd_db_kernel 5.50 over 8 launches\n")
    r = bench.recorded_trace("bwd_dw_kernel", "wl")
    assert r["avg_us"] == pytest.approx(700.0) and r["file"].endswith("flce_step_wl_kernel_trace.md")
    assert bench.recorded_trace("bwd_dw_kernel + bwd_db_kernel", "wl")["avg_us"] == pytest.approx(705.5)
    assert bench.recorded_trace("fwd_lse_kernel", "wl") is None
    (tmp_path / "lm_head_cross_flce_amd" / "csrc" / "k.hip").write_text("int k() { return 2; }")
    assert bench.recorded_trace("bwd_dw_kernel", "wl") is None


def test_summarize_trace_averages_over_template_instances(tmp_path, capsys):
    rows = [("void flce::bwd_dx_kernel<unsigned short, 1, false>(flce::DxArgs)", 0, 700_000),
            ("void flce::bwd_dx_kernel<unsigned short, 1, false>(flce::DxArgs)", 0, 720_000),
            ("void flce::bwd_dx_kernel<unsigned short, 2, false>(flce::DxArgs)", 0, 600_000),
            ("flce::fwd_combine_kernel(flce::CombineArgs)", 0, 9_000)]
    with open(tmp_path / "run_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for n, s, e in rows:
            f.write(f"\"{n}\",{s},{e}\n")
    bench.summarize_trace(str(tmp_path))
    out = capsys.readouterr().out
    assert "kernel_avg_us: bwd_dx_kernel 673.33 over 3 launches" in out
    assert "kernel_avg_us: fwd_combine_kernel 9.00 over 1 launches" in out
    # the warm average leaves out an instance's first launch
    assert "| `flce::bwd_dx_kernel<unsigned short, 1, false>` | 2 | 710.0 | 720.0 |" in out


def test_summarize_pmc_per_dispatch(tmp_path, capsys):
    with open(tmp_path / "pmc_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        f.write("1,\"flce::fwd_lse_kernel<unsigned short>(A)\",FETCH_SIZE,100\n")
        f.write("2,\"flce::fwd_lse_kernel<unsigned short>(A)\",FETCH_SIZE,300\n")
        f.write("3,\"flce::bwd_dz_kernel<unsigned short>(B)\",FETCH_SIZE,50\n")
    bench.summarize_pmc(str(tmp_path))
    out = capsys.readouterr().out
    assert "| `flce::fwd_lse_kernel<unsigned short>` | FETCH_SIZE | 200 | 2 |" in out
    assert "| `flce::bwd_dz_kernel<unsigned short>` | FETCH_SIZE | 50 | 1 |" in out


def test_metric_names_the_workload_shape():
    class W:
        N, H, V, dtype = 4096, 2048, 32000, "bf16"
    assert bench.metric_for(W) == "FLCE fwd+bwd tokens/s and % bf16 MFMA peak at N=4096,H=2048,V=32000"
    W.dtype = "f16"
    assert "fp16 inputs" in bench.metric_for(W)
    W.dtype = "f32"
    assert "fp32 MFMA peak" in bench.metric_for(W)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""   # no JSON line
