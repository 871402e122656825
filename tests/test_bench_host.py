"""Host-side logic of bench.py, on the CPU: the one-GPU contract, the
rocprofv3 summaries (counter scaling, per-predecessor split), the roofline's
choice of kernel, and the rule that a counter figure is used only while the
kernel sources still hash to the digest its summary was taken on."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

MAIN = "bn2d_train_fwd_bwd_nchw_256x32x32x32_f32"
BIG = "bn2d_train_fwd_bwd_nchw_64x256x56x56_bf16"


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          env=e, timeout=300, cwd=ROOT)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    r = _run(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_list_names_the_workloads():
    r = _run(["--list"])
    assert r.returncode == 0
    names = r.stdout.split()
    assert MAIN in names and BIG in names
    assert "rms_bwd_2048x8192_bf16_saved_rms" in names and "ln_bwd_16x512x1600_xf32_dybf16_wbf16" in names


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _trace(path, seq):
    """seq: (kernel name, duration in us) in dispatch order."""
    t, rows = 1000, []
    for i, (name, us) in enumerate(seq):
        rows.append([i + 1, name, t, t + int(us * 1000)])
        t += int(us * 1000)
    _write_csv(path, ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)


def test_summarize_workload_scales_the_counters(tmp_path):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counter reads for the calibration add of two 32 MiB reads and one 32 MiB
    write; durations and the split by predecessor come from the trace."""
    n = 8 * 1024 * 1024
    stats = "void nh::bn_stats_kernel<float, 4, 6>(float const*)"
    grads = "void nh::bn_grad_sums_kernel<float, 4, 6, 0>(float const*)"
    seq = [(stats, 7.0), (grads, 12.0)] * 6
    _trace(tmp_path / "trace.csv", seq)
    # counters read half the true bytes on fetch (scale 2) and all of them on write (scale 1)
    _write_csv(tmp_path / "fetch.csv", ["Kernel_Name", "Counter_Value"],
               [[stats, 33554432 / 1024 / 2], [grads, 67108864 / 1024 / 2]] * 2)
    _write_csv(tmp_path / "write.csv", ["Kernel_Name", "Counter_Value"], [[stats, 16], [grads, 32]] * 2)
    cal = "void nh::calib_add4_kernel(float const*)"
    _write_csv(tmp_path / "cf.csv", ["Kernel_Name", "Counter_Value"], [[cal, 2 * n * 4 / 1024 / 2]] * 3)
    _write_csv(tmp_path / "cw.csv", ["Kernel_Name", "Counter_Value"], [[cal, n * 4 / 1024]] * 3)
    out = tmp_path / "summary.txt"
    bench.summarize_workload(MAIN, str(tmp_path / "trace.csv"), str(tmp_path / "fetch.csv"),
                             str(tmp_path / "write.csv"), str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), str(out))
    text = out.read_text().splitlines()
    assert "fetch_scale: 2.00000" in text and "write_scale: 1.00000" in text
    assert f"source_sha256_16: {bench.sources_digest(bench.workload_sources(MAIN))}" in text
    rows = {ln[:70].strip(): ln[70:].split() for ln in text if ln.startswith("nh::")}
    s, g = rows["nh::bn_stats_kernel<float, 4, 6>"], rows["nh::bn_grad_sums_kernel<float, 4, 6, 0>"]
    assert int(s[0]) == 6 and float(s[1]) == pytest.approx(7.0)
    assert float(s[4]) == pytest.approx(33.55, abs=0.01) and float(s[5]) == pytest.approx(0.02, abs=0.01)
    assert float(g[1]) == pytest.approx(12.0)
    assert float(g[4]) == pytest.approx(67.11, abs=0.01) and float(g[5]) == pytest.approx(0.03, abs=0.01)
    # every grad_sums dispatch followed a stats dispatch
    i = text.index(next(ln for ln in text if ln.startswith("nh::bn_grad_sums")))
    assert text[i + 1].split()[:2] == ["after", "bn_stats_kernel<float,"]
    assert int(text[i + 1].split()[-2]) == 6


def test_summarize_stats_splits_by_predecessor(tmp_path):
    a = "void nh::bn_apply_kernel<float, 4, 1, 6, 0>(float const*)"
    b = "void nh::bn_stats_kernel<float, 4, 6>(float const*)"
    seq = [(b, 7.0), (a, 8.0)] * 5 + [(b, 6.0)] * 6
    _trace(tmp_path / "trace.csv", seq)
    _write_csv(tmp_path / "stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[b, 11, 6450, 6000, 7000], [a, 5, 8000, 8000, 8000]])
    out = tmp_path / "s.txt"
    bench.summarize_stats(str(tmp_path / "stats.csv"), str(tmp_path / "trace.csv"), str(out), "cmd")
    text = out.read_text().splitlines()
    assert text[1] == "command: cmd"
    i = next(k for k, ln in enumerate(text) if ln.startswith("nh::bn_stats_kernel"))
    after = {ln.split()[1]: (int(ln.split()[-2]), float(ln.split()[-1])) for ln in text[i + 1:i + 4]
             if ln.startswith("    after")}
    # dispatch order: s a s a s a s a s a s s s s s s.  After an apply: four at
    # 7.0 and one at 6.0; after a stats: five at 6.0; the first stats has no
    # predecessor (a group of one, below the five a line needs)
    assert after["bn_apply_kernel<float,"] == (5, pytest.approx(6.8))
    assert after["bn_stats_kernel<float,"] == (5, pytest.approx(6.0))
    assert len(after) == 2


def _res(**kernels):
    return {"kernels": {k: {"avg_us": us, "input_from": src, "gbs": 1000.0 * i, "frac_of_peak": 0.1 * i,
                            "bytes": 100 * i}
                        for i, (k, (us, src)) in enumerate(kernels.items(), 1)}}


def test_roofline_takes_the_slowest_kernel_fed_from_hbm():
    res = _res(bn_stats=(7.5, "hbm"), bn_apply=(7.6, "infinity cache"), bn_grad_sums=(12.8, "hbm"),
               bn_dx=(30.0, "infinity cache"))
    r = bench._roofline(res, "no_such_workload")
    assert r["kernel"] == "bn_grad_sums"
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert r["achieved"] == 3000.0 and r["frac"] == pytest.approx(0.3) and r["avg_us"] == 12.8
    assert r["traffic"] is None  # no summary for this workload


def _fake_root(tmp_path):
    csrc = tmp_path / "bwd_bn_stats_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES:
        (csrc / f).write_text(f"// {f}\n")
    (tmp_path / "profiles").mkdir()
    return csrc


def test_traffic_only_while_the_sources_match(tmp_path, monkeypatch):
    csrc = _fake_root(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.sources_digest(bench.workload_sources(MAIN))
    name = "nh::bn_grad_sums_kernel<float, 4, 6, 0>"
    (tmp_path / "profiles" / f"{MAIN}.txt").write_text(
        f"# {MAIN}\nsource_sha256_16: {digest}\n\n"
        f"{'kernel':70s} calls avg_us min_us max_us read_MB write_MB\n"
        f"{name:70s} {10:6d} {12.8:8.3f} {12.0:8.3f} {13.0:8.3f} {67.12:9.2f} {0.02:9.2f}\n")
    assert bench._traffic_for("bn_grad_sums", MAIN) == 67140000
    assert bench._traffic_for("bn_dx", MAIN) is None          # no line for that kernel
    # a rows source is not one of the BatchNorm kernels' sources: the figure stands
    (csrc / "rows_kernels.hip").write_text("// changed\n")
    assert bench._traffic_for("bn_grad_sums", MAIN) == 67140000
    # a comment changed in a BatchNorm source: the summary no longer describes the build
    (csrc / "bn_kernels.hip").write_text("// bn_kernels.hip, edited\n")
    assert bench._traffic_for("bn_grad_sums", MAIN) is None


def test_workload_sources_split():
    assert "bn_kernels.hip" in bench.workload_sources(MAIN)
    assert "rows_kernels.hip" not in bench.workload_sources(MAIN)
    assert "rows_kernels.hip" in bench.workload_sources("rms_bwd_2048x8192_bf16_saved_rms")
    assert "bn_kernels.hip" not in bench.workload_sources("ln_bwd_16x512x1600_xf32_dybf16_wbf16")
    for f in ("nh_device.hpp", "nh_internal.hpp"):
        assert f in bench.workload_sources(MAIN) and f in bench.workload_sources("rms_fwd_2048x8192_bf16")


def test_summarize_util_means_per_kernel(tmp_path):
    """One --pmc pass's counters averaged per library kernel; other kernels
    (torch's fills) left out."""
    k1 = "void nh::bn_grad_sums_kernel<float, 4, 6, 0>(float const*)"
    rows = []
    for v in (10.0, 12.0):
        rows += [[k1, "VALUBusy", v], [k1, "MemUnitStalled", v / 10], [k1, "SQ_WAVES", 8192]]
    rows += [["at::native::fill_kernel(float*)", "VALUBusy", 99.0]]
    _write_csv(tmp_path / "c.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    out = tmp_path / "u.txt"
    bench.summarize_util(MAIN, str(tmp_path / "c.csv"), str(out))
    text = out.read_text().splitlines()
    assert text[1].startswith("command: rocprofv3 --pmc VALUBusy MemUnitStalled")
    lines = [ln for ln in text if ln.startswith("nh::")]
    assert len(lines) == 1
    f = lines[0][70:].split()
    assert int(f[0]) == 2 and float(f[1]) == pytest.approx(11.0) and float(f[2]) == pytest.approx(1.1)
    assert f[3] == "-" and f[4] == "-" and float(f[5]) == 8192
