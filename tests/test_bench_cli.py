"""bench.py's command line on the CPU: the one-GPU contract."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "one gpu" in r.stderr.lower(), r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a configuration it does not run


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_cpu_model_is_a_string():
    assert isinstance(_bench().cpu_model(), str)


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    # Counter CSVs shaped as rocprofv3 writes them: the copy of COPY_BYTES reads
    # 2x its size in FETCH_SIZE and 0.5x in WRITE_SIZE, so the kernel's raw
    # counts are scaled by 1/2 and 2.
    bench = _bench()
    kib = bench.COPY_BYTES / 1024
    fwd = bench.KERNELS["fwd"][1] + "(skl::FwdParams)"
    rows = lambda counter, copy_v, k_v: (
        "Kernel_Name,Counter_Name,Counter_Value\n"
        f"\"void at::native::elementwise_kernel<copy>\",{counter},{copy_v}\n"
        f"\"{fwd}\",{counter},{k_v}\n"
        f"\"{fwd}\",{counter},{k_v * 3}\n")
    (tmp_path / "f.csv").write_text(rows("FETCH_SIZE", 2 * kib, 1000.0))
    (tmp_path / "w.csv").write_text(rows("WRITE_SIZE", 0.5 * kib, 10.0))
    rec_path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec_path))
    bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    assert rec_path.exists()
    got = bench.recorded_traffic("fwd")
    # Mean over the two dispatches, in bytes, times each counter's scale.
    assert abs(got - (2000.0 * 1024 / 2 + 20.0 * 1024 * 2)) < 1e-6
    assert bench.recorded_traffic("bwd_dk") is None
