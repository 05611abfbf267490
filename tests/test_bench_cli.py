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


def test_materialised_baseline_computes_the_oracle_kl(monkeypatch):
    # The bench's PyTorch materialise-then-reduce leg, run on CPU tensors: its
    # per-row KL (compared inside the leg against the KL it is handed, here the
    # oracle's) must agree, causal and not, with row blocks smaller than NQ.
    import math
    import types

    import numpy as np
    import torch

    import oracle
    bench = _bench()

    class Ev:
        def record(self):
            pass

        def elapsed_time(self, other):
            return 1.0

    monkeypatch.setattr(torch.cuda, "Event", lambda enable_timing=True: Ev())
    monkeypatch.setattr(torch.cuda, "synchronize", lambda: None)
    monkeypatch.setattr(torch.cuda, "empty_cache", lambda: None)
    monkeypatch.setattr(torch.cuda, "max_memory_allocated", lambda: 0)
    B, H, NQ, NK, D = 1, 3, 40, 70, 16
    gen = torch.Generator().manual_seed(5)
    q1, k1, q2, k2 = (torch.randn(B, H, n, D, generator=gen) for n in (NQ, NK, NQ, NK))
    g = torch.full((B, H, NQ), 1.0 / (B * H * NQ))
    for causal in (False, True):
        w = types.SimpleNamespace(B=B, H=H, NQ=NQ, NK=NK, scale=1 / math.sqrt(D), causal=causal)
        kl = torch.zeros(B, H, NQ)
        for h in range(H):
            f = lambda t: t[0, h].double().numpy()
            kl[0, h] = torch.from_numpy(np.asarray(oracle.fwd(f(q1), f(k1), f(q2), f(k2), w.scale, causal)[0]))
        monkeypatch.setattr(bench, "materialised_rows", lambda nk: 16, raising=False)
        res = bench.materialised_baseline(torch, w, q1, k1, q2, k2, g, kl, heads=2)
        assert res["kl_max_rel_diff_vs_fused"] < 1e-5, res
        assert res["heads_timed"] == 2 and res["scaled_to_heads"] == 3
