"""CPU checks of the benchmark's command line and bookkeeping (no GPU needed)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_every_kernel_class_names_existing_sources():
    for name, files in bench.KERNEL_SOURCES.items():
        assert files, name
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "parameter_efficient_fine_amd", "csrc", f)), (name, f)
        assert len(bench.kernel_source_hash(name)) == 16


def test_counted_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    # a counter summary counts only while the kernel's sources hash to the recorded value
    prof = tmp_path / "profiles"
    prof.mkdir()
    (tmp_path / "parameter_efficient_fine_amd").mkdir()
    os.symlink(os.path.join(ROOT, "parameter_efficient_fine_amd", "csrc"),
               tmp_path / "parameter_efficient_fine_amd" / "csrc")
    h = bench.kernel_source_hash("gemm_bwd")
    (prof / "gemm_bwd_attn_counters.md").write_text(f"traffic_bytes_per_launch: 123456\nsource_hash: {h} (x)\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counted_traffic("gemm_bwd", "attn") == 123456.0
    (prof / "gemm_bwd_attn_counters.md").write_text("traffic_bytes_per_launch: 123456\nsource_hash: 0000\n")
    assert bench.counted_traffic("gemm_bwd", "attn") is None
    assert bench.counted_traffic("gemm_fwd", "attn") is None  # no summary at all


def test_gpu_state_is_null_without_a_readable_rocm_smi(monkeypatch):
    monkeypatch.setenv("PATH", "/nonexistent")
    assert bench.gpu_state_under_load(lambda: None, lambda: None, cap_s=1) is None


def test_priming_defaults_and_can_be_turned_off(monkeypatch):
    # untimed back-to-back steps before the warm-up steps (the GPU ramps up from idle)
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    assert bench.parse().prime_s == bench.PRIME_S > 0
    monkeypatch.setattr(sys, "argv", ["bench.py", "--prime-s", "0", "--steps", "20", "--warmup", "5"])
    a = bench.parse()
    assert a.prime_s == 0 and a.steps == 20 and a.warmup == 5
