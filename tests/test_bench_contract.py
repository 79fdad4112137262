"""Host-side checks of bench.py's command-line contract (no GPU needed).

* More than one GPU is refused with a message and a non-zero status before any
  device work: this path measures one GPU.
* The committed counter summary is read only while the kernel source it was
  taken on is unchanged (the HBM traffic field is null otherwise).
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode != 0
    assert "one GPU" in out.stderr or "single" in out.stderr
    assert out.stdout.strip() == ""


def test_traffic_needs_the_counted_source(tmp_path, monkeypatch):
    import bench
    src = tmp_path / "step.hip"
    src.write_text("kernel v1\n")
    counters = tmp_path / "markov_step_cfg_tiled_counters.txt"
    counters.write_text(f"kernel_source_sha256_16: {bench._sha(str(src))}\n"
                        "traffic_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "COUNTERS_FMT", str(tmp_path / "markov_step_{cfg}_{layout}_counters.txt"))
    monkeypatch.setattr(bench, "STEP_SRC", str(src))
    assert bench.read_traffic("cfg", "tiled") == 12345
    src.write_text("kernel v2\n")
    assert bench.read_traffic("cfg", "tiled") is None
    assert bench.read_traffic("other", "tiled") is None
