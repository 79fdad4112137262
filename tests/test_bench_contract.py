"""Host-side checks of bench.py's command-line contract (no GPU needed).

* More than one GPU is refused with a message and a non-zero status before any
  device work: this path measures one GPU.
* The committed counter summary is read only while the step kernels' sources
  it was taken on are unchanged (the HBM traffic field is null otherwise).
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
    counters = tmp_path / "markov_step_cfg_rgv_counters.txt"
    counters.write_text(f"step_source_hash: {bench.source_hash()}\n"
                        "traffic_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "COUNTERS_FMT", str(tmp_path / "markov_step_{cfg}_{layout}_counters.txt"))
    assert bench.read_traffic("cfg", "rgv") == 12345
    monkeypatch.setattr(bench, "source_hash", lambda: "another build")
    assert bench.read_traffic("cfg", "rgv") is None
    assert bench.read_traffic("other", "rgv") is None


def test_step_hash_covers_the_step_kernel_sources():
    import bench
    from draft_head_step_amd import build
    names = {os.path.basename(f) for f in build.source_files()}
    assert set(bench.STEP_SOURCES) <= names
    assert any(n.startswith("markov_pick_") for n in bench.STEP_SOURCES)
    assert len(bench.source_hash()) == 32
