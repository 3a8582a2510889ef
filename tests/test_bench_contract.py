"""CPU checks of bench.py's command-line contract (no GPU is touched)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_digest_ignores_comments_only(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench

    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {  // one\n  return x + 1; /* two */\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ("k.hip",))
    d0 = bench.kernel_source_digest()
    src.write_text("int f(int x) {  // a different comment\n\n  return x + 1;\n}\n")
    assert bench.kernel_source_digest() == d0
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_source_digest() != d0
