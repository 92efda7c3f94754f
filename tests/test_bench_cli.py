"""Host logic of bench.py (no GPU): the command-line rejections, and the
stored HBM-traffic figure, which counts only while the gate/up kernel's
sources are unchanged since its counters were read."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,msg", [
    (["--gpus", "2"], "one GPU only"),
    (["--shape", "30b", "--workload", "prefill"], "--shape applies to the decode workload only"),
    (["--quant", "q2", "--workload", "copy"], "--quant q2 applies to"),
])
def test_bench_rejects_unsupported_runs(argv, msg):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=300)
    assert p.returncode == 2
    assert msg in p.stderr
    assert p.stdout == ""


def test_stored_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "kernel.hip"
    src.write_text("// gate/up kernel\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "GATE_UP_SOURCES", ("kernel.hip",))
    monkeypatch.setattr(bench, "TRAFFIC_FILES", {("235b", 4): "traffic.txt"})
    assert bench.stored_traffic(4) is None  # no summary
    digest = bench.sources_digest(("kernel.hip",))
    (tmp_path / "traffic.txt").write_text(
        "counters ...\n  indented: 1\nsource_sha256: %s\ntraffic_bytes_per_launch: 56984696\n" % digest)
    assert bench.stored_traffic(4) == 56984696.0
    src.write_text("// gate/up kernel, changed\n")  # the kernel changed since the counters were read
    assert bench.stored_traffic(4) is None


def test_committed_traffic_summaries_name_a_figure():
    sys.path.insert(0, ROOT)
    import bench
    for path in bench.TRAFFIC_FILES.values():
        kv = {}
        with open(os.path.join(ROOT, path)) as f:
            for line in f:
                if ":" in line and not line.startswith(" "):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        assert len(kv.get("source_sha256", "")) == 64, path
        assert float(kv["traffic_bytes_per_launch"]) > 0, path
