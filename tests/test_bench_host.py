"""Host-side logic of bench.py: the one-GPU refusal and the counter-record lookup that
reports HBM traffic only while the kernel sources still match the record."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def _record(tmp_path, monkeypatch, src_text, sha_of_sources):
    src = tmp_path / "kernel.hip"
    src.write_text(src_text)
    prof = tmp_path / "summary.md"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "probe", ("summary.md", ("kernel.hip",)))
    sha = bench.sources_sha256("probe") if sha_of_sources else "0" * 64
    prof.write_text("# summary\n\ntraffic-record: kernel=probe sources_sha256=%s "
                    "fetch_kib=1.0 traffic_bytes=123456\n" % sha)
    return src


def test_traffic_record_matches_current_sources(tmp_path, monkeypatch):
    _record(tmp_path, monkeypatch, "kernel v1", True)
    assert bench.profiled_traffic("probe") == 123456


def test_traffic_record_goes_stale_when_sources_change(tmp_path, monkeypatch):
    src = _record(tmp_path, monkeypatch, "kernel v1", True)
    src.write_text("kernel v2")
    assert bench.profiled_traffic("probe") is None


def test_traffic_record_with_another_hash_is_ignored(tmp_path, monkeypatch):
    _record(tmp_path, monkeypatch, "kernel v1", False)
    assert bench.profiled_traffic("probe") is None


def test_missing_summary_gives_no_traffic(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "probe", ("absent.md", ("kernel.hip",)))
    assert bench.profiled_traffic("probe") is None


def test_algorithmic_byte_counts_of_the_32k_layer_step():
    """264 B per (KV head, token) for the sketch stream (bf16 key row + float64 r; the
    float64 weights the kernel writes are scratch), 520 B per pivot row, and one bit per
    (KV head, token) for each of the resident and fetch bitmasks."""
    tok = 8 * 32768
    assert bench.sketch_bytes(tok) == 69206016
    assert bench.step_algorithmic_bytes(tok, 2048 * 8) == 69206016 + 2048 * 8 * 520 + 65536


def test_step_percentiles():
    p = bench.percentiles([float(x) for x in range(1, 101)])
    assert p["p50"] == 50.5 and abs(p["p10"] - 10.9) < 1e-9 and abs(p["p90"] - 90.1) < 1e-9
