"""Host-side logic of bench.py (no GPU): the one-GPU contract, the algorithmic byte
counts, and the traffic record that is reported only while the attention kernel's
sources match the hash stored with the counters."""
import json
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_algorithmic_bytes_of_the_quantisation_pass():
    w = workloads.get("flux_like")
    E = w.B * w.H * w.N * w.d
    assert bench.quant_bytes(w) == 9 * E      # read Q, K, V in bf16, write three 1-byte codes


def test_metric_counts_four_b_h_n2_d():
    w = workloads.get("flux_like")
    assert w.ops == 4 * w.B * w.H * w.N * w.N * w.d


def _write_record(tmp_path, source_hash):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel": "k", "workload": "flux_like", "source_hash": source_hash, "fetch_bytes": 10,
           "write_bytes": 5, "traffic_bytes": 15, "algorithmic_bytes": 12}
    (prof / "attn_flux_like_traffic.md").write_text("# summary\n\ntraffic-record: " + json.dumps(rec) + "\n")
    return rec


def test_traffic_record_is_used_only_while_the_sources_match(tmp_path, monkeypatch):
    current = bench.kernel_source_hash()
    rec = _write_record(tmp_path, current)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for f in bench.ATTN_SOURCES:                   # the hashed sources, copied unchanged
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, f), "rb").read())
    assert bench.kernel_source_hash() == current
    assert bench.recorded_traffic("flux_like") == rec
    assert bench.recorded_traffic("stress") is None            # no record for that workload
    # a comment or a blank line leaves the code unchanged; any edit of the code
    # invalidates the record
    src = tmp_path / bench.ATTN_SOURCES[0]
    src.write_bytes(src.read_bytes() + b"\n// a comment\n/* another */\n")
    assert bench.recorded_traffic("flux_like") == rec
    src.write_bytes(src.read_bytes() + b"static int x;\n")
    assert bench.recorded_traffic("flux_like") is None
