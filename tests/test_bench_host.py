"""Host-side logic of bench.py (no GPU): the kernel code hash and the
traffic and counter lookups keyed by it."""

import json

import bench


def test_kernel_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a = 1;  // one\n\n// note\nint b = 2;\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h0 = bench.kernel_hash()
    src.write_text("// header\nint a = 1;   // first\nint b = 2;\n\n")
    assert bench.kernel_hash() == h0
    src.write_text("int a = 1;\nint b = 3;\n")
    assert bench.kernel_hash() != h0


def test_traffic_only_for_matching_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a = 1;\n")
    tf = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    tf.write_text(json.dumps({"w": {"kernel_sha256_16": bench.kernel_hash(), "bytes_per_launch": 123}}))
    assert bench.traffic_for("w") == 123
    assert bench.traffic_for("other") is None
    src.write_text("int a = 2;\n")
    assert bench.traffic_for("w") is None



def test_counters_only_for_matching_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a = 1;\n")
    tf = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    ent = {"kernel_sha256_16": bench.kernel_hash(), "bytes_per_launch": 123, "mfma_busy_pct": 70.5,
           "lds_bank_conflict_cycles": 10.0, "lds_active_cycles": 1000.0, "lds_conflict_rate": 0.01, "source": "s.md"}
    tf.write_text(json.dumps({"w": ent, "old": {"kernel_sha256_16": bench.kernel_hash(), "bytes_per_launch": 1}}))
    got = bench.counters_for("w")
    assert got["mfma_busy_pct"] == 70.5 and got["lds_conflict_rate"] == 0.01 and got["source"] == "s.md"
    assert bench.counters_for("old") is None  # an entry without counter figures
    assert bench.counters_for("other") is None
    src.write_text("int a = 2;\n")
    assert bench.counters_for("w") is None
