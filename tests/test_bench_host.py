"""Host-side logic of bench.py (CPU only): the kernel-source hash that keeps
the committed HBM-traffic counters tied to the kernel they were taken on."""
import json
import os

import bench


def test_code_tokens_ignore_comments_and_layout():
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n/* trailing\n block */\n"
    b = "int f(int x) { return x + 1; }   // edited comment\n"
    assert bench._code_tokens(a) == bench._code_tokens(b)
    # code changes and string contents count
    assert bench._code_tokens(a) != bench._code_tokens(a.replace("x + 1", "x + 2"))
    s1 = 'const char *s = "a // b";'
    s2 = 'const char *s = "a /* b */";'
    assert bench._code_tokens(s1) != bench._code_tokens(s2)
    assert "// b" in bench._code_tokens(s1)
    assert bench._code_tokens("char q = '\\'';  // quote") == "char q = '\\'';"


def test_traffic_file_matches_current_kernel_or_reads_as_stale(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    assert len(h) == 16
    # a traffic file taken on other sources is not used
    stale = {"kernel_source_hash": "0" * 16, "launches_per_step": 1, "algorithmic_bytes_per_launch": 1,
             "by_rows": {"1": {"bytes_per_launch": 2}}}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.load_traffic(1) is None
    stale["kernel_source_hash"] = h
    p.write_text(json.dumps(stale))
    assert bench.load_traffic(1) == 2
    # the committed file, if present, names a 16-hex-digit hash
    committed = os.path.join(bench.ROOT, "profiles", "decode_step_traffic.json")
    if os.path.exists(committed):
        with open(committed) as f:
            assert len(json.load(f)["kernel_source_hash"]) == 16
