"""Host-side behaviour of bench.py that needs no GPU."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_sha_follows_code_not_comments(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) {  /* block */ return x + 1; }  // tail\n")
    b = tmp_path / "b.hip"
    b.write_text("// another header\n\nint f(int x) {\n  return x + 1;\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_sha(str(a)) == bench.source_sha(str(b))
    assert bench.source_sha(str(a)) != bench.source_sha(str(c))


def test_measured_traffic_needs_matching_code_and_workload(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    rec = tmp_path / "t.json"
    rec.write_text(json.dumps({"workload": "w1", "source_sha": bench.source_sha(str(src)),
                               "bytes_per_launch": 1234}))
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.measured_traffic("w1") == 1234
    assert bench.measured_traffic("w2") is None               # another workload
    src.write_text("// a comment only\n__global__ void k() {}\n")
    assert bench.measured_traffic("w1") == 1234               # comments do not void it
    src.write_text("__global__ void k() { int x = 0; }\n")
    assert bench.measured_traffic("w1") is None               # changed code does
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("w1") is None


def test_algorithmic_bytes_of_the_headline_step():
    import numpy as np
    import synth
    w = synth.WORKLOADS["bf16_b64_ragged1k_8k"]
    lengths = np.full(w.B, 4096, dtype=np.int64)
    attn_bytes, attn_flops, commit_bytes = bench.algorithmic(w, lengths)
    # 512 B per cached key per KV head (K and V, bf16, D = 128) plus 278,528 B
    # per sequence for Q, block K/V and the output
    assert attn_bytes == int(lengths.sum()) * 2 * 512 + w.B * 278528
    assert attn_flops == 4 * w.Hq * w.S * w.D * (int(lengths.sum()) + w.B * w.S)
    assert commit_bytes == w.B * w.S * w.V * 2 + w.B * w.S * 10


def test_algorithmic_bytes_of_the_cache_append():
    import synth
    w = synth.WORKLOADS["bf16_b64_ragged1k_8k"]
    # K and V rows of 2 x 128 bf16 (512 B each), read once and written once,
    # for the 300,000 old rows and the 64 x 16 new ones; offsets read + written
    assert bench.append_algorithmic(w, 300000) == 4 * (300000 + 1024) * 512 + 16 * 65


def test_algorithmic_bytes_of_the_mamba_scan():
    import synth
    w = synth.MAMBA_WORKLOADS["mamba_b64_s16_h128"]
    state = 64 * 128 * 64 * 128 * 4                      # fp32 seed states
    xy = 2 * 64 * 16 * 128 * 64 * 2                      # x in, y out (bf16)
    bc = 2 * 64 * 16 * 8 * 128 * 2                       # Bm, Cm (bf16)
    assert bench.mamba_algorithmic(w) == state + xy + bc + 64 * 16 * 128 * 4 + 2 * 128 * 4


def test_algorithmic_bytes_of_the_adaln_modulation():
    import synth
    w = synth.ADALN_WORKLOADS["adaln_b64_s16_h4096"]
    act = 64 * 16 * 4096 * 2                      # one bf16 [B, S, H] tensor
    assert bench.adaln_algorithmic(w) == 4 * act + 64 * 3 * 4096 * 4 + 4 * 4096 * 4
