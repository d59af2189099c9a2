"""Host logic of bench.py (no GPU): the byte count behind the metric, the one-GPU
guard, and the source check that decides whether a committed counter profile
still describes the library being measured."""
import json
import os
import subprocess
import sys

import bench
import workloads as W
from conftest import ROOT


def _words(r, b):
    return 1 + (r * b + 31) // 32  # one header word, then r codes of b bits in whole words


def test_step_bytes_of_the_128k_layer():
    """The decode step's algorithmic bytes at 128K, 2 bits per dimension, written out
    from the record format: every record of both tensors, the fp16 queries, both
    bases, the fp32 output, and the append (two fp16 vectors per KV head, their two
    records, the bases it encodes with)."""
    wl = W.llama_t128k(2.0)
    alloc, _, _ = bench.calibrate(wl)
    T = wl.context + 1
    B, hq, hkv, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    rec = sum(4 * (_words(rk, bk) + _words(rv, bv)) for rk, bk, rv, bv in alloc)
    bases = sum(4 * d * (rk + rv) for rk, _, rv, _ in alloc)
    attend = B * T * rec + B * hq * d * 2 + bases + B * hq * d * 4
    append = B * hkv * 2 * d * 2 + B * rec + bases
    assert bench.step_bytes(wl, alloc, T) == (attend, append)
    assert attend + append == 303059456
    # 72 bytes per token and KV head at 2 bits per dimension (64 + 64 code bits, two header words)
    assert rec == 8 * 72


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_profile_fields_follow_the_library_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "decode_attention_04_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    (csrc / "k.hip").write_text("// kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.sources_digest()
    (tmp_path / "profiles" / "p.md").write_text(
        f"# a profile\n\n- sources_sha256: `{digest}`\n- traffic_bytes_per_launch: `123`\n")
    assert bench.profile_fields("p.md") == {"sources_sha256": digest, "traffic_bytes_per_launch": "123"}
    (csrc / "k.hip").write_text("// kernel v2\n")  # the library changed: the profile no longer applies
    assert bench.sources_digest() != digest
    assert bench.profile_fields("p.md") is None
    assert bench.profile_fields("missing.md") is None
