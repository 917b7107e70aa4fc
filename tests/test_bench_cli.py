"""Host-side contract of bench.py (no GPU needed).

The timed run itself needs an MI355X; here: more than one GPU is refused
with a message, a host without a visible GPU exits non-zero instead of
timing anything, the command line accepts the documented flags, and the
traffic figure is reported only while the attention sources still hash to
the value recorded with the counters.
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr


def test_help_lists_the_workload_flags():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--config", "--batch", "--tree", "--window",
                 "--top-k", "--top-p", "--cpu-sample"):
        assert flag in r.stdout, flag


def test_no_gpu_exits_nonzero():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _run("--steps", "1", "--warmup", "0", "--cpu-sample", "0")
    assert r.returncode != 0
    assert not r.stdout.strip().startswith("{")


def test_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    """bench.py reports the recorded traffic only while the listed sources
    still hash to the recorded value (checked on a copy, so the test does not
    depend on the committed record being current)."""
    sys.path.insert(0, ROOT)
    import bench
    rec_path = os.path.join(ROOT, "profiles", "attn_llama8b_b64_traffic.json")
    with open(rec_path) as f:
        rec = json.load(f)
    fake_root = tmp_path
    (fake_root / "profiles").mkdir()
    for p in rec["source_files"]:
        dst = fake_root / p
        dst.parent.mkdir(parents=True, exist_ok=True)
        with open(os.path.join(ROOT, p), "rb") as f:
            dst.write_bytes(f.read())
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    rec_file = fake_root / "profiles" / "attn_llama8b_b64_traffic.json"
    # A record taken on these very files: the figure is reported.
    good = dict(rec, source_sha256_16=bench._files_hash(rec["source_files"]))
    rec_file.write_text(json.dumps(good))
    assert bench._traffic() == rec["bytes_per_launch"]
    # A record whose hash does not match its files is ignored.
    rec_file.write_text(json.dumps(dict(rec, source_sha256_16="0" * 16)))
    assert bench._traffic() is None
    # So is one whose files changed after it was taken.
    rec_file.write_text(json.dumps(good))
    first = fake_root / rec["source_files"][0]
    first.write_bytes(first.read_bytes() + b"\n// edited\n")
    assert bench._traffic() is None
