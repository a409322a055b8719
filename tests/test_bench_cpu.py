"""bench.py host logic that needs no GPU: it parses, refuses more than one
GPU, and keys committed traffic figures on the measured kernel's sources."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_help_and_one_gpu_only():
    assert _run("--help").returncode == 0
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_profile_tags():
    assert bench.profile_tag("batched", 1) == "batched"
    assert bench.profile_tag("batched", 4) == "batched_verify4"
    assert bench.profile_tag("lowbit", 1, "rot3:rot3") == "lowbit_rot3_rot3"
    assert bench.profile_tag("lowbit", 3, "rot3:q4_0") == "lowbit_rot3_q4_0_verify3"


def test_codec_override_is_checked():
    r = _run("--codecs", "rot3")
    assert r.returncode != 0 and "K:V" in r.stderr
    r = _run("--codecs", "rot5:rot3")
    assert r.returncode != 0


def test_traffic_is_taken_only_on_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kind="decode": "abc")
    (prof / "decode_batched_traffic.json").write_text(json.dumps(
        {"kernel_source_hash": "abc", "n_splits": 4, "hbm_bytes_per_launch": 123}))
    assert bench.load_traffic("decode", "batched", 4) == 123
    assert bench.load_traffic("decode", "batched", 8) is None       # other split count
    (prof / "decode_batched_traffic.json").write_text(json.dumps(
        {"kernel_source_hash": "old", "n_splits": 4, "hbm_bytes_per_launch": 123}))
    assert bench.load_traffic("decode", "batched", 4) is None       # other sources
    assert bench.load_traffic("transcode", "f16_to_q8_0_k") is None  # no file


def test_kernel_source_hashes_follow_the_source_sets():
    # kernels built from the same files (append and transcode share
    # append.hip) share a hash; different file sets give different hashes
    h = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    for a in h:
        for b in h:
            same = set(bench.KERNEL_SOURCES[a]) == set(bench.KERNEL_SOURCES[b])
            assert (h[a] == h[b]) == same, (a, b)
