"""Host logic that runs without a GPU (test code): the one-GPU guard of
bench.py, the rule that a committed HBM-traffic summary is reported only
while the kernel sources match the ones its counters were taken with, and
the host model of the backward's schedule against the kernels' constants."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_traffic_summary_is_used_only_with_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "mala_bwd_traffic_128k.txt").write_text(
        "kernel: mala_bwd\n  bwd_kv_kernel  fetch 1 GB\nhbm_bytes_per_launch: 1.5e+10\n"
        "kernel_source_hash: abcdef0123456789\n")
    (prof / "mala_fwd_traffic_128k.txt").write_text(
        "hbm_bytes_per_launch: 2e9\nkernel_source_hash: 0000000000000000\n")
    (prof / "mala_decode_traffic_128k.txt").write_text(
        "hbm_bytes_per_launch: not-a-number\nkernel_source_hash: abcdef0123456789\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abcdef0123456789")
    assert bench.read_traffic("mala_bwd") == 1.5e10
    assert bench.read_traffic("mala_fwd") is None       # taken with other sources
    assert bench.read_traffic("mala_decode") is None    # unreadable value
    assert bench.read_traffic("mala_other") is None     # no summary


def test_source_hash_covers_the_kernels_and_not_the_host_api(tmp_path, monkeypatch):
    csrc = tmp_path / "adaptive_softmax_attention_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "mala_fwd.hip").write_text("kernel a")
    (csrc / "mala_api.hip").write_text("host b")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "mala_api.hip").write_text("host c")
    assert bench.kernel_source_hash() == h0
    (csrc / "mala_fwd.hip").write_text("kernel a // a note\n/* more\nnotes */\n\n")
    assert bench.kernel_source_hash() == h0  # comments and blank lines change no kernel
    (csrc / "mala_fwd.hip").write_text("kernel a2")
    assert bench.kernel_source_hash() != h0


def test_committed_profiles_name_their_commands():
    for name in ("bench_kernels_128k.txt", "mala_fwd_traffic_128k.txt", "mala_bwd_traffic_128k.txt",
                 "mala_decode_traffic_128k.txt", "sq_counters_128k.txt", "sq_activity_128k.txt"):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        assert "rocprofv3" in text and "bench.py" in text, name


def test_host_schedule_model_uses_the_kernels_constants():
    """tests/bwd_schedule.py restates the dK/dV pass's pairing and
    segmentation rule to choose the key blocks the full-size tests compare;
    its constants must be the kernels' (items per segment, segments per
    pair, partial-sum slots per pair)."""
    import re

    import bwd_schedule as S
    csrc = os.path.join(ROOT, "adaptive_softmax_attention_amd", "csrc")
    text = "".join(open(os.path.join(csrc, f)).read()
                   for f in ("mala_internal.h", "mala_bwd.h", "mala_bwd.hip", "mala_bwd_kv.hip"))

    def const(name):
        m = re.search(r"constexpr int " + name + r"\s*=\s*(\d+)\s*;", text)
        assert m, name
        return int(m.group(1))
    assert S.SEG_KEPT == const("kSegKept")
    assert S.SEG_MAX == const("kSegMax")
    assert S.SLOTS_PER_PAIR == const("kSlotsPerPair")
