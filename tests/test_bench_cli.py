"""Host-side checks of bench.py (CPU only): the single-GPU contract and the gate that reports the
profiled HBM traffic only while the committed counter summary matches the kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (its main() runs only as a script)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("profile,key,srcs,kernel", [
    (bench.PROFILE, "forward_sources_sha256", bench.KERNEL_SRCS, "decode"),
    (bench.BLOCK_PROFILE, "project_sources_sha256", bench.PROJECT_SRCS, "project"),
])
def test_committed_profiles_match_the_kernel_sources(profile, key, srcs, kernel):
    # The committed counter summaries were taken on the kernels as they are now, so the benchmark
    # reports their traffic (it reports null once a kernel source changes).
    t = bench.profiled_traffic(kernel, profile=profile, key=key, srcs=srcs)
    assert t is not None and t > 0


def test_committed_backward_profile_matches_the_kernel_sources():
    # The backward's dominant kernel: its roofline fraction is also reported on the committed trace's
    # average duration while that trace matches the sources.
    us = bench.profiled_kernel_us("bwd_token_decode", bench.BWD_PROFILE, "backward_sources_sha256", bench.BWD_SRCS)
    assert us is not None and us > 0


def test_profiled_traffic_is_null_for_another_source(tmp_path):
    sha = bench.kernel_source_hash()
    rec = {"forward_sources_sha256": sha, "per_launch_bytes": {"decode": 123.0}}
    good = tmp_path / "good.md"
    good.write_text("# summary\n\ntraffic-json: " + json.dumps(rec) + "\n")
    assert bench.profiled_traffic("decode", profile=str(good)) == 123.0
    assert bench.profiled_traffic("encode_partial", profile=str(good)) is None
    rec["forward_sources_sha256"] = "0" * 64
    stale = tmp_path / "stale.md"
    stale.write_text("traffic-json: " + json.dumps(rec) + "\n")
    assert bench.profiled_traffic("decode", profile=str(stale)) is None
    assert bench.profiled_traffic("decode", profile=str(tmp_path / "missing.md")) is None
