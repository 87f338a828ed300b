"""The measurement code's pure parts (CPU): per-launch algorithmic bytes,
the committed traffic summaries and the guard against a multi-GPU run."""

from __future__ import annotations

import hashlib
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_partial_bytes_count_out_only_when_the_launch_writes_it():
    spec = W.CONFIGS["long"]
    st = {"algorithmic_bytes": 1_000_000, "mode_name": "split", "launches": 1}
    out = 1 * spec.num_q_heads * spec.head_dim * 2
    assert bench.partial_kernel_bytes(st, spec, 1) == 1_000_000          # fused: writes out
    st2 = dict(st, launches=2)
    assert bench.partial_kernel_bytes(st2, spec, 1) == 1_000_000 - out  # separate merge writes out
    st3 = dict(st, mode_name="unsplit", launches=1)
    assert bench.partial_kernel_bytes(st3, spec, 1) == 1_000_000


def test_traffic_is_reported_only_for_the_source_it_was_taken_on():
    # A committed counter summary counts only while the kernel source is the
    # one it records (else the bench reports null); when it counts, the
    # measured bytes are within a few percent of the algorithmic bytes.
    digest = hashlib.sha256(bench.kernel_sources()).hexdigest()
    for key, name in bench.TRAFFIC_PROFILES.items():
        text = open(os.path.join(ROOT, "profiles", name)).read()
        got = bench.measured_traffic(*key)
        if f"kernel_source_sha256: {digest}" not in text:
            assert got is None, name
            continue
        assert isinstance(got, int) and got > 0
        alg = int(text.split("algorithmic bytes per launch\n")[1].split(" B")[0].replace(",", ""))
        assert 1.0 <= got / alg < 1.05, (name, got, alg)
    assert bench.measured_traffic("long", "split", 7, "fused") is None
    assert bench.measured_traffic("b64", "workqueue", 0, "fused") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
