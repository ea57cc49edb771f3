"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the source-hash
check that keeps stale traffic counters out of the roofline, and argument
checks that end before any device work."""

import argparse
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_group_size_override_is_refused_for_mxfp4():
    r = _run("--config", "c4_mxfp4", "--group-size", "64")
    assert r.returncode != 0
    assert "mxfp4 groups are 32 columns" in r.stderr


def _args(config, group_size=0, traffic=None):
    return argparse.Namespace(config=config, group_size=group_size, traffic=traffic)


@pytest.mark.parametrize("kernel,config", [("k_moe_decode", "c2"), ("k_moe_decode", "c3"),
                                           ("k_batch", "c5"), ("k_gqmm", "c4"), ("k_requant2", "requant")])
def test_committed_traffic_figures_match_the_current_sources(kernel, config):
    # every committed traffic figure was taken on the kernel sources as they are
    v = bench.traffic_for(_args(config), kernel)
    assert isinstance(v, int) and v > 0


def test_traffic_is_null_for_stale_sources_and_other_group_sizes(monkeypatch):
    assert bench.traffic_for(_args("c2", group_size=32), "k_moe_decode") is None
    assert bench.traffic_for(_args("c2", traffic=123.0), "k_moe_decode") == 123.0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel: "0" * 16)
    assert bench.traffic_for(_args("c2"), "k_moe_decode") is None
    assert bench.traffic_for(_args("no-such-workload"), "k_moe_decode") is None
