import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built libmoeq.so")
    config.addinivalue_line("markers", "slow: full-size workload (minutes)")


@pytest.fixture(autouse=True)
def _decode_waits_end_in_time(request):
    """For every GPU test: every decode-family workspace made through the
    binding during the test must end with its error word clear (no bounded
    wait inside a decode launch gave up)."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    from quantized_moe_expert_unpack_amd import moeq
    moeq.track_workspaces(True)
    try:
        yield
        moeq.check_workspaces()
    finally:
        moeq.track_workspaces(False)


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows
