import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def guard_bands(request):
    """In every GPU test, the outputs and workspaces the binding allocates
    carry sentinel margins on both sides, checked after the test."""
    if request.node.get_closest_marker("gpu") is None:
        yield None
        return
    import decode_attention_kv_attn_amd as L
    from helpers import GuardBands
    g = GuardBands()
    saved = L._empty
    L._empty = g.empty
    try:
        yield g
    finally:
        L._empty = saved
    g.check()
