"""The guard-band allocator the GPU tests wrap around the binding's outputs
and workspaces: the tensor it returns is aligned and contiguous, untouched
margins pass, and a single changed byte on either side fails."""

import pytest
import torch

from helpers import GuardBands


def test_clean_buffers_pass():
    g = GuardBands()
    t = g.empty((3, 5, 7), torch.float32, "cpu")
    assert t.is_contiguous() and t.shape == (3, 5, 7)
    assert t.data_ptr() % 256 == g.buffers[0][0].data_ptr() % 256
    t.fill_(1.0)
    g.empty((0, 8), torch.float32, "cpu")
    g.check()


@pytest.mark.parametrize("where", ["before", "after"])
def test_a_stray_byte_is_caught(where):
    g = GuardBands()
    t = g.empty((16,), torch.float32, "cpu")
    t.fill_(2.0)
    buf, nbytes = g.buffers[0][0], g.buffers[0][1]
    buf[g.MARGIN - 1 if where == "before" else g.MARGIN + nbytes] = 0
    with pytest.raises(AssertionError, match="guard band"):
        g.check()
