"""Host-side logic of the Python binding (no GPU needed)."""
import pytest
import torch

import draft_token_verification_verify_amd as sv


def test_tree_stochastic_give_up_is_reported():
    """A request marked num_accepted = -2 (its split walk gave up waiting) makes
    the binding's check raise; valid counts, zero included, pass."""
    sv.check_tree_stochastic_result(torch.tensor([0, 3, 6, 1], dtype=torch.int32))
    with pytest.raises(sv.SpecVerifyError, match=r"request\(s\) \[1, 3\]"):
        sv.check_tree_stochastic_result(torch.tensor([2, -2, 0, -2], dtype=torch.int32))
    assert sv.GAVE_UP == -2


def test_workspace_keys_on_stream():
    """The default workspace cache keys buffers by (device, stream): two streams
    never share one buffer."""
    ws = sv.Workspace()

    class FakeStream:
        def __init__(self, h):
            self.cuda_stream = h

    # Fill the cache by hand (no device here): get() must look up per stream.
    a, b = torch.zeros(256, dtype=torch.uint8), torch.zeros(512, dtype=torch.uint8)
    dev = torch.device("cpu")
    ws._buf[(dev, 11)] = a
    ws._buf[(dev, 22)] = b
    assert ws.get(100, dev, FakeStream(11)) is a
    assert ws.get(100, dev, FakeStream(22)) is b
