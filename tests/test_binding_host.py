"""Host-side checks of the Python binding, on the CPU (no kernel launched).

* A hand-built Layer whose tensors do not have the shapes K, N and group_size
  imply, or that sits on two devices, is rejected before the C call: the
  library trusts the view it is given, and a wrong one would read past the
  tensors' ends.
* Outputs and workspaces created for a call enqueued on a stream other than
  the current one are recorded on that stream, so the caching allocator does
  not hand their memory out again while the call's kernels still run.
"""
import pytest
import torch

from w4a16_group_quantized_amd import binding


def _layer(K=256, N=64, G=128, sym=False, **override):
    t = dict(qweight=torch.zeros((K // 8, N), dtype=torch.int32),
             scales=torch.zeros((K // G, N), dtype=torch.float16),
             qzeros=None if sym else torch.zeros((K // G, N // 8), dtype=torch.int32))
    t.update(override)
    return binding.Layer(t["qweight"], t["scales"], t["qzeros"], K, N, G)


@pytest.mark.parametrize("what,override", [
    ("qweight", dict(qweight=torch.zeros((16, 64), dtype=torch.int32))),     # K/8 rows wrong
    ("qweight", dict(qweight=torch.zeros((32, 72), dtype=torch.int32))),     # N columns wrong
    ("scales", dict(scales=torch.zeros((1, 64), dtype=torch.float16))),      # K/G rows wrong
    ("scales", dict(scales=torch.zeros((2, 56), dtype=torch.float16))),
    ("qzeros", dict(qzeros=torch.zeros((2, 64), dtype=torch.int32))),        # not N/8 words
    ("qzeros", dict(qzeros=torch.zeros((1, 8), dtype=torch.int32))),
])
def test_layer_shapes_checked_before_the_call(what, override):
    with pytest.raises(ValueError, match=what):
        _layer(**override).c_struct()


def test_layer_on_one_device():
    lay = _layer(scales=torch.zeros((2, 64), dtype=torch.float16, device="meta"))
    with pytest.raises(ValueError, match="scales is on"):
        lay.c_struct()


def test_consistent_layer_reaches_the_device_check():
    """Right shapes pass the shape checks; CPU tensors then fail as not GPU."""
    for sym in (False, True):
        with pytest.raises(TypeError, match="CUDA"):
            _layer(sym=sym).c_struct()


class _FakeTensor:
    def __init__(self):
        self.device = "cpu"
        self.recorded = []

    def record_stream(self, s):
        self.recorded.append(s)


def test_outputs_recorded_on_a_side_stream(monkeypatch):
    current, side = object(), object()
    made = []

    def fake_empty(*a, **k):
        made.append(_FakeTensor())
        return made[-1]

    monkeypatch.setattr(binding.torch, "empty", fake_empty)
    monkeypatch.setattr(binding.torch.cuda, "current_stream", lambda device=None: current)
    binding._new(16, torch.uint8, "cpu", side)
    binding._new(16, torch.uint8, "cpu", current)
    binding._new(16, torch.uint8, "cpu", None)
    assert [t.recorded for t in made] == [[side], [], []]
