"""Host-side checks of the Python binding (CPU: no kernel is launched).  The
C ABI takes bare pointers, so the binding must refuse tensors and streams of
another GPU before it calls the library."""
from types import SimpleNamespace

import pytest

torch = pytest.importorskip("torch")
fw_binding = pytest.importorskip("linear_attention_rnn_finch_amd._binding")


def test_same_device_accepts_one_gpu():
    dev = torch.device("cuda", 0)
    on = SimpleNamespace(device=torch.device("cuda", 0))
    fw_binding._same_device(dev, SimpleNamespace(device=dev), k=on, v=on, u=None)


@pytest.mark.parametrize("what", ["tensor", "stream"])
def test_same_device_refuses_another_gpu(what):
    dev = torch.device("cuda", 0)
    other = SimpleNamespace(device=torch.device("cuda", 1))
    with pytest.raises(ValueError, match="cuda:1"):
        if what == "tensor":
            fw_binding._same_device(dev, None, k=SimpleNamespace(device=dev), v=other)
        else:
            fw_binding._same_device(dev, other, k=SimpleNamespace(device=dev))
