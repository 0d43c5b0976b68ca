"""The Python binding's checks on caller-supplied buffers.

The kernels read and write every buffer through a raw address the C ABI
cannot inspect, so the binding must refuse, with ValueError and before any
launch, a host tensor, a tensor on another device, a wrongly shaped or typed
tensor, a non-contiguous one and a workspace that is too small.  These tests
run the checks on stand-in objects (no device needed) and on CPU tensors.
"""

from __future__ import annotations

import pytest
import torch

import exact_tiled_attention_33_amd as fa2


class FakeTensor:
    def __init__(self, shape, dtype=torch.float32, device="cuda:0", contiguous=True, itemsize=4):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = self.device.type == "cuda"
        self._contig = contiguous
        self._itemsize = itemsize

    def is_contiguous(self):
        return self._contig

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return self._itemsize


DEV0 = torch.device("cuda:0")


def test_buffer_accepts_the_exact_device_tensor():
    fa2._check_buffer(FakeTensor((2, 3, 5)), "delta", (2, 3, 5), torch.float32, DEV0)


@pytest.mark.parametrize("t, what", [
    (FakeTensor((2, 3, 5), device="cpu"), "host tensor"),
    (FakeTensor((2, 3, 5), device="cuda:1"), "other device"),
    (FakeTensor((2, 3, 4)), "short"),
    (FakeTensor((2, 3, 5, 1)), "extra dim"),
    (FakeTensor((2, 3, 5), dtype=torch.bfloat16), "dtype"),
    (FakeTensor((2, 3, 5), contiguous=False), "strided"),
])
def test_buffer_rejects(t, what):
    with pytest.raises(ValueError):
        fa2._check_buffer(t, "delta", (2, 3, 5), torch.float32, DEV0)


def test_inputs_on_device():
    fa2._check_on_device(DEV0, q=FakeTensor((1,)), k=FakeTensor((1,)))
    with pytest.raises(ValueError, match="k must be a device tensor"):
        fa2._check_on_device(DEV0, q=FakeTensor((1,)), k=FakeTensor((1,), device="cpu"))
    with pytest.raises(ValueError, match="v must be a device tensor"):
        fa2._check_on_device(DEV0, q=FakeTensor((1,)), v=FakeTensor((1,), device="cuda:1"))
    with pytest.raises(ValueError, match="contiguous"):
        fa2._check_on_device(DEV0, q=FakeTensor((1,), contiguous=False))


def test_workspace_size_and_device():
    fa2._check_workspace(FakeTensor((100,), torch.uint8, itemsize=1), "workspace", 100, DEV0)
    fa2._check_workspace(FakeTensor((25,), torch.float32, itemsize=4), "workspace", 100, DEV0)
    with pytest.raises(ValueError, match="bytes"):
        fa2._check_workspace(FakeTensor((99,), torch.uint8, itemsize=1), "workspace", 100, DEV0)
    with pytest.raises(ValueError):
        fa2._check_workspace(FakeTensor((100,), torch.uint8, device="cpu", itemsize=1), "workspace", 100, DEV0)
    with pytest.raises(ValueError):
        fa2._check_workspace(FakeTensor((100,), torch.uint8, contiguous=False, itemsize=1), "workspace", 100, DEV0)


def test_entry_points_refuse_host_inputs():
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError):
        fa2.forward(q, q, q)
    with pytest.raises(ValueError):
        fa2.backward(q, q, q, q, lse, q)
    with pytest.raises(ValueError):
        fa2.forward_fp8(q, q, q)
