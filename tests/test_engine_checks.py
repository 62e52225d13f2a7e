"""The Python engine rejects tensors the library cannot take before any
address reaches it (no GPU: only the rejections are exercised here; the GPU
tests pass valid tensors through the same checks)."""
import numpy as np
import pytest
import torch

from expert_offload_serving_amd import engine as eg

H, E, k, TMAX = 256, 8, 2, 16


def _cpu(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def test_host_tensor_rejected():
    with pytest.raises(ValueError, match="CUDA"):
        eg.check_forward(H, E, k, TMAX, _cpu((4, H), torch.int16), None, _cpu((4, H), torch.int16),
                         None, None, None)


def test_not_a_tensor_rejected():
    with pytest.raises(ValueError, match="torch tensor"):
        eg.check_device("x", np.zeros((4, H), np.int16), ("int16",), (4, H))


class FakeCuda:
    """Stands in for a CUDA tensor so that the shape, dtype and layout
    checks can run without a GPU."""

    def __init__(self, shape, dtype="int16", contiguous=True, device="cuda:0"):
        self.shape, self.dtype, self._c, self.device = tuple(shape), f"torch.{dtype}", contiguous, device
        self.is_cuda = True

    def data_ptr(self):
        return 0

    def is_contiguous(self):
        return self._c


def test_shape_dtype_layout_checks():
    x, y = FakeCuda((4, H)), FakeCuda((4, H))
    assert eg.check_forward(H, E, k, TMAX, x, None, y, None, None, None) == 4
    cases = [
        (dict(x=FakeCuda((4, H + 1))), "shape"),                       # wrong hidden size
        (dict(x=FakeCuda((4, H), dtype="float32")), "dtype"),          # 4-byte activations
        (dict(x=FakeCuda((4, H), contiguous=False)), "contiguous"),    # transposed view
        (dict(x=FakeCuda((TMAX + 1, H)), y=FakeCuda((TMAX + 1, H))), "at most"),
        (dict(y=FakeCuda((3, H))), "shape"),                           # y too small
        (dict(bias=FakeCuda((4, E), dtype="float16")), "dtype"),
        (dict(bias=FakeCuda((4, E + 1), dtype="float32")), "shape"),
        (dict(ids=FakeCuda((4, k), dtype="int64")), "dtype"),
        (dict(gates=FakeCuda((4, k + 1), dtype="float32")), "shape"),
        (dict(y32=FakeCuda((4, H), dtype="bfloat16")), "dtype"),
        (dict(y=FakeCuda((4, H), device="cuda:1")), "on cuda:1"),
    ]
    for over, msg in cases:
        a = dict(x=x, bias=None, y=y, ids=None, gates=None, y32=None)
        a.update(over)
        with pytest.raises(ValueError, match=msg):
            eg.check_forward(H, E, k, TMAX, a["x"], a["bias"], a["y"], a["ids"], a["gates"],
                             a["y32"])


def test_prefill_checks():
    xs = [FakeCuda((100, H)), FakeCuda((100, H))]
    ys = [FakeCuda((100, H)), FakeCuda((100, H))]
    assert eg.check_prefill(H, E, 2, 128, xs, ys, None, None) == 100
    with pytest.raises(ValueError, match="layers"):
        eg.check_prefill(H, E, 1, 128, xs, ys, None, None)
    with pytest.raises(ValueError, match="1..64"):
        eg.check_prefill(H, E, 2, 64, xs, ys, None, None)
    with pytest.raises(ValueError, match="entries"):
        eg.check_prefill(H, E, 2, 128, xs, ys[:1], None, None)
    with pytest.raises(ValueError, match="shape"):
        eg.check_prefill(H, E, 2, 128, xs, [ys[0], FakeCuda((99, H))], None, None)
    with pytest.raises(ValueError, match="shape"):
        eg.check_prefill(H, E, 2, 128, xs, ys, [FakeCuda((100, E), "float32"),
                                                FakeCuda((100, E + 2), "float32")], None)
    # a None entry in the optional lists is allowed
    assert eg.check_prefill(H, E, 2, 128, xs, ys, [None, None], [None, FakeCuda((100, H), "float32")]) == 100


def test_host_weight_shapes():
    eg.check_host("w", np.zeros((H, E), np.float32), (H, E))
    with pytest.raises(ValueError, match="shape"):
        eg.check_host("w", np.zeros((E, H), np.float32), (H, E))


def test_prefetch_list_checks():
    """set_prefetch takes a 1-D contiguous int32 CUDA tensor (or nothing)."""
    stub = type("S", (), {"ctx": None})()
    for bad, msg in ((_cpu((3,), torch.int32), "CUDA"), (np.arange(3, dtype=np.int32), "torch tensor")):
        with pytest.raises(ValueError, match=msg):
            eg.MoEEngine.set_prefetch(stub, 1, bad)
