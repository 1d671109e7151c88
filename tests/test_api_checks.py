"""The torch wrappers reject caller-supplied output buffers that the kernels
would write out of bounds (wrong size, dtype, device or layout) before any
call into the library.  Checked on the CPU through the wrappers' own
validation helpers (there is no GPU here; the checks compare tensors only)."""
import pytest
import torch

from cross_correlation_amd import _lib, api

CPU = torch.device("cpu")


def test_check_out_accepts_dense_match():
    api._check_out(torch.empty(6, 7, dtype=torch.float32), "o", 42, (torch.float32,), CPU)
    api._check_out(torch.empty(42, dtype=torch.uint32), "o", 42, api._SUM_DTYPES, CPU)


@pytest.mark.parametrize("t,msg", [
    (torch.empty(6, 6, dtype=torch.float32), "elements"),             # too small
    (torch.empty(6, 8, dtype=torch.float32), "elements"),             # too large
    (torch.empty(6, 7, dtype=torch.float64), "dtype"),                # wrong dtype
    (torch.empty(7, 6, dtype=torch.float32).t(), "contiguous"),       # strided view
    (torch.empty(6, 14, dtype=torch.float32)[:, ::2], "contiguous"),  # every other column
    ([0.0] * 42, "tensor"),                                           # not a tensor
])
def test_check_out_rejects(t, msg):
    with pytest.raises(ValueError, match=msg):
        api._check_out(t, "o", 42, (torch.float32,), CPU)


def test_check_out_rejects_other_device():
    with pytest.raises(ValueError, match="is on"):
        api._check_out(torch.empty(42, dtype=torch.float32), "o", 42, (torch.float32,), torch.device("meta"))


def test_check_maps():
    good = {"sum_i": torch.empty(3, 5, dtype=torch.int32), "coef": torch.empty(3, 5, dtype=torch.float32)}
    api._check_maps(good, 3, 5, CPU)
    with pytest.raises(ValueError, match="dtype"):
        api._check_maps({"coef": torch.empty(3, 5, dtype=torch.int32)}, 3, 5, CPU)
    with pytest.raises(ValueError, match="dtype"):
        api._check_maps({"sum_it": torch.empty(3, 5, dtype=torch.float32)}, 3, 5, CPU)
    with pytest.raises(ValueError, match="elements"):
        api._check_maps({"sum_isq": torch.empty(3, 4, dtype=torch.int32)}, 3, 5, CPU)
    with pytest.raises(ValueError, match="unknown"):
        api._check_maps({"peak": torch.empty(3, 5, dtype=torch.int32)}, 3, 5, CPU)


def test_check_bytes():
    api._check_bytes(torch.empty(_lib.PEAK_BYTES // 8, dtype=torch.int64), "peak", _lib.PEAK_BYTES, CPU)
    api._check_bytes(torch.empty(100, dtype=torch.uint8), "ws", 100, CPU)
    with pytest.raises(ValueError, match="bytes"):
        api._check_bytes(torch.empty(2, dtype=torch.int64), "peak", _lib.PEAK_BYTES, CPU)
    with pytest.raises(ValueError, match="contiguous"):
        api._check_bytes(torch.empty(64, dtype=torch.uint8)[::2], "ws", 16, CPU)
    with pytest.raises(ValueError, match="is on"):
        api._check_bytes(torch.empty(64, dtype=torch.uint8), "ws", 16, torch.device("meta"))
