"""The seeded input generator gives the same bits from numpy and from torch
(CPU here; the GPU variant is in the GPU tests)."""
import numpy as np
import pytest
import torch

import synth


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("start", [0, 12345, (1 << 32) - 1000, (1 << 34) + 7])
def test_numpy_equals_torch_cpu(dtype, start):
    a = synth.values_np(5, 2, start, 50000, 0.5, dtype)
    b = synth.values_torch(5, 2, start, 50000, 0.5, dtype, "cpu", chunk=7000)
    if dtype == "bf16":
        np.testing.assert_array_equal(a, b.view(torch.int16).numpy().view(np.uint16))
    else:
        np.testing.assert_array_equal(a.view(np.uint32), b.numpy().view(np.uint32))


def test_distribution_and_seeds():
    x = synth.unit_values_np(1, 0, 0, 1 << 20)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    assert np.abs(x).max() < 3.47
    y = synth.unit_values_np(2, 0, 0, 1 << 10)
    z = synth.unit_values_np(1, 1, 0, 1 << 10)
    assert not np.array_equal(x[:1024], y) and not np.array_equal(x[:1024], z)


def test_bf16_rounding_rne():
    vals = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3], np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    t = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, t)


def test_row_slices_consistent():
    full = synth.tensor_np(3, 1, (10, 2, 4), 0.5, "bf16")
    part = synth.tensor_np(3, 1, (10, 2, 4), 0.5, "bf16", row_start=3, rows=4)
    np.testing.assert_array_equal(full[3:7], part)


def test_values_at_and_head_slice():
    full = synth.tensor_np(4, 2, (50, 3, 8), 0.5, "bf16")
    np.testing.assert_array_equal(synth.head_slice_np(4, 2, (50, 3, 8), 1, 0.5, "bf16"), full[:, 1:2, :])
    np.testing.assert_array_equal(synth.head_slice_np(4, 2, (50, 3, 8), 2, 0.5, "bf16", 7, 20), full[7:27, 2:3])
    idx = np.array([[5, 900], [1199, 0]])
    np.testing.assert_array_equal(synth.values_at_np(4, 2, idx, 0.5, "bf16"), full.reshape(-1)[idx])
