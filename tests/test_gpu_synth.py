"""The seeded generator gives the same bits on the GPU (torch int64 ops) as
numpy on the CPU, so GPU inputs and oracle inputs are the same numbers."""
import numpy as np
import pytest

import synth
from gpu_helpers import need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("start", [0, 999_983, (1 << 32) - 4096, (1 << 33) + 12345])
def test_generator_gpu_equals_numpy(dtype, start):
    need_gpu()
    import torch
    a = synth.values_np(2, 1, start, 1 << 18, 0.5, dtype)
    b = synth.values_torch(2, 1, start, 1 << 18, 0.5, dtype, "cuda", chunk=50000).cpu()
    if dtype == "bf16":
        np.testing.assert_array_equal(a, b.view(torch.int16).numpy().view(np.uint16))
    else:
        np.testing.assert_array_equal(a.view(np.uint32), b.numpy().view(np.uint32))
