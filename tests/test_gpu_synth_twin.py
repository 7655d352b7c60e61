"""The device twin of the seeded input generator writes the same bytes as the host one."""
import numpy as np
import pytest

import synth
from gpu_common import cuda_ok

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not cuda_ok(), reason="needs a GPU")]


@pytest.mark.parametrize("first,n", [(0, 1000), (123456789, 4097), (2**40 + 3, 64)])
def test_normal_f32_and_bf16_twins(first, n):
    import torch
    t = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.normal_f32_device(7, 99, first, n, 0.5, t.data_ptr())
    h = synth.normal_f32(7, 99, first, n, 0.5)
    assert np.array_equal(t.cpu().numpy().view(np.uint32), h.view(np.uint32))
    b = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.normal_bf16_device(7, 100, first, n, 0.02, b.data_ptr())
    hb = synth.normal_bf16(7, 100, first, n, 0.02)
    assert np.array_equal(b.cpu().numpy().view(np.uint16), hb)


@pytest.mark.parametrize("row0,rows,cols", [(0, 3, 64), (1000, 5, 7168), (2**30, 2, 2048)])
def test_mxfp4_twins(row0, rows, cols):
    import torch
    c = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    synth.mxfp4_device(3, 555, row0, rows, cols, 0.02, c.data_ptr(), s.data_ptr())
    hc, hs = synth.mxfp4(3, 555, row0, rows, cols, 0.02)
    assert np.array_equal(c.cpu().numpy(), hc)
    assert np.array_equal(s.cpu().numpy(), hs)
