"""The guard-zone helper of the GPU canary tests, checked on the CPU: a byte
written just before or just past a guarded view is reported, the view itself
may be written whole."""
import pytest
import torch

from test_gpu_canaries import GUARD, Guarded


@pytest.mark.parametrize("shape,dtype", [((5, 7), torch.bfloat16), ((3,), torch.int64), ((4, 4), torch.float32),
                                         ((9,), torch.int32), ((1,), torch.bfloat16)])
def test_guard_reports_neighbouring_writes(shape, dtype):
    g = Guarded("t", shape, dtype, "cpu")
    assert g.view.is_contiguous() and tuple(g.view.shape) == shape
    assert g.view.data_ptr() - g.big.data_ptr() == 4 * GUARD
    g.view.fill_(1)
    g.check()
    nbytes = g.view.numel() * g.view.element_size()
    for at in (0, 4 * GUARD - 1, 4 * GUARD + nbytes, 4 * g.big.numel() - 1):
        h = Guarded("t", shape, dtype, "cpu")
        h.view.fill_(1)
        h.big.view(torch.uint8)[at] = 0
        with pytest.raises(AssertionError, match="guard bytes"):
            h.check()
