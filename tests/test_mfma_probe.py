"""The matrix-core probe beside the library (include/mfma_probe.h): one small
launch runs and leaves finite, non-zero sums.  Its products are a measurement
load, not part of the attention path; that it issues exactly 4 products per
iteration per wave is checked by the SQ_INSTS_MFMA counter in the committed
profile."""

import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_probe_launch():
    L = ctypes.CDLL(os.path.join(ROOT, "attention_forward_mode_amd", "libmfma_probe.so"))
    f = L.mfma_probe_launch
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    wgs, iters = 8, 64
    sink = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    print(f"  launch mfma_probe_kernel workgroups={wgs} iters={iters}", flush=True)
    assert f(wgs, iters, ctypes.c_void_p(sink.data_ptr()), stream) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    assert (sink != 0).any()
