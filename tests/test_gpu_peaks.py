"""The measurement helpers of libcskv_peaks.so run on the GPU, leave their sinks untouched (the
never-met condition) and give ceilings of the right order for MI355X."""
import ctypes

import pytest
import torch

from compressed_sparse_kv_03_amd import build_lib
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def test_peak_kernels_run():
    say("peaks")
    L = ctypes.CDLL(build_lib.PEAKS_LIB)
    L.cskv_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.cskv_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    buf = torch.ones(1 << 30, dtype=torch.uint8, device=DEV)  # beyond the 256 MB Infinity Cache
    sink = torch.zeros(4096, dtype=torch.float32, device=DEV)
    assert L.cskv_peak_hbm_read(buf.data_ptr(), buf.numel() - 48, sink.data_ptr(), 4096, stream) == 0
    for kind in range(3):
        assert L.cskv_peak_mfma(kind, 64, 1024, sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(sink)) == 0
    # timed once each: order-of-magnitude checks only (HBM 8 TB/s, bf16 2.5 PFLOP/s, fp4 10.1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    assert L.cskv_peak_hbm_read(buf.data_ptr(), buf.numel(), sink.data_ptr(), 2048, stream) == 0
    e1.record()
    torch.cuda.synchronize()
    gbs = buf.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
    say("hbm read GB/s", round(gbs))
    assert 1000 < gbs < 9000
    e0.record()
    assert L.cskv_peak_mfma(0, 1024, 1024, sink.data_ptr(), stream) == 0
    e1.record()
    torch.cuda.synchronize()
    tf = 1024 * 4 * 1024 * 4 * 32768 / (e0.elapsed_time(e1) / 1e3) / 1e12
    say("bf16 MFMA TFLOP/s", round(tf))
    assert 200 < tf < 2600
