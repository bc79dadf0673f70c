"""GPU sanity checks of the peak-rate probes (libsa_probes.so) that bench.py --peak-probes uses to
re-measure the bf16 MFMA rate and the HBM read rate; needs an MI355X.  A probe whose work count
were wrong would show a rate above the published peak (2.5 PFLOP/s dense bf16, 8 TB/s HBM)."""
import ctypes
import os

import pytest
import torch

from gpu_util import announce

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_flash_amd", "libsa_probes.so"))
    V, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.sa_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.sa_probe_mfma_bf16_flops.argtypes = [I, I]
    lib.sa_probe_mfma_bf16.argtypes = [V, I, I, I, V]
    lib.sa_probe_read.argtypes = [V, Z, V, I, V]
    return lib


def _time(fn, reps=5):
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


@pytest.mark.parametrize("random_operands", [1, 0])
def test_mfma_probe_rate_is_below_the_published_peak(random_operands):
    announce(f"mfma probe, random operands {random_operands}")
    lib = _lib()
    wgs, iters = 1024, 4000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ms = _time(lambda: lib.sa_probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()), wgs, iters,
                                              random_operands, stream))
    tflops = lib.sa_probe_mfma_bf16_flops(wgs, iters) / ms / 1e9
    announce(f"mfma probe {tflops:.0f} TFLOP/s")
    assert torch.isfinite(out).all()
    assert 500.0 < tflops < 2500.0


def test_read_probe_rate_is_below_the_published_peak():
    announce("read probe")
    lib = _lib()
    nbytes = 1 << 28
    bufs = [torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(4)]
    sink = torch.empty(512 * 512, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    turn = [0]

    def read():
        x = bufs[turn[0] % 4]
        turn[0] += 1
        assert lib.sa_probe_read(ctypes.c_void_p(x.data_ptr()), nbytes,
                                 ctypes.c_void_p(sink.data_ptr()), 512, stream) == 0
    ms = _time(read, 8)
    gbps = nbytes / ms / 1e6
    announce(f"read probe {gbps:.0f} GB/s")
    assert (sink == 0).all()     # XOR of zeros: every lane ran to its store
    assert 1000.0 < gbps < 8000.0
