"""ctypes binding of librfw_probes.so (include/atf_probes.h): attainable
dense-bf16 MFMA and HBM-read rates of the GPU, for reading roofline fractions
against measured as well as published peaks.  Argument marshalling and event
timing only; the work runs in the probe kernels."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_HERE, "librfw_probes.so")
_LIB = None


def library():
    global _LIB
    if _LIB is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError("librfw_probes.so is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.atf_probe_mfma_bf16.argtypes = [vp, vp, i32, i32, vp]
        lib.atf_probe_mfma_bf16.restype = ctypes.c_int
        lib.atf_probe_hbm_read.argtypes = [vp, ctypes.c_size_t, vp, i32, vp]
        lib.atf_probe_hbm_read.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _timed(torch, stream, fn, reps):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def mfma_bf16_tflops(torch, device, n_wg: int = 1024, iters: int = 20000, reps: int = 3) -> float:
    """Sustained dense bf16 MFMA rate (TFLOP/s): 8 independent 32x32x16 chains per wave."""
    lib = library()
    stream = torch.cuda.current_stream(device)
    ops = torch.randn(32, device=device).to(torch.bfloat16)
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device=device)

    def run():
        rc = lib.atf_probe_mfma_bf16(ops.data_ptr(), sink.data_ptr(), n_wg, iters, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError("atf_probe_mfma_bf16 failed (%d)" % rc)

    ms = _timed(torch, stream, run, reps)
    return n_wg * 4 * 8 * iters * 32768 / (ms * 1e-3) / 1e12


def hbm_read_gbs(torch, device, nbytes: int = 8 << 30, n_wg: int = 16384, reps: int = 5) -> float:
    """Sustained HBM read rate (GB/s) of one pass over an nbytes buffer."""
    lib = library()
    stream = torch.cuda.current_stream(device)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    buf.fill_(1)
    sink = torch.empty(n_wg * 256, dtype=torch.int32, device=device)

    def run():
        rc = lib.atf_probe_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(), n_wg, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError("atf_probe_hbm_read failed (%d)" % rc)

    ms = _timed(torch, stream, run, reps)
    del buf
    return nbytes / (ms * 1e-3) / 1e9
