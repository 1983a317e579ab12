"""ctypes binding of libmoepeaks.so (include/moe_peaks.h): the achievable HBM
read rate and the achievable dense bf16 MFMA rate of the GPU in use, measured
with two microbenchmarks, for comparison with the layer's kernels."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoepeaks.so")

_LIB = None


def load():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_layer_38_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.peak_stream_read.argtypes = [vp, sz, i32, vp, vp]
    lib.peak_stream_read.restype = i32
    lib.peak_stream_sink_words.argtypes = [i32]
    lib.peak_stream_sink_words.restype = sz
    lib.peak_mfma_loop.argtypes = [vp, i32, i32, vp, vp]
    lib.peak_mfma_loop.restype = i32
    lib.peak_mfma_data_bytes.restype = sz
    lib.peak_mfma_sink_words.argtypes = [i32]
    lib.peak_mfma_sink_words.restype = sz
    lib.peak_mfma_flops.argtypes = [i32, i32]
    lib.peak_mfma_flops.restype = ctypes.c_double
    _LIB = lib
    return lib


def _time(fn, reps: int) -> float:
    """Median milliseconds of one fn() call over reps calls (HIP events on the current stream)."""
    import torch
    fn()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    ms.sort()
    return ms[len(ms) // 2]


def hbm_read_gbs(nbytes: int = 4 << 30, grids=(256, 512, 1024, 2048, 4096), reps: int = 10):
    """Achievable read rate in GB/s: one pass over an nbytes buffer (far larger
    than the L2 and the 256 MB last-level cache), the best over a few grid
    sizes.  Returns (GB/s, workgroups of the best grid)."""
    import torch
    lib = load()
    buf = torch.randint(0, 1 << 30, (nbytes // 4,), dtype=torch.int32, device="cuda")
    sink = torch.empty(lib.peak_stream_sink_words(max(grids)), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = (0.0, 0)
    for blocks in grids:
        def run():
            if lib.peak_stream_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), stream) != 0:
                raise RuntimeError("peak_stream_read failed")
        gbs = nbytes / (_time(run, reps) * 1e-3) / 1e9
        best = max(best, (gbs, blocks))
    del buf
    return best


def mfma_bf16_tfs(iters: int = 20000, blocks: int = 1024, reps: int = 5) -> float:
    """Achievable dense bf16 MFMA rate in TFLOP/s (random register operands)."""
    import torch
    lib = load()
    g = torch.Generator(device="cuda").manual_seed(7)
    n = lib.peak_mfma_data_bytes() // 4
    data = torch.randint(-(1 << 30), 1 << 30, (n,), dtype=torch.int32, device="cuda", generator=g)
    # bf16 values below 2 in magnitude with random signs: clear the top exponent bit of each half
    data = data & -1073758209  # 0xBFFFBFFF
    sink = torch.empty(lib.peak_mfma_sink_words(blocks), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        if lib.peak_mfma_loop(data.data_ptr(), iters, blocks, sink.data_ptr(), stream) != 0:
            raise RuntimeError("peak_mfma_loop failed")
    ms = _time(run, reps)
    return lib.peak_mfma_flops(iters, blocks) / (ms * 1e-3) / 1e12
