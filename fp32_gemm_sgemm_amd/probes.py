"""ctypes binding of libsgemm_probes.so: measurement probes that put the
GEMM's numbers in context (not part of the product path)."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES_PATH = os.path.join(HERE, "libsgemm_probes.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (same HIP runtime as torch)
        if not os.path.exists(PROBES_PATH):
            raise RuntimeError(f"{PROBES_PATH} is not built")
        lib = ctypes.CDLL(PROBES_PATH)
        lib.sgemm_probe_mfma_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                              ctypes.c_void_p]
        lib.sgemm_probe_mfma_peak.restype = ctypes.c_int
        lib.sgemm_probe_mfma_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.sgemm_probe_mfma_peak_flops.restype = ctypes.c_double
        lib.sgemm_probe_valu_peak.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                              ctypes.c_void_p]
        lib.sgemm_probe_valu_peak.restype = ctypes.c_int
        lib.sgemm_probe_valu_peak_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.sgemm_probe_valu_peak_flops.restype = ctypes.c_double
        lib.sgemm_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.sgemm_probe_empty.restype = ctypes.c_int
        _lib = lib
    return _lib


def _best_tflops(launch, flops, wgs, iters, reps):
    import torch
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    best = 0.0
    for rep in range(reps + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = launch(wgs, iters, out.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"probe launch failed with hipError_t {rc}")
        torch.cuda.synchronize()
        if rep:
            t = e0.elapsed_time(e1) * 1e-3
            best = max(best, flops(wgs, iters) / t / 1e12)
    if not torch.isfinite(out).all():
        raise RuntimeError("probe produced non-finite values")
    return best


def _cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def mfma_peak_tflops(workgroups_per_cu=2, iters=20000, reps=3):
    """Sustained v_mfma_f32_32x32x2_f32 throughput of the whole chip, TFLOP/s
    (best of `reps` launches after one warm-up)."""
    lib = load()
    return _best_tflops(lib.sgemm_probe_mfma_peak, lib.sgemm_probe_mfma_peak_flops,
                        _cus() * workgroups_per_cu, iters, reps)


def valu_peak_tflops(workgroups_per_cu=16, iters=40000, reps=3):
    """Sustained single-precision v_fma_f32 throughput of the whole chip
    (non-packed, 16 independent chains per thread, 16 workgroups of 4 waves per CU), TFLOP/s
    (best of `reps` launches after one warm-up)."""
    lib = load()
    return _best_tflops(lib.sgemm_probe_valu_peak, lib.sgemm_probe_valu_peak_flops,
                        _cus() * workgroups_per_cu, iters, reps)


def empty_launch(workgroups=256):
    """A launch of `workgroups` empty workgroups of 512 threads (the grid of
    the 512^3 plan): returns a callable that enqueues it on the current
    stream, for timing the floor of such a launch."""
    import torch
    lib = load()
    out = torch.empty(workgroups, dtype=torch.float32, device="cuda")

    def launch():
        rc = lib.sgemm_probe_empty(workgroups, out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"probe launch failed with hipError_t {rc}")
    launch.out = out
    return launch
