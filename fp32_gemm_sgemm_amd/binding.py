"""ctypes binding of libsgemm.so: the C ABI of include/sgemm.h under the same
names, plus `sgemm(A, B, out=None)` for torch tensors.  Argument marshalling
only: the product is computed by the library's HIP kernels, and nothing here
falls back to another implementation.  If the library is missing, every call
raises.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (both carry the soname libamdhip64.so.7):
streams and device pointers from torch are then valid in the library.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsgemm.so")

SGEMM_KERNEL_MFMA = 0
SGEMM_KERNEL_VALU = 1


class SgemmError(RuntimeError):
    def __init__(self, code, where):
        super().__init__(f"{where} failed with hipError_t {code}")
        self.code = code


class SgemmCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "id", "kernel", "bm", "bn", "bk", "waves_m", "waves_n",
        "group_m", "xcd_remap", "grid", "threads", "lds_bytes",
        "tiles_m", "tiles_n")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def load():
    """Load libsgemm.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    try:
        import torch  # noqa: F401  (binds the shared HIP runtime first)
    except ImportError:  # pragma: no cover
        pass
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built: run `python -m fp32_gemm_sgemm_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    i, p = ctypes.c_int, ctypes.c_void_p
    cfgp = ctypes.POINTER(SgemmCfg)
    lib.sgemm_f32.argtypes = [i, i, i, p, i, p, i, p, i, p]
    lib.sgemm_f32.restype = i
    lib.sgemm_f32_ex.argtypes = [i, i, i, p, i, p, i, p, i, p, cfgp]
    lib.sgemm_f32_ex.restype = i
    lib.sgemm_f32_plan.argtypes = [i, i, i, i, i, i, i, cfgp]
    lib.sgemm_f32_plan.restype = i
    lib.sgemm_f32_query.argtypes = [i, i, i, p, i, p, i, p, i, cfgp]
    lib.sgemm_f32_query.restype = i
    lib.sgemm_f32_num_variants.argtypes = []
    lib.sgemm_f32_num_variants.restype = i
    lib.sgemm_f32_variant.argtypes = [i, cfgp]
    lib.sgemm_f32_variant.restype = i
    lib.sgemm_f32_version.argtypes = []
    lib.sgemm_f32_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(code, where):
    if code != 0:
        raise SgemmError(code, where)


def sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=0):
    """Raw ABI call with integer device addresses; returns the hipError_t."""
    return load().sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def sgemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, stream=0, cfg=None):
    ref = ctypes.byref(cfg) if cfg is not None else None
    return load().sgemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, stream, ref)


def sgemm_f32_plan(M, N, K, lda, ldb, ldc, num_cus=0):
    out = SgemmCfg()
    _check(load().sgemm_f32_plan(M, N, K, lda, ldb, ldc, num_cus,
                                 ctypes.byref(out)), "sgemm_f32_plan")
    return out


def sgemm_f32_query(M, N, K, A, lda, B, ldb, C, ldc):
    out = SgemmCfg()
    _check(load().sgemm_f32_query(M, N, K, A, lda, B, ldb, C, ldc,
                                  ctypes.byref(out)), "sgemm_f32_query")
    return out


def sgemm_f32_num_variants():
    return load().sgemm_f32_num_variants()


def sgemm_f32_variant(vid):
    out = SgemmCfg()
    _check(load().sgemm_f32_variant(vid, ctypes.byref(out)), "sgemm_f32_variant")
    return out


def sgemm_f32_version():
    return load().sgemm_f32_version().decode()


def _row_major_view(t, name):
    """(rows, cols, row stride) of a 2-D float32 tensor with unit column stride."""
    import torch
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    ld = t.stride(0) if rows > 1 else max(cols, 1)
    return rows, cols, max(ld, cols, 1)


def sgemm(A, B, out=None, stream=None, cfg=None):
    """C = A @ B for float32 CUDA (HIP) tensors on one device.

    `out`, if given, is written in place (it may have a row stride larger than
    N).  The work is enqueued on `stream` (default: torch's current stream) and
    this call does not synchronise.
    """
    import torch
    M, K, lda = _row_major_view(A, "A")
    K2, N, ldb = _row_major_view(B, "B")
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be device tensors on the same GPU")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    Mo, No, ldc = _row_major_view(out, "out")
    if (Mo, No) != (M, N) or out.device != A.device:
        raise ValueError("out has the wrong shape or device")
    if stream is None:
        stream = torch.cuda.current_stream(A.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(A.device):
        code = sgemm_f32_ex(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                            out.data_ptr(), ldc, handle, cfg)
    _check(code, "sgemm_f32")
    return out
