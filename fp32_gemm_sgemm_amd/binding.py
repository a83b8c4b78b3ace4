"""ctypes binding of libsgemm.so: the C ABI of include/sgemm.h under the same
names, plus `sgemm(A, B, out=None)` for torch tensors.  Argument marshalling
only: the product is computed by the library's HIP kernels, and nothing here
falls back to another implementation.  If the library is missing, every call
raises.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (both carry the soname libamdhip64.so.7):
streams and device pointers from torch are then valid in the library.
"""
import contextlib
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsgemm.so")
# The LDS race check build of the same sources (LDS words set to NaN before
# each refill); only tests route calls to it, through library().
POISON_LIB_PATH = os.path.join(HERE, "libsgemm_lds_poison.so")
# The timeline build (clock readings inside the direct-load kernel, read
# through the functions of include/sgemm_timeline.h); timeline.py drives it.
TIMELINE_LIB_PATH = os.path.join(HERE, "libsgemm_timeline.so")

SGEMM_KERNEL_MFMA = 0
SGEMM_KERNEL_VALU = 1


class SgemmError(RuntimeError):
    def __init__(self, code, where):
        super().__init__(f"{where} failed with hipError_t {code}")
        self.code = code


SGEMM_OP_N = 0
SGEMM_OP_T = 1


class SgemmCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "id", "kernel", "bm", "bn", "bk", "waves_m", "waves_n",
        "group_m", "xcd_remap", "splits", "k_chunk", "grid", "threads",
        "lds_bytes", "tiles_m", "tiles_n")] + [("workspace_bytes", ctypes.c_longlong)] + [
        (n, ctypes.c_int) for n in ("strip_m", "strip_n", "fixed_ns", "spill_permille",
                                 "spill_full_permille", "coresident")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_libs = {}      # loaded builds by path
_active = None  # path calls go to while library() is in effect (None: LIB_PATH)


@contextlib.contextmanager
def library(path):
    """Route every call of this module to another build of the library (such
    as POISON_LIB_PATH) until the block ends.  Not thread-safe: meant for
    tests."""
    global _active
    load(path)
    prev, _active = _active, path
    try:
        yield
    finally:
        _active = prev


def load(path=None):
    """Load a build of the library once (by default libsgemm.so, or the one
    library() selected); raise if it is not built."""
    path = path or _active or LIB_PATH
    if path in _libs:
        return _libs[path]
    try:
        import torch  # noqa: F401  (binds the shared HIP runtime first)
    except ImportError:  # pragma: no cover
        pass
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m fp32_gemm_sgemm_amd.build` first")
    lib = ctypes.CDLL(path)
    i, p, f = ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    ll, sz = ctypes.c_longlong, ctypes.c_size_t
    cfgp = ctypes.POINTER(SgemmCfg)
    sigs = {
        "sgemm_f32": [i, i, i, p, i, p, i, p, i, p],
        "sgemm_f32_gemm": [i, i, i, i, i, f, p, i, p, i, f, p, i, p, sz, p],
        "sgemm_f32_strided_batched": [i, i, i, i, i, f, p, i, ll, p, i, ll, f, p, i, ll, i, p, sz, p],
        "sgemm_f32_ex": [i, i, i, i, i, f, p, i, ll, p, i, ll, f, p, i, ll, i, p, sz, p, cfgp],
        "sgemm_f32_ex_noalloc": [i, i, i, i, i, f, p, i, ll, p, i, ll, f, p, i, ll, i, p, cfgp],
        "sgemm_f32_workspace_size": [i, i, i, i, i, i, i, i, i, ctypes.POINTER(sz)],
        "sgemm_f32_plan": [i, i, i, i, i, i, i, i, i, i, ll, cfgp],
        "sgemm_f32_cfg_geometry": [i, i, i, i, i, i, i, i, i, cfgp],
        "sgemm_f32_query": [i, i, i, i, i, p, i, ll, p, i, ll, p, i, ll, i, p, sz, cfgp],
        "sgemm_f32_num_variants": [],
        "sgemm_f32_variant": [i, cfgp],
        "sgemm_f32_variant_ops": [i],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = i
    lib.sgemm_f32_version.argtypes = []
    lib.sgemm_f32_version.restype = ctypes.c_char_p
    if hasattr(lib, "sgemm_f32_timeline_read"):  # the timeline build only
        ip = ctypes.POINTER(i)
        lib.sgemm_f32_timeline_layout.argtypes = [ip, ip, ip, ip]
        lib.sgemm_f32_timeline_read.argtypes = [p, sz, p, sz]
        lib.sgemm_f32_timeline_clear.argtypes = []
        lib.sgemm_f32_timeline_clock_khz.argtypes = [ip]
        for name in ("sgemm_f32_timeline_layout", "sgemm_f32_timeline_read",
                     "sgemm_f32_timeline_clear", "sgemm_f32_timeline_clock_khz"):
            getattr(lib, name).restype = i
    _libs[path] = lib
    return lib


def _check(code, where):
    if code != 0:
        raise SgemmError(code, where)


def sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=0):
    """Raw ABI call with integer device addresses; returns the hipError_t."""
    return load().sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream)


def sgemm_f32_gemm(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                   workspace=0, workspace_bytes=0, stream=0):
    return load().sgemm_f32_gemm(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta,
                                 C, ldc, workspace, workspace_bytes, stream)


def sgemm_f32_strided_batched(transa, transb, M, N, K, alpha, A, lda, stride_a, B, ldb,
                              stride_b, beta, C, ldc, stride_c, batch,
                              workspace=0, workspace_bytes=0, stream=0):
    return load().sgemm_f32_strided_batched(
        transa, transb, M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b, beta,
        C, ldc, stride_c, batch, workspace, workspace_bytes, stream)


def sgemm_f32_ex(transa, transb, M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b,
                 beta, C, ldc, stride_c, batch, workspace=0, workspace_bytes=0,
                 stream=0, cfg=None):
    ref = ctypes.byref(cfg) if cfg is not None else None
    return load().sgemm_f32_ex(transa, transb, M, N, K, alpha, A, lda, stride_a, B, ldb,
                               stride_b, beta, C, ldc, stride_c, batch, workspace,
                               workspace_bytes, stream, ref)


# Bytes of the library's per-GPU scratch (SGEMM_SCRATCH_BYTES in sgemm.h).
SGEMM_SCRATCH_BYTES = 32 << 20


def sgemm_f32_ex_noalloc(transa, transb, M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b,
                         beta, C, ldc, stride_c, batch, stream=0, cfg=None):
    """Raw ABI call; K splits use the library's static per-GPU scratch."""
    ref = ctypes.byref(cfg) if cfg is not None else None
    return load().sgemm_f32_ex_noalloc(transa, transb, M, N, K, alpha, A, lda, stride_a, B,
                                       ldb, stride_b, beta, C, ldc, stride_c, batch, stream, ref)


def sgemm_f32_workspace_size(transa, transb, M, N, K, lda, ldb, ldc, batch=1):
    out = ctypes.c_size_t(0)
    _check(load().sgemm_f32_workspace_size(transa, transb, M, N, K, lda, ldb, ldc, batch,
                                           ctypes.byref(out)), "sgemm_f32_workspace_size")
    return out.value


def sgemm_f32_plan(M, N, K, lda, ldb, ldc, num_cus=0, transa=0, transb=0, batch=1,
                   workspace_bytes=0):
    out = SgemmCfg()
    _check(load().sgemm_f32_plan(transa, transb, M, N, K, lda, ldb, ldc, batch, num_cus,
                                 workspace_bytes, ctypes.byref(out)), "sgemm_f32_plan")
    return out


def sgemm_f32_cfg_geometry(cfg, transa, transb, M, N, K, lda, ldb, ldc, batch=1):
    """Copy of a forced configuration with its launch geometry filled in."""
    out = SgemmCfg.from_buffer_copy(cfg)
    _check(load().sgemm_f32_cfg_geometry(transa, transb, M, N, K, lda, ldb, ldc, batch,
                                         ctypes.byref(out)), "sgemm_f32_cfg_geometry")
    return out


def sgemm_f32_query(transa, transb, M, N, K, A, lda, stride_a, B, ldb, stride_b, C, ldc,
                    stride_c, batch=1, workspace=0, workspace_bytes=0):
    out = SgemmCfg()
    _check(load().sgemm_f32_query(transa, transb, M, N, K, A, lda, stride_a, B, ldb, stride_b,
                                  C, ldc, stride_c, batch, workspace, workspace_bytes,
                                  ctypes.byref(out)), "sgemm_f32_query")
    return out


def sgemm_f32_num_variants():
    return load().sgemm_f32_num_variants()


def sgemm_f32_variant(vid):
    out = SgemmCfg()
    _check(load().sgemm_f32_variant(vid, ctypes.byref(out)), "sgemm_f32_variant")
    return out


def sgemm_f32_variant_ops(vid):
    return load().sgemm_f32_variant_ops(vid)


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


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream, (stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _workspace(nbytes, device, stream):
    """Scratch device memory from torch's caching allocator, tied to `stream`."""
    import torch
    if nbytes <= 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if hasattr(stream, "cuda_stream") and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


def _operand(t, trans, name):
    """(rows, cols of op(t), row stride of t) for a 2-D row-major operand."""
    rows, cols, ld = _row_major_view(t, name)
    return (cols, rows, ld) if trans else (rows, cols, ld)


def sgemm(A, B, out=None, stream=None, cfg=None, transa=False, transb=False,
          alpha=1.0, beta=0.0, workspace=True):
    """C = alpha * op(A) @ op(B) + beta * C for float32 device tensors.

    op(X) is X, or X.T when trans* is set: a transposed operand is passed as
    stored (for example the K x M tensor whose transpose is the M x K
    operand), never copied.  `out`, if given, is written in place (it may have
    a row stride larger than N) and is read only when beta != 0.  With
    `workspace` true the library may split K across workgroups, using scratch
    memory from torch's caching allocator; false forbids it, and a uint8
    device tensor supplies the scratch memory itself.  The work is enqueued on
    `stream` (default: torch's current stream); this call does not
    synchronise.
    """
    import torch
    M, K, lda = _operand(A, transa, "A")
    K2, N, ldb = _operand(B, transb, "B")
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be device tensors on the same GPU")
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs `out`")
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    Mo, No, ldc = _row_major_view(out, "out")
    if (Mo, No) != (M, N) or out.device != A.device:
        raise ValueError("out has the wrong shape or device")
    ta, tb = int(bool(transa)), int(bool(transb))
    with torch.cuda.device(A.device):
        stream, handle = _stream_handle(stream, A.device)
        ws, ws_ptr, ws_bytes = _pick_workspace(workspace, cfg, ta, tb, M, N, K, lda, ldb, ldc,
                                               1, A.device, stream)
        code = sgemm_f32_ex(ta, tb, M, N, K, float(alpha), A.data_ptr(), lda, 0,
                            B.data_ptr(), ldb, 0, float(beta), out.data_ptr(), ldc, 0, 1,
                            ws_ptr, ws_bytes, handle, cfg)
    del ws
    _check(code, "sgemm_f32_ex")
    return out


def _pick_workspace(workspace, cfg, ta, tb, M, N, K, lda, ldb, ldc, batch, device, stream):
    """(tensor or None, address, bytes) of the workspace for one call."""
    import torch
    if isinstance(workspace, torch.Tensor):
        if not workspace.is_cuda or workspace.device != device:
            raise ValueError("workspace must be a device tensor on the operands' GPU")
        return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if not workspace:
        return None, 0, 0
    if cfg is not None:
        need = 0
        if cfg.splits > 1:
            need = sgemm_f32_cfg_geometry(cfg, ta, tb, M, N, K, lda, ldb, ldc, batch).workspace_bytes
    else:
        need = sgemm_f32_workspace_size(ta, tb, M, N, K, lda, ldb, ldc, batch)
    ws = _workspace(need, device, stream)
    return ws, (ws.data_ptr() if ws is not None else 0), need


def sgemm_batched(A, B, out=None, stream=None, cfg=None, transa=False, transb=False,
                  alpha=1.0, beta=0.0, workspace=True):
    """out[z] = alpha * op(A[z]) @ op(B[z]) + beta * out[z] for 3-D float32 tensors.

    Each of A, B and out is a (batch, rows, cols) tensor whose matrices are
    row-major with unit column stride; the batch stride may be anything >= 0
    (0 broadcasts one matrix).  One strided-batched launch.
    """
    import torch

    def view(t, name):
        if t.dtype != torch.float32 or t.dim() != 3:
            raise ValueError(f"{name} must be a 3-D float32 tensor")
        rows, cols, ld = _row_major_view(t[0] if t.shape[0] > 0 else t.new_empty(t.shape[1:]), name)
        return t.shape[0], rows, cols, ld, (t.stride(0) if t.shape[0] > 1 else 0)

    ba, ra, ca, lda, sa = view(A, "A")
    bb, rb, cb, ldb, sb = view(B, "B")
    M, K = (ca, ra) if transa else (ra, ca)
    K2, N = (cb, rb) if transb else (rb, cb)
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    batch = max(ba, bb)
    if ba not in (1, batch) or bb not in (1, batch):
        raise ValueError("batch sizes differ")
    if ba == 1:
        sa = 0
    if bb == 1:
        sb = 0
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs `out`")
        out = torch.empty((batch, M, N), dtype=torch.float32, device=A.device)
    bo, Mo, No, ldc, sc = view(out, "out")
    if (bo, Mo, No) != (batch, M, N):
        raise ValueError("out has the wrong shape")
    ta, tb = int(bool(transa)), int(bool(transb))
    with torch.cuda.device(A.device):
        stream, handle = _stream_handle(stream, A.device)
        ws, ws_ptr, ws_bytes = _pick_workspace(workspace, cfg, ta, tb, M, N, K, lda, ldb, ldc,
                                               batch, A.device, stream)
        code = sgemm_f32_ex(ta, tb, M, N, K, float(alpha), A.data_ptr(), lda, sa,
                            B.data_ptr(), ldb, sb, float(beta), out.data_ptr(), ldc, sc, batch,
                            ws_ptr, ws_bytes, handle, cfg)
    del ws
    _check(code, "sgemm_f32_ex")
    return out
