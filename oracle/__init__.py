"""CPU reference for single-precision GEMM, and the acceptance check.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline leg
of the benchmark use this package; the product path (the HIP library and its
Python binding) never imports it, and this package imports nothing from the
product.

What it computes (oracle.c holds the arithmetic):
  ref[i, j]  = sum over ascending k of float64(A[i, k]) * float64(B[k, j])
  absb[i, j] = sum over k of |float64(A[i, k]) * float64(B[k, j])|
for row-major A (M x K) and B (K x N): the definition C = A x B of
"4.1 CUDA GEMM operator performance optimization", section 1.1, with the
double-accumulating CPU reference of the DD2360 workbook ("Applied GPU
Programming"), section 14.3, lab "tiled matmul, square case".

The general form used by the library's BLAS-style entry points,
  C = alpha * op(A) x op(B) + beta * C0,   op(X) = X or its transpose,
is taken in float64 on top of that: gemm_ref forms op(A) and op(B) with
numpy's transpose of the stored operand (a transposed operand is the matrix
stored the other way round, as a row-major matrix looks to a column-major
library: DD2360 workbook, Module 15, section 15.2), computes the product
above, and returns
  ref  = alpha * ref_AB + beta * C0
  absb = |alpha| * absb_AB + |beta * C0|
with C0 not read at all when beta == 0 and A, B not read when alpha == 0
(BLAS conventions, which the pages do not spell out).  gemm_ref_batched
repeats it per batch entry, as for the batched products of multi-head
attention ("4.1 CUDA GEMM operator performance optimization", section 1.2).

Acceptance: |C - ref| <= 1e-4 * absb for every checked element, and C finite.
The workbook's lab uses 1e-4 relative to |ref|; absb >= |ref| always and does
not collapse when the terms cancel, so the bound is taken relative to absb.
"""
import ctypes
import os

import numpy as np

from .build import LIB

TOL = 1e-4

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(
                f"{LIB} is missing: build it with `python oracle/build.py`")
        lib = ctypes.CDLL(LIB)
        i64, ptr = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_sgemm_full.argtypes = [i64, i64, i64, ptr, i64, ptr, i64,
                                          ptr, ptr, i64, ctypes.c_int]
        lib.oracle_sgemm_full.restype = ctypes.c_int
        lib.oracle_sgemm_sampled.argtypes = [i64, i64, i64, ptr, i64, ptr, i64,
                                             i64, ptr, ptr, ptr, ptr,
                                             ctypes.c_int]
        lib.oracle_sgemm_sampled.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads the oracle uses: the cores this process may run on,
    capped at 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _as_f32_2d(x, name):
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError(f"{name} must be a 2-D float32 array")
    if x.size and ((x.shape[1] > 1 and x.strides[1] != 4) or x.strides[0] % 4 != 0
                   or x.strides[0] < 0):
        raise ValueError(f"{name} must have unit column stride")
    return x


def sgemm_ref(A, B, nthreads=None):
    """Full product: returns (ref, absb), both float64 of shape (M, N).

    A is (M, K) float32, B is (K, N) float32; row strides may exceed the
    widths (leading dimensions), column strides must be 1.
    """
    A = _as_f32_2d(A, "A")
    B = _as_f32_2d(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    ref = np.zeros((M, N), dtype=np.float64)
    absb = np.zeros((M, N), dtype=np.float64)
    lda = max(A.strides[0] // 4, K, 1)
    ldb = max(B.strides[0] // 4, N, 1)
    rc = _load().oracle_sgemm_full(
        M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
        ref.ctypes.data, absb.ctypes.data, max(N, 1),
        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_full failed with code {rc}")
    return ref, absb


def sgemm_ref_sampled(A, B, rows, cols, nthreads=None):
    """The outputs at (rows[t], cols[t]): returns (ref, absb), float64 1-D."""
    A = _as_f32_2d(A, "A")
    B = _as_f32_2d(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D and of equal length")
    n = rows.shape[0]
    ref = np.zeros(n, dtype=np.float64)
    absb = np.zeros(n, dtype=np.float64)
    lda = max(A.strides[0] // 4, K, 1)
    ldb = max(B.strides[0] // 4, N, 1)
    rc = _load().oracle_sgemm_sampled(
        M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb, n,
        rows.ctypes.data, cols.ctypes.data, ref.ctypes.data, absb.ctypes.data,
        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_sgemm_sampled failed with code {rc}")
    return ref, absb


def gemm_ref(A, B, transa=False, transb=False, alpha=1.0, beta=0.0, C0=None, nthreads=None):
    """General form: returns (ref, absb) of alpha * op(A) @ op(B) + beta * C0.

    A and B are the stored float32 operands: op(A) is A (M x K) or, with
    transa, A.T for A stored K x M; likewise B (K x N, or N x K with transb).
    C0 (M x N, float32) is read only when beta != 0.
    """
    A = _as_f32_2d(A, "A")
    B = _as_f32_2d(B, "B")
    opa = np.ascontiguousarray(A.T) if transa else A
    opb = np.ascontiguousarray(B.T) if transb else B
    M, K = opa.shape
    K2, N = opb.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    if alpha != 0.0 and K > 0:
        ab, ab_abs = sgemm_ref(opa, opb, nthreads)
        ref = alpha * ab
        absb = abs(alpha) * ab_abs
    else:
        ref = np.zeros((M, N), dtype=np.float64)
        absb = np.zeros((M, N), dtype=np.float64)
    if beta != 0.0:
        if C0 is None:
            raise ValueError("beta != 0 needs C0")
        c0 = np.asarray(C0, dtype=np.float64)
        if c0.shape != (M, N):
            raise ValueError("C0 has the wrong shape")
        ref = ref + beta * c0
        absb = absb + np.abs(beta * c0)
    return ref, absb


def gemm_ref_batched(A, B, transa=False, transb=False, alpha=1.0, beta=0.0, C0=None,
                     nthreads=None):
    """gemm_ref per batch entry of 3-D stacks (a stack of one broadcasts)."""
    A = np.asarray(A)
    B = np.asarray(B)
    if A.ndim != 3 or B.ndim != 3:
        raise ValueError("A and B must be 3-D stacks")
    batch = max(A.shape[0], B.shape[0])
    if A.shape[0] not in (1, batch) or B.shape[0] not in (1, batch):
        raise ValueError("batch sizes differ")
    refs, absbs = [], []
    for z in range(batch):
        a = A[z if A.shape[0] > 1 else 0]
        b = B[z if B.shape[0] > 1 else 0]
        c0 = None if C0 is None else C0[z]
        r, s = gemm_ref(a, b, transa, transb, alpha, beta, c0, nthreads)
        refs.append(r)
        absbs.append(s)
    if not refs:
        return np.zeros((0, 0, 0)), np.zeros((0, 0, 0))
    return np.stack(refs), np.stack(absbs)


def compare(C, ref, absb, tol=TOL):
    """Check C against the reference: |C - ref| <= tol * absb and C finite.

    Returns a dict: n (checked), n_bad, max_norm_err (max |C-ref|/absb, with
    0/0 read as 0 and x/0 as inf), rrmse (sqrt(sum (C-ref)^2 / sum ref^2),
    reported, not gated) and first_bad (flat index of the first violation or
    -1).
    """
    c = np.asarray(C, dtype=np.float64).reshape(-1)
    r = np.asarray(ref, dtype=np.float64).reshape(-1)
    s = np.asarray(absb, dtype=np.float64).reshape(-1)
    if not (c.shape == r.shape == s.shape):
        raise ValueError("C, ref and absb must have the same number of elements")
    finite = np.isfinite(c)
    err = np.where(finite, np.abs(c - r), np.inf)
    ok = finite & (err <= tol * s)
    with np.errstate(divide="ignore", invalid="ignore"):
        norm = np.where(s > 0, err / np.where(s > 0, s, 1.0),
                        np.where(err > 0, np.inf, 0.0))
    bad = np.flatnonzero(~ok)
    den = float(np.sum(r * r))
    num = float(np.sum(np.where(finite, (c - r) ** 2, np.inf)))
    return {
        "n": int(c.size),
        "n_bad": int(bad.size),
        "max_norm_err": float(norm.max()) if c.size else 0.0,
        "rrmse": (num / den) ** 0.5 if den > 0 else (0.0 if num == 0 else float("inf")),
        "first_bad": int(bad[0]) if bad.size else -1,
    }
