"""Helpers for the GPU parity tests: upload seeded operands, run the library
through its C ABI binding, and compare with the CPU reference (full or at
seeded sample positions)."""
import sys

import numpy as np

import oracle
import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import inputs

FULL_CHECK_MAX = 1024 ** 3     # full M x N comparison up to this M*N*K


def note(msg):
    """Name the case before the GPU work starts, and flush."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def run(A_np, B_np, cfg=None, out=None):
    """C = A x B on the GPU through the binding; returns C as numpy float32."""
    import torch
    A, B = to_device(A_np), to_device(B_np)
    C = sg.sgemm(A, B, out=out, cfg=cfg)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check_full(C, A, B, tol=oracle.TOL):
    ref, absb = oracle.sgemm_ref(A, B)
    rep = oracle.compare(C, ref, absb, tol)
    assert rep["n_bad"] == 0, rep
    return rep


def check_sampled(C, A, B, seed, last=0, tol=oracle.TOL):
    M, N = C.shape
    rows, cols = inputs.sample_indices(M, N, seed, last=last)
    ref, absb = oracle.sgemm_ref_sampled(A, B, rows, cols)
    rep = oracle.compare(C[rows, cols], ref, absb, tol)
    assert rep["n_bad"] == 0, rep
    return rep


def forced(vid, group_m=8, xcd_remap=1):
    cfg = sg.SgemmCfg()
    cfg.id = vid
    cfg.group_m = group_m
    cfg.xcd_remap = xcd_remap
    return cfg


def place(x, pad=0, shift=0):
    """Upload a 2-D float32 array into a device buffer whose rows are `pad`
    floats longer than needed and whose start is `shift` floats past an
    allocation (shift 1: only 4-byte aligned); returns the view."""
    import torch
    rows, cols = x.shape
    ld = cols + pad
    buf = torch.zeros(shift + rows * ld + 4, dtype=torch.float32, device="cuda")
    view = buf[shift:shift + rows * ld].view(rows, ld)[:, :cols] if rows * ld else \
        torch.zeros((rows, cols), dtype=torch.float32, device="cuda")
    if x.size:
        view.copy_(torch.from_numpy(np.ascontiguousarray(x)))
    return view


def stored(X, trans):
    """The array stored for operand X (its transpose when trans)."""
    return np.ascontiguousarray(X.T) if trans else X


def run_general(As, Bs, ta, tb, alpha=1.0, beta=0.0, C0=None, cfg=None, workspace=True,
                pad=(0, 0, 0), shift=(0, 0, 0)):
    """alpha * op(As) @ op(Bs) + beta * C0 on the GPU; returns C as numpy."""
    import torch
    M = As.shape[1] if ta else As.shape[0]
    N = Bs.shape[0] if tb else Bs.shape[1]
    A = place(As, pad[0], shift[0])
    B = place(Bs, pad[1], shift[1])
    C = place(C0 if C0 is not None else np.full((M, N), np.nan, np.float32), pad[2], shift[2])
    sg.sgemm(A, B, out=C, cfg=cfg, transa=ta, transb=tb, alpha=alpha, beta=beta,
             workspace=workspace)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def check_general(C, As, Bs, ta, tb, alpha=1.0, beta=0.0, C0=None, tol=oracle.TOL):
    ref, absb = oracle.gemm_ref(As, Bs, ta, tb, alpha, beta, C0)
    rep = oracle.compare(C, ref, absb, tol)
    assert rep["n_bad"] == 0, rep
    return rep


def forced_split(vid, splits, group_m=8, xcd_remap=1):
    cfg = forced(vid, group_m, xcd_remap)
    cfg.splits = splits
    return cfg
