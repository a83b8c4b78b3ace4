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
