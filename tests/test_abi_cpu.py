"""The C-ABI library on the host: it loads, exports every entry point that
include/sgemm.h declares, rejects invalid arguments before any HIP call, and
its selector's geometry follows round-up-and-guard sizing.  No compute call
is made here (there may be no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import metrics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")
HIP_ERROR_INVALID_VALUE = 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sg.LIB_PATH):
        from fp32_gemm_sgemm_amd import build
        build.build()
    return sg.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(sgemm_f32\w*)\s*\(", text, re.M)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    assert "sgemm_f32" in names and "sgemm_f32_ex" in names and "sgemm_f32_plan" in names
    assert len(names) >= 7


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sg.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_no_undefined_own_symbols(lib):
    """Every kernel's host-side stub is present (a kernel template whose body
    cannot be compiled for the host would otherwise be left undefined)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", sg.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    assert "sgemm" not in out, out


def test_version_and_variants(lib):
    assert "gfx950" in sg.sgemm_f32_version()
    n = sg.sgemm_f32_num_variants()
    assert n >= 2
    kinds = set()
    for i in range(n):
        v = sg.sgemm_f32_variant(i)
        assert v.id == i
        kinds.add(v.kernel)
        assert v.threads == 64 * v.waves_m * v.waves_n or v.kernel == sg.binding.SGEMM_KERNEL_VALU
        assert 0 < v.lds_bytes <= 160 * 1024
        assert v.bm % 32 == 0 and v.bn % 32 == 0 and v.bk % 8 == 0
    assert kinds == {sg.binding.SGEMM_KERNEL_MFMA, sg.binding.SGEMM_KERNEL_VALU}
    with pytest.raises(sg.SgemmError):
        sg.sgemm_f32_variant(n)
    with pytest.raises(sg.SgemmError):
        sg.sgemm_f32_variant(-1)


# Arguments that must be rejected with hipErrorInvalidValue before any HIP
# call.  Pointers are fake but never dereferenced: validation fails first.
P = 1 << 20  # a 16-byte aligned fake address
BAD = [
    dict(M=-1, N=4, K=4),
    dict(M=4, N=-1, K=4),
    dict(M=4, N=4, K=-1),
    dict(M=4, N=4, K=8, lda=7),          # lda < K
    dict(M=4, N=8, K=4, ldb=7),          # ldb < N
    dict(M=4, N=8, K=4, ldc=7),          # ldc < N
    dict(M=4, N=4, K=0, lda=0),          # lda < 1
    dict(M=4, N=4, K=4, A=0),            # null A with non-zero extent
    dict(M=4, N=4, K=4, B=0),
    dict(M=4, N=4, K=4, C=0),
    dict(M=4, N=4, K=4, A=P + 2),        # not 4-byte aligned
    dict(M=4, N=4, K=4, C=P + 1),
    dict(M=4, N=4, K=4, A=P, C=P + 8),   # C overlaps A
    dict(M=4, N=4, K=4, B=3 * P, C=3 * P + 60),
]


def _call(M, N, K, A=P, lda=None, B=2 * P, ldb=None, C=3 * P, ldc=None):
    lda = max(K, 1) if lda is None else lda
    ldb = max(N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return sg.sgemm_f32(M, N, K, A, lda, B, ldb, C, ldc, 0)


@pytest.mark.parametrize("args", BAD)
def test_invalid_arguments_rejected(lib, args):
    assert _call(**args) == HIP_ERROR_INVALID_VALUE


def test_empty_output_is_a_noop(lib):
    # nothing to compute: success without touching the device or the pointers
    assert _call(0, 5, 7, A=0, B=0, C=0) == 0
    assert _call(5, 0, 7, A=0, B=0, C=0) == 0


def test_ex_rejects_bad_forced_variant(lib):
    cfg = sg.binding.SgemmCfg()
    cfg.id = sg.sgemm_f32_num_variants()
    assert sg.sgemm_f32_ex(4, 4, 4, P, 4, 2 * P, 4, 3 * P, 4, 0, cfg) == HIP_ERROR_INVALID_VALUE
    cfg.id = 0
    cfg.group_m = -1  # negative group height
    assert sg.sgemm_f32_ex(4, 4, 4, P, 4, 2 * P, 4, 3 * P, 4, 0, cfg) == HIP_ERROR_INVALID_VALUE


def test_ex_rejects_limits(lib):
    # lda beyond the 32-bit in-slice offset limit
    assert sg.sgemm_f32(4, 4, 4, P, 1 << 22, 2 * P, 4, 3 * P, 4, 0) == HIP_ERROR_INVALID_VALUE
    assert sg.sgemm_f32(4, 4, 4, P, 4, 2 * P, 1 << 25, 3 * P, 4, 0) == HIP_ERROR_INVALID_VALUE


SHAPES = [(512, 512, 512), (2048, 2048, 2048), (3072, 3072, 3072), (8192, 8192, 4096),
          (4096, 4096, 8192), (4099, 4099, 4099), (8192, 8192, 8192), (1, 1, 1), (5, 3, 0),
          (513, 8192, 1023), (100, 70, 50)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_plan_geometry(lib, M, N, K):
    for cus in (256, 80):
        p = sg.sgemm_f32_plan(M, N, K, max(K, 1), N, N, cus)
        assert p.kernel == sg.binding.SGEMM_KERNEL_MFMA
        assert p.tiles_m == metrics.ceil_div(M, p.bm)
        assert p.tiles_n == metrics.ceil_div(N, p.bn)
        assert p.grid == p.tiles_m * p.tiles_n
        assert p.threads == 64 * p.waves_m * p.waves_n
        assert p.group_m > 0 and p.xcd_remap == 1


def test_selector_prefers_full_waves(lib):
    """Wave quantisation on 256 CUs: 2048^3 has only 64 tiles of 256 x 256 but
    256 of 128 x 128; 3072^3 has 144 of 256 x 256, 576 of 128 x 128 and exactly
    256 of 192 x 192; 8192^3 fills the chip with the largest tile."""
    assert sg.sgemm_f32_plan(2048, 2048, 2048, 2048, 2048, 2048, 256).bm == 128
    p = sg.sgemm_f32_plan(3072, 3072, 3072, 3072, 3072, 3072, 256)
    assert p.grid == 256 and p.bm == 192          # one 192 x 192 tile per CU
    p = sg.sgemm_f32_plan(8192, 8192, 8192, 8192, 8192, 8192, 256)
    assert p.grid * p.bm * p.bn == 8192 * 8192


def test_plan_rejects_invalid(lib):
    out = sg.binding.SgemmCfg()
    assert lib.sgemm_f32_plan(-1, 4, 4, 4, 4, 4, 256, ctypes.byref(out)) == HIP_ERROR_INVALID_VALUE
    assert lib.sgemm_f32_plan(4, 4, 8, 4, 4, 4, 256, ctypes.byref(out)) == HIP_ERROR_INVALID_VALUE
    assert lib.sgemm_f32_plan(4, 4, 4, 4, 4, 4, 256, None) == HIP_ERROR_INVALID_VALUE
