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


@pytest.mark.parametrize("path", [sg.LIB_PATH, sg.POISON_LIB_PATH, sg.TIMELINE_LIB_PATH],
                         ids=["product", "lds_poison", "timeline"])
def test_every_declared_symbol_is_exported(lib, path):
    """The product library, its LDS race check build and its timeline build
    export every entry point the header declares."""
    out = subprocess.run(["nm", "-D", "--defined-only", path],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    handle = sg.load(path)
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(handle, name)


def timeline_functions():
    text = open(os.path.join(ROOT, "include", "sgemm_timeline.h")).read()
    return sorted(set(re.findall(r"^\s*int\s*(sgemm_f32_timeline\w*)\s*\(", text, re.M)))


def test_timeline_functions_only_in_the_timeline_build(lib):
    """include/sgemm_timeline.h's functions are exported by the timeline build
    and by no other; without a GPU, layout() reports the array sizes and
    read() refuses oversized copies before any HIP call."""
    names = timeline_functions()
    assert names == ["sgemm_f32_timeline_clear", "sgemm_f32_timeline_clock_khz",
                     "sgemm_f32_timeline_layout", "sgemm_f32_timeline_read"]

    def exported(path):
        out = subprocess.run(["nm", "-D", "--defined-only", path],
                             capture_output=True, text=True, check=True).stdout
        return {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(names) <= exported(sg.TIMELINE_LIB_PATH)
    assert not set(names) & exported(sg.LIB_PATH)
    assert not set(names) & exported(sg.POISON_LIB_PATH)
    tl = sg.load(sg.TIMELINE_LIB_PATH)
    vals = [ctypes.c_int() for _ in range(4)]
    assert tl.sgemm_f32_timeline_layout(*[ctypes.byref(v) for v in vals]) == 0
    assert [v.value for v in vals] == [4096, 16, 16, 256]
    assert tl.sgemm_f32_timeline_layout(None, None, None, None) == HIP_ERROR_INVALID_VALUE
    assert tl.sgemm_f32_timeline_read(None, 4096 * 6 * 8 + 8, None, 0) == HIP_ERROR_INVALID_VALUE
    assert tl.sgemm_f32_timeline_clock_khz(None) == HIP_ERROR_INVALID_VALUE
    assert tl.sgemm_f32_timeline_read(None, 8, None, 0) == HIP_ERROR_INVALID_VALUE


def test_library_switch_routes_calls():
    """library() sends calls to the other build and restores the default."""
    from fp32_gemm_sgemm_amd import binding
    assert binding.load() is binding.load(sg.LIB_PATH)
    with sg.library(sg.POISON_LIB_PATH):
        assert binding.load() is binding.load(sg.POISON_LIB_PATH)
        assert sg.sgemm_f32_num_variants() == binding.load(sg.LIB_PATH).sgemm_f32_num_variants()
    assert binding.load() is binding.load(sg.LIB_PATH)


def test_scratch_size_matches_header(lib):
    """The binding's scratch size is the header's, and the no-allocation
    entry point is declared and exported."""
    m = re.search(r"#define\s+SGEMM_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m, "SGEMM_SCRATCH_BYTES not found"
    assert sg.SGEMM_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    assert "sgemm_f32_ex_noalloc" in declared_functions()


def test_noalloc_refuses_bad_arguments_before_any_hip_call(lib):
    """Invalid sizes or a forced variant out of range come back as errors from
    the host checks (no device is touched: none exists here)."""
    P = 1 << 20
    assert sg.sgemm_f32_ex_noalloc(0, 0, -1, 4, 4, 1.0, P, 4, 0, 2 * P, 4, 0, 0.0, 3 * P, 4, 0,
                                   1) == HIP_ERROR_INVALID_VALUE
    cfg = sg.SgemmCfg()
    cfg.id = sg.sgemm_f32_num_variants()
    assert sg.sgemm_f32_ex_noalloc(0, 0, 4, 4, 4, 1.0, P, 4, 0, 2 * P, 4, 0, 0.0, 3 * P, 4, 0,
                                   1, 0, cfg) == HIP_ERROR_INVALID_VALUE


@pytest.mark.parametrize("M,N,K,tb", [(4, 32, 4194204, 0), (3, 100, 3000000, 0),
                                     (4, 256, 1048576, 0), (4, 64, 2000000, 1)])
def test_few_strip_workgroups_take_a_split_when_a_workspace_fits(lib, M, N, K, tb):
    """A product of at most 4 rows whose strips would run on a handful of
    workgroups (each covers all of K) is split across workgroups instead when
    a workspace allows it.  Without one, the plan needs none: the strips, or
    16 x 16 or 8 x 8 tiles that split K inside the workgroup (NN: more
    workgroups than the strip; 16 x 16 ones were 20-38% faster on MI355X at
    these sizes)."""
    ldb = K if tb else N
    q = sg.sgemm_f32_plan(M, N, K, K, ldb, N, 256, 0, tb, 1, 1 << 30)
    assert q.grid > 0 and q.splits > 1 and q.grid >= 64, q.as_dict()
    q = sg.sgemm_f32_plan(M, N, K, K, ldb, N, 256, 0, tb, 1, 0)
    assert q.splits == 1 and q.workspace_bytes == 0, q.as_dict()
    strips = q.grid == 0 and q.strip_m == M
    assert strips or (q.bm in (8, 16) and q.strip_m == 0), q.as_dict()


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
        assert v.bm % 8 == 0 and v.bn % 8 == 0 and v.bk % 8 == 0
        # tiles under 32 x 32 are the 16 x 16 and 8 x 8 ones that split K
        assert v.bm % 32 == 0 or (v.bm, v.bn, v.bk) in ((16, 16, 16), (8, 8, 32))
    assert kinds == {sg.binding.SGEMM_KERNEL_MFMA, sg.binding.SGEMM_KERNEL_VALU}
    # cost-model figures: every variant reports a fixed cost (2.5 us or its
    # own); only the tiles that split K inside the workgroup (32 x 32 x 8,
    # 16 x 16 x 16, 8 x 8 x 32) price an L2 spill and overlap the fixed costs
    # of co-resident workgroups
    for i in range(n):
        v = sg.sgemm_f32_variant(i)
        assert 0 < v.fixed_ns < 20000 and v.coresident >= 1
        if (v.bm, v.bn, v.bk) in ((32, 32, 8), (16, 16, 16), (8, 8, 32)):
            assert v.spill_permille > 0 and v.spill_full_permille > 0
            # LDS bounds the workgroups that can share a CU
            assert v.coresident * v.lds_bytes <= 160 * 1024
        else:
            assert v.spill_permille == 0 and v.spill_full_permille == 0 and v.coresident == 1
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


def _ex(cfg, M=4, N=4, K=4, ta=0, tb=0, ws=0, ws_bytes=0):
    lda = (M if ta else K)
    ldb = (K if tb else N)
    return sg.sgemm_f32_ex(ta, tb, M, N, K, 1.0, P, lda, 0, 2 * P, ldb, 0, 0.0, 3 * P, N, 0, 1,
                           ws, ws_bytes, 0, cfg)


def test_ex_rejects_bad_forced_variant(lib):
    cfg = sg.binding.SgemmCfg()
    cfg.id = sg.sgemm_f32_num_variants()
    assert _ex(cfg) == HIP_ERROR_INVALID_VALUE
    cfg.id = 0
    cfg.group_m = -1  # negative group height
    assert _ex(cfg) == HIP_ERROR_INVALID_VALUE
    cfg.group_m = 8
    cfg.id = 2        # the vector-FMA comparison has no transposed-operand kernels
    assert sg.sgemm_f32_variant_ops(2) == 1
    assert _ex(cfg, ta=1) == HIP_ERROR_INVALID_VALUE
    cfg.id = 0
    cfg.splits = 4    # a split needs a workspace
    assert _ex(cfg, K=1024) == HIP_ERROR_INVALID_VALUE


def test_large_leading_dimensions_go_to_64_bit_kernels(lib):
    """Any leading dimension up to INT_MAX - 1024 is accepted.  Past the
    LDS-tiled kernels' 32-bit in-slice offsets (lda 2^22 - 64 for a
    k-contiguous A, ldb 2^25 - 512 for B) the plan keeps to the variants that
    address in 64 bits and the strip kernel; a forced tiled variant is
    refused."""
    lib_ = sg.load()
    ld64 = {i for i in range(sg.sgemm_f32_num_variants())
            if (sg.sgemm_f32_variant(i).bm, sg.sgemm_f32_variant(i).bk) in ((32, 8), (16, 16), (8, 32))}
    big = (1 << 31) - 1 - 1024
    cases = [(0, 0, 64, 64, 64, 1 << 23, 64), (0, 0, 64, 64, (1 << 22) + 64, (1 << 22) + 64, 64),
             (0, 0, 1, 1, (1 << 22) + 64, (1 << 22) + 64, 1), (0, 0, 300, 200, 8, 8, 1 << 25),
             (1, 0, 300, 200, 100, 1 << 26, 200), (0, 1, 300, 200, 100, 100, 1 << 23),
             (0, 0, 4000, 4000, 100, big, big)]
    for ta, tb, M, N, K, lda, ldb in cases:
        out = sg.binding.SgemmCfg()
        assert lib_.sgemm_f32_plan(ta, tb, M, N, K, lda, ldb, N, 1, 256, 0,
                                   ctypes.byref(out)) == 0, (ta, tb, M, N, K, lda, ldb)
        assert out.grid == 0 or out.id in ld64, (out.id, out.grid)
        for ws in (0, 1 << 30):
            q = sg.sgemm_f32_plan(M, N, K, lda, ldb, N, 256, ta, tb, 1, ws)
            assert q.grid == 0 or q.id in ld64
    # below the limits the tiled kernels stay available
    assert sg.sgemm_f32_plan(4096, 4096, 4096, (1 << 22) - 64, 4096, 4096, 256).id not in ld64
    # a forced tiled variant past its limit is refused; a 64-bit one is not
    cfg = sg.binding.SgemmCfg()
    cfg.id, cfg.group_m, cfg.xcd_remap = 4, 8, 1
    assert lib_.sgemm_f32_cfg_geometry(0, 0, 64, 64, 64, 1 << 23, 64, 64, 1,
                                       ctypes.byref(cfg)) == HIP_ERROR_INVALID_VALUE
    cfg.id = min(ld64)
    assert lib_.sgemm_f32_cfg_geometry(0, 0, 64, 64, 64, 1 << 23, 64, 64, 1,
                                       ctypes.byref(cfg)) == 0
    # past INT_MAX - 1024 still refused
    assert sg.sgemm_f32(4, 4, 4, P, (1 << 31) - 1, 2 * P, 4, 3 * P, 4, 0) == HIP_ERROR_INVALID_VALUE


def _gen(ta=0, tb=0, M=4, N=4, K=4, A=P, lda=None, sa=0, B=2 * P, ldb=None, sb=0,
         C=3 * P, ldc=None, sc=0, batch=1, ws=0, ws_bytes=0, alpha=1.0, beta=0.0):
    lda = max(M if ta else K, 1) if lda is None else lda
    ldb = max(K if tb else N, 1) if ldb is None else ldb
    ldc = max(N, 1) if ldc is None else ldc
    return sg.sgemm_f32_strided_batched(ta, tb, M, N, K, alpha, A, lda, sa, B, ldb, sb, beta,
                                        C, ldc, sc, batch, ws, ws_bytes, 0)


GEN_BAD = [
    dict(ta=2),                                  # not a layout
    dict(tb=-1),
    dict(ta=1, M=8, K=4, lda=7),                 # transposed A: lda >= M
    dict(tb=1, N=4, K=8, ldb=7),                 # transposed B: ldb >= K
    dict(batch=-1),
    dict(batch=2, sa=-4, sc=64),                 # negative stride
    dict(batch=2, sc=8),                         # C entries overlap (need 16)
    dict(batch=3, sc=16, C=2 * P + 64, sb=16),   # C's span overlaps B's span
    dict(ws=4 * P + 4, ws_bytes=1024),           # workspace not 16-byte aligned
    dict(ws=0, ws_bytes=0, C=0),                 # null C
    dict(ws=3 * P, ws_bytes=64),                 # workspace overlaps C
    dict(ws=P, ws_bytes=64),                     # workspace overlaps A
]


@pytest.mark.parametrize("args", GEN_BAD)
def test_general_invalid_arguments_rejected(lib, args):
    assert _gen(**args) == HIP_ERROR_INVALID_VALUE


def test_general_noops(lib):
    # batch 0, M 0 or N 0: nothing to do, pointers never looked at
    assert _gen(batch=0, A=0, B=0, C=0) == 0
    assert _gen(M=0, A=0, B=0, C=0) == 0
    # K == 0 (or alpha == 0) with beta == 1 leaves C as it is: no launch
    assert _gen(K=0, A=0, B=0, beta=1.0) == 0
    assert _gen(alpha=0.0, beta=1.0) == 0


def test_variant_layouts(lib):
    """Every variant has the plain layout; the direct-load tiles also carry
    the transposed ones (the 96-row wave tiles only a transposed B)."""
    n = sg.sgemm_f32_num_variants()
    masks = [sg.sgemm_f32_variant_ops(i) for i in range(n)]
    assert all(m & 1 for m in masks)
    assert sum(1 for m in masks if m == 0xF) >= 2
    assert sg.sgemm_f32_variant_ops(n) == -1
    for ta in (0, 1):
        for tb in (0, 1):
            p = sg.sgemm_f32_plan(1000, 900, 800, 1000 if ta else 800, 800 if tb else 900, 900,
                                  256, ta, tb)
            assert masks[p.id] & (1 << (ta + 2 * tb))


SHAPES = [(512, 512, 512), (2048, 2048, 2048), (3072, 3072, 3072), (8192, 8192, 4096),
          (4096, 4096, 8192), (4099, 4099, 4099), (8192, 8192, 8192), (1, 1, 1), (5, 3, 0),
          (513, 8192, 1023), (100, 70, 50)]


def _main_block(p, M, N):
    """Rows and columns of C left to the tiles once the plan's edge strips
    (at most 4 rows, 4 columns: the remainder past the last full tile row or
    column, or all of a dimension that small) are taken out."""
    assert 0 <= p.strip_m <= min(4, M) and 0 <= p.strip_n <= min(4, N)
    assert p.strip_m in (0, M % p.bm) and p.strip_n in (0, N % p.bn)
    return M - p.strip_m, N - p.strip_n


def _check_tiles(p, M, N, batch=1):
    Mm, Nn = _main_block(p, M, N)
    if Mm == 0 or Nn == 0:
        assert p.grid == 0 and p.splits == 1 and p.workspace_bytes == 0
        return Mm, Nn
    assert p.tiles_m == metrics.ceil_div(Mm, p.bm)
    assert p.tiles_n == metrics.ceil_div(Nn, p.bn)
    assert p.grid == p.tiles_m * p.tiles_n * p.splits * batch
    return Mm, Nn


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_plan_geometry(lib, M, N, K):
    for cus in (256, 80):
        for ws in (0, 1 << 40):
            p = sg.sgemm_f32_plan(M, N, K, max(K, 1), N, N, cus, workspace_bytes=ws)
            # matrix-core tiles, or the 8 x 8 vector-FMA tiles that split K
            assert p.kernel == sg.binding.SGEMM_KERNEL_MFMA or (p.bm, p.bn) == (8, 8)
            Mm, Nn = _check_tiles(p, M, N)
            assert p.threads == 64 * p.waves_m * p.waves_n
            assert p.group_m > 0 and p.xcd_remap == 1
            if ws == 0:
                assert p.splits == 1 and p.workspace_bytes == 0
            _check_split(p, Mm, Nn, K, 1)


def _check_split(p, M, N, K, batch):
    """A split's K ranges tile [0, K) in multiples of 64, and its workspace
    holds one partial result (rows padded to 4 floats) per split and entry."""
    assert p.splits >= 1
    if p.splits == 1:
        assert p.workspace_bytes == 0 and p.k_chunk >= max(K, 1)
        return
    assert p.k_chunk % 64 == 0
    assert (p.splits - 1) * p.k_chunk < K <= p.splits * p.k_chunk
    assert p.workspace_bytes == batch * p.splits * M * ((N + 3) // 4 * 4) * 4


def test_selector_prefers_full_waves(lib):
    """Wave quantisation on 256 CUs: 2048^3 has only 64 tiles of 256 x 256 but
    256 of 128 x 128; 3072^3 has 144 of 256 x 256, 576 of 128 x 128 and exactly
    256 of 192 x 192; 8192^3 fills the chip with the largest tile."""
    assert sg.sgemm_f32_plan(2048, 2048, 2048, 2048, 2048, 2048, 256).bm == 128
    p = sg.sgemm_f32_plan(3072, 3072, 3072, 3072, 3072, 3072, 256)
    assert p.grid == 256 and p.bm == 192          # one 192 x 192 tile per CU
    p = sg.sgemm_f32_plan(8192, 8192, 8192, 8192, 8192, 8192, 256)
    assert p.grid * p.bm * p.bn == 8192 * 8192


def test_selector_unaligned_rows(lib):
    """Rows that are not 16-byte aligned (ld = 4099) cannot take 16-byte
    direct loads: a 4-byte direct-load tile serves them.  At 4099^3 the
    tiles cover the 4096^2 block exactly (whole rounds), and the last 3 rows
    and 3 columns go to the strip kernel (no workspace needed), for every
    layout."""
    for ta in (0, 1):
        for tb in (0, 1):
            p = sg.sgemm_f32_plan(4099, 4099, 4099, 4099, 4099, 4099, 256, ta, tb, 1, 0)
            assert sg.sgemm_f32_variant(p.id).bm == p.bm and p.splits == 1
            assert (p.strip_m, p.strip_n) == (3, 3)
            assert p.grid * p.bm * p.bn == 4096 * 4096 and p.grid % 256 == 0
            assert sg.sgemm_f32_variant_ops(p.id) & (1 << (ta + 2 * tb))
    # without an edge a few rows wide there is no strip
    p = sg.sgemm_f32_plan(4000, 4000, 4000, 4001, 4001, 4000, 256)
    assert (p.strip_m, p.strip_n) == (0, 0)


def test_selector_strips(lib):
    """A few rows or columns past the last full tile go to the strip kernel
    when a tile row of them would cost a round; products with at most 4 rows
    or columns run on the strip kernel alone, or (without a workspace) on the
    16 x 16 or 8 x 8 tiles that split K inside the workgroup, which give such
    a product more workgroups than its strips (16 x 16: measured 0.6-1.1x the
    strip plans' time on MI355X)."""
    p = sg.sgemm_f32_plan(8196, 8192, 8192, 8192, 8192, 8192, 256)
    assert (p.strip_m, p.strip_n, p.bm, p.grid) == (4, 0, 256, 1024)
    p = sg.sgemm_f32_plan(2049, 2050, 2048, 2048, 2052, 2050, 256)
    assert (p.strip_m, p.strip_n) == (1, 2) and p.grid * p.bm * p.bn == 2048 * 2048
    for M, N in [(1, 4096), (4, 4096), (4096, 1), (4096, 3), (1, 1), (3, 2)]:
        for ta in (0, 1):
            for tb in (0, 1):
                p = sg.sgemm_f32_plan(M, N, 4096, M if ta else 4096, 4096 if tb else N, N, 256,
                                      ta, tb)
                strips = p.grid == 0 and (p.strip_m == M or p.strip_n == N)
                assert strips or (p.bm in (8, 16) and p.splits == 1), (M, N, p.as_dict())


def test_cfg_geometry_of_forced_strips(lib):
    cfg = sg.SgemmCfg()
    cfg.id, cfg.group_m, cfg.xcd_remap = 4, 8, 1
    for sm, sn in [(0, 0), (1, 0), (0, 4), (3, 3), (4, 4)]:
        cfg.strip_m, cfg.strip_n = sm, sn
        g = sg.sgemm_f32_cfg_geometry(cfg, 0, 0, 1000, 700, 300, 300, 700, 700)
        assert (g.strip_m, g.strip_n) == (sm, sn)
        assert g.tiles_m == metrics.ceil_div(1000 - sm, 256)
        assert g.tiles_n == metrics.ceil_div(700 - sn, 256)
    cfg.strip_m, cfg.strip_n = 3, 0
    g = sg.sgemm_f32_cfg_geometry(cfg, 0, 0, 3, 700, 300, 300, 700, 700)
    assert g.grid == 0 and g.splits == 1
    for sm, sn in [(5, 0), (0, 5), (-1, 0), (4, 0)]:
        cfg.strip_m, cfg.strip_n = sm, sn
        with pytest.raises(sg.SgemmError):
            sg.sgemm_f32_cfg_geometry(cfg, 0, 0, 3 if sm == 4 else 100, 700, 300, 300, 700, 700)


def test_selector_splits_k_for_few_tiles(lib):
    """With a workspace, a long-K product with few output tiles is split
    across workgroups (one 128 x 128 output is a single tile otherwise); a
    grid that already fills the chip is not."""
    p = sg.sgemm_f32_plan(128, 128, 32768, 32768, 128, 128, 256, workspace_bytes=1 << 30)
    assert p.splits >= 16
    _check_split(p, 128, 128, 32768, 1)
    p = sg.sgemm_f32_plan(8192, 8192, 8192, 8192, 8192, 8192, 256, workspace_bytes=1 << 40)
    assert p.splits == 1
    # the workspace limit is respected
    p = sg.sgemm_f32_plan(128, 128, 32768, 32768, 128, 128, 256, workspace_bytes=4 * 128 * 128 * 4)
    assert p.splits <= 4 and p.workspace_bytes <= 4 * 128 * 128 * 4
    # batches fill the chip by themselves
    p = sg.sgemm_f32_plan(128, 128, 4096, 4096, 128, 128, 256, batch=512,
                          workspace_bytes=1 << 40)
    assert p.splits == 1 and p.grid == 512


def test_selector_k_split_tiles_follow_the_l2(lib):
    """Without a workspace, an output of 256 32 x 32 tiles goes to the tiles
    that split K over their waves.  Once the operand rows and columns one XCD
    reads (8 tile rows and 4 tile columns: 384 rows of 4 K bytes) exceed the
    15/16 of its 4 MiB L2 that the model gives operands (K above 2560), the
    width picked slows no more from the spill than the one picked below that
    point."""
    spill = {}
    for i in range(sg.sgemm_f32_num_variants()):
        v = sg.sgemm_f32_variant(i)
        if (v.bm, v.bn, v.bk) == (32, 32, 8):
            spill[i] = v.spill_permille
    assert len(spill) >= 2
    ids = {}
    for K in (512, 2048, 8192, 16384):
        p = sg.sgemm_f32_plan(512, 512, K, K, 512, 512, 256)
        assert p.id in spill and p.splits == 1
        ids[K] = p.id
    assert max(spill[ids[8192]], spill[ids[16384]]) <= min(spill[ids[512]], spill[ids[2048]])


def test_deep_slice_variants_respect_their_stride_limit(lib):
    """Variants with 64-deep slices hold 64 rows of the index-contiguous
    operand per slice, so they serve its leading dimension only up to 2^23:
    the selector passes them over beyond that, and a forced one is refused."""
    deep = [i for i in range(sg.sgemm_f32_num_variants()) if sg.sgemm_f32_variant(i).bk == 64]
    assert deep
    big = (1 << 23) + 4
    for transb, ldb in [(0, big), (0, 1 << 23)]:
        p = sg.sgemm_f32_plan(1024, 1024, 4096, 4096, ldb, 1024, 256, transb=transb)
        if ldb > (1 << 23):
            assert p.id not in deep
        for vid in deep:
            cfg = sg.SgemmCfg()
            cfg.id, cfg.group_m, cfg.xcd_remap = vid, 8, 1
            r = lib.sgemm_f32_cfg_geometry(0, transb, 1024, 1024, 4096, 4096, ldb, 1024, 1,
                                           ctypes.byref(cfg))
            assert (r == HIP_ERROR_INVALID_VALUE) == (ldb > (1 << 23))
    # a transposed A is index-contiguous too
    cfg = sg.SgemmCfg()
    cfg.id, cfg.group_m, cfg.xcd_remap = deep[0], 8, 1
    assert lib.sgemm_f32_cfg_geometry(1, 0, 64, 64, 64, big, 64, 64, 1,
                                      ctypes.byref(cfg)) == HIP_ERROR_INVALID_VALUE


def test_cfg_geometry_of_forced_splits(lib):
    for want, K in [(2, 1000), (3, 1000), (7, 4099), (64, 32768), (100, 32768), (8, 64), (4, 65)]:
        cfg = sg.SgemmCfg()
        cfg.id, cfg.splits, cfg.group_m, cfg.xcd_remap = 1, want, 8, 1
        g = sg.sgemm_f32_cfg_geometry(cfg, 0, 0, 300, 200, K, K, 200, 200, 3)
        assert g.id == 1 and g.group_m == 8 and g.xcd_remap == 1
        assert g.splits <= max(min(want, 64), 1)
        _check_split(g, 300, 200, K, 3)
        assert g.grid == g.tiles_m * g.tiles_n * g.splits * 3


def test_plan_rejects_invalid(lib):
    out = sg.binding.SgemmCfg()
    plan = lib.sgemm_f32_plan
    assert plan(0, 0, -1, 4, 4, 4, 4, 4, 1, 256, 0, ctypes.byref(out)) == HIP_ERROR_INVALID_VALUE
    assert plan(0, 0, 4, 4, 8, 4, 4, 4, 1, 256, 0, ctypes.byref(out)) == HIP_ERROR_INVALID_VALUE
    assert plan(0, 0, 4, 4, 4, 4, 4, 4, 1, 256, 0, None) == HIP_ERROR_INVALID_VALUE
    assert plan(3, 0, 4, 4, 4, 4, 4, 4, 1, 256, 0, ctypes.byref(out)) == HIP_ERROR_INVALID_VALUE
    assert plan(0, 0, 4, 4, 4, 4, 4, 4, -1, 256, 0, ctypes.byref(out)) == HIP_ERROR_INVALID_VALUE


def test_plan_invariants_random(lib):
    """Seeded random problems: every plan serves the layout, its grid covers
    tiles x splits x batch, its K ranges tile [0, K) in multiples of 64, its
    workspace is what the split needs and never more than offered, and a
    forced configuration completed by sgemm_f32_cfg_geometry agrees with the
    selector's own choice."""
    import numpy as np
    rng = np.random.default_rng(2024)
    for _ in range(400):
        M, N, K = (int(x) for x in rng.integers(1, 9000, size=3))
        if rng.random() < 0.3:
            M, N = (int(x) for x in rng.integers(1, 300, size=2))
        ta, tb = (int(x) for x in rng.integers(0, 2, size=2))
        batch = int(rng.choice([1, 1, 1, 2, 7, 64]))
        lda = (M if ta else K) + int(rng.integers(0, 5))
        ldb = (K if tb else N) + int(rng.integers(0, 5))
        ldc = N + int(rng.integers(0, 5))
        ws = int(rng.choice([0, 1 << 20, 1 << 26, 1 << 40]))
        cus = int(rng.choice([256, 304, 80]))
        p = sg.sgemm_f32_plan(M, N, K, lda, ldb, ldc, cus, ta, tb, batch, ws)
        assert sg.sgemm_f32_variant_ops(p.id) & (1 << (ta + 2 * tb))
        Mm, Nn = _check_tiles(p, M, N, batch)
        assert p.workspace_bytes <= ws
        _check_split(p, Mm, Nn, K, batch)
        cfg = sg.SgemmCfg()
        cfg.id, cfg.splits, cfg.group_m, cfg.xcd_remap = p.id, p.splits, p.group_m, p.xcd_remap
        cfg.strip_m, cfg.strip_n = p.strip_m, p.strip_n
        g = sg.sgemm_f32_cfg_geometry(cfg, ta, tb, M, N, K, lda, ldb, ldc, batch)
        assert (g.splits, g.k_chunk, g.grid, g.workspace_bytes) == \
            (p.splits, p.k_chunk, p.grid, p.workspace_bytes)


def test_plan_cache_returns_each_problems_own_plan(lib):
    """The library remembers recent plans per thread; cycling through more
    distinct problems than it keeps, with the same sizes under different
    layouts, workspaces and CU counts, every answer equals a cold one."""
    import itertools
    probs = []
    for (M, N, K), (ta, tb), ws, cus in itertools.product(
            [(512, 512, 512), (4099, 4099, 4099), (128, 128, 32768), (3, 700, 900)],
            [(0, 0), (1, 1)], [0, 1 << 40], [256, 80]):
        probs.append((M, N, K, ta, tb, ws, cus))
    def plan(M, N, K, ta, tb, ws, cus):
        p = sg.sgemm_f32_plan(M, N, K, M if ta else K, K if tb else N, N, cus, ta, tb, 1, ws)
        return (p.id, p.splits, p.strip_m, p.strip_n, p.grid, p.workspace_bytes)
    first = [plan(*q) for q in probs]
    for _ in range(3):
        for q, want in zip(probs, first):
            assert plan(*q) == want, q
    for q, want in zip(reversed(probs), reversed(first)):
        assert plan(*q) == want, q
