"""Parity of the HIP path with the CPU reference, through the C ABI.

Bound (for every checked element): |C - ref| <= 1e-4 * sum_k |a_ik * b_kj|,
C finite.  Full comparison up to 1024^3; above that the seeded 4096-position
sample (uniform positions plus the edge band), and for 4099^3 also every
element of the last 3 rows and columns.  Integer-exact cases (identity,
permutations, small integers, all-ones, K = 1) must match bit for bit.

The five measured workloads run through the default selector, i.e. in the
launch configuration the benchmark times.
"""
import numpy as np
import pytest

import oracle
import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import inputs

from gpu_cases import check_full, check_sampled, forced, note, run, to_device

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

W = inputs.WORKLOADS


def _workload(name, last=0):
    w = W[name]
    note(f"{name}: M={w.M} N={w.N} K={w.K} seed={w.seed} dist={w.dist} variant={w.variant}")
    A, B = inputs.workload_operands(w)
    C = run(A, B)
    if w.variant == "identity":
        assert np.array_equal(C, B), "A = I must reproduce B exactly"
        return
    if w.check == "full":
        check_full(C, A, B)
    else:
        check_sampled(C, A, B, w.seed, last=last)


# ---- the measured workloads ----------------------------------------------------------

def test_512_uniform_full():
    _workload("sgemm_512x512x512_uniform_seed0")


def test_2048_uniform_sampled():
    _workload("sgemm_2048x2048x2048_uniform_seed1")


def test_2048_identity_exact():
    _workload("sgemm_2048x2048x2048_identityA_seed1")


def test_3072_normal_sampled():
    _workload("sgemm_3072x3072x3072_normal_seed2")


def test_8192x8192x4096_sampled():
    _workload("sgemm_8192x8192x4096_uniform_seed3")


def test_4096x4096x8192_sampled():
    _workload("sgemm_4096x4096x8192_uniform_seed3")


def test_4099_ragged_sampled_and_last_rows_cols():
    _workload("sgemm_4099x4099x4099_uniform_seed3", last=3)


def test_8192_uniform_sampled():
    _workload("sgemm_8192x8192x8192_uniform_seed4")


def test_1024_uniform_full():
    _workload("sgemm_1024x1024x1024_uniform_seed5")


def test_workbook_lab_shapes():
    _workload("sgemm_100x70x50_uniform_seed7")
    _workload("sgemm_513x8192x1023_uniform_seed6")
    note("64x64x64")
    A, B = inputs.make_operands(64, 64, 64, seed=8)
    check_full(run(A, B), A, B)


# ---- edges ---------------------------------------------------------------------------

EDGE_SIZES = [1, 2, 3, 15, 16, 17, 31, 33, 63, 65, 127, 129, 255, 257]


def _edge_shapes():
    rng = np.random.default_rng(2024)
    shapes = [(s, s, s) for s in EDGE_SIZES]
    for _ in range(30):
        shapes.append(tuple(int(x) for x in rng.choice(EDGE_SIZES, size=3)))
    return shapes


@pytest.mark.parametrize("M,N,K", _edge_shapes())
def test_edge_sweep(M, N, K):
    note(f"edge M={M} N={N} K={K}")
    A, B = inputs.make_operands(M, N, K, seed=M * 7 + N * 11 + K * 13)
    check_full(run(A, B), A, B)


def _padded(x, ld, fill=np.nan):
    """x (rows x cols) stored with row stride ld; the padding holds `fill`."""
    rows, cols = x.shape
    buf = np.full((rows, ld), fill, dtype=np.float32)
    buf[:, :cols] = x
    return buf


@pytest.mark.parametrize("M,N,K,pad", [(300, 260, 200, 4), (257, 129, 65, 3), (64, 1000, 33, 1)])
def test_leading_dimensions_and_untouched_padding(M, N, K, pad):
    note(f"leading dims M={M} N={N} K={K} pad={pad}")
    A, B = inputs.make_operands(M, N, K, seed=31)
    Ad = to_device(_padded(A, K + pad))[:, :K]
    Bd = to_device(_padded(B, N + pad))[:, :N]
    Cbuf = to_device(_padded(np.zeros((M, N), np.float32), N + pad, fill=np.nan))
    Cbuf[:, :N] = float("nan")
    out = Cbuf[:, :N]
    sg.sgemm(Ad, Bd, out=out)
    torch.cuda.synchronize()
    full = Cbuf.cpu().numpy()
    assert np.all(np.isnan(full[:, N:])), "padding columns of C were written"
    check_full(full[:, :N], A, B)


@pytest.mark.parametrize("M,N,K", [(200, 300, 100), (129, 257, 4099)])
def test_misaligned_base_pointers(M, N, K):
    """Operands starting one float past a 16-byte boundary (16-byte loads and
    stores at dword alignment)."""
    note(f"misaligned pointers M={M} N={N} K={K}")
    A, B = inputs.make_operands(M, N, K, seed=32)

    def shifted(x):
        flat = torch.empty(x.size + 1, dtype=torch.float32, device="cuda")
        v = flat[1:].view(x.shape)
        v.copy_(torch.from_numpy(x))
        return v

    Ad, Bd = shifted(A), shifted(B)
    Cd = torch.empty(M * N + 1, dtype=torch.float32, device="cuda")[1:].view(M, N)
    assert Ad.data_ptr() % 16 != 0 and Cd.data_ptr() % 16 != 0
    sg.sgemm(Ad, Bd, out=Cd)
    torch.cuda.synchronize()
    check_full(Cd.cpu().numpy(), A, B)


def test_nan_prefilled_c_is_overwritten():
    note("NaN-prefilled C 333x444x555")
    A, B = inputs.make_operands(333, 444, 555, seed=33)
    out = torch.full((333, 444), float("nan"), device="cuda")
    C = run(A, B, out=out)
    assert np.all(np.isfinite(C))
    check_full(C, A, B)


def test_k_zero_gives_zeros():
    note("K=0")
    out = torch.full((70, 90), float("nan"), device="cuda")
    A = torch.empty((70, 0), device="cuda")
    B = torch.empty((0, 90), device="cuda")
    sg.sgemm(A, B, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item()


def test_empty_output_leaves_memory_alone():
    note("M=0 / N=0")
    A = torch.ones((0, 16), device="cuda")
    B = torch.ones((16, 8), device="cuda")
    assert sg.sgemm(A, B).shape == (0, 8)
    sentinel = torch.full((4, 4), 7.0, device="cuda")
    assert sg.sgemm_f32(4, 0, 16, A.data_ptr(), 16, B.data_ptr(), 8, sentinel.data_ptr(), 4, 0) == 0
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0).item()


# ---- exact cases ---------------------------------------------------------------------

def test_small_integers_bit_exact_2048():
    """Integer inputs in [-2, 2]: every partial sum is an integer below 2^24, so
    any summation order is exact and C must equal the reference bit for bit."""
    note("small integers 2048^3")
    rng = np.random.default_rng(41)
    A = inputs.small_integers(rng, (2048, 2048))
    B = inputs.small_integers(rng, (2048, 2048))
    C = run(A, B)
    rows, cols = inputs.sample_indices(2048, 2048, seed=41)
    ref, _ = oracle.sgemm_ref_sampled(A, B, rows, cols)
    assert np.array_equal(C[rows, cols].astype(np.float64), ref)
    ref_full, _ = oracle.sgemm_ref(A[:64], B)          # first 64 rows in full
    assert np.array_equal(C[:64].astype(np.float64), ref_full)


def test_all_ones_gives_k():
    note("all ones 300x260x4099")
    C = run(inputs.ones((300, 4099)), inputs.ones((4099, 260)))
    assert np.all(C == 4099.0)


def test_k1_outer_product_bit_exact():
    note("K=1 outer product 513x1025")
    A, B = inputs.make_operands(513, 1025, 1, seed=42)
    C = run(A, B)
    assert np.array_equal(C, (A * B).astype(np.float32))   # one rounding per product


def test_permutation_exact():
    note("row permutation 1000x700")
    _, B = inputs.make_operands(1000, 700, 1000, seed=43)
    P, perm = inputs.permutation(1000, seed=44)
    assert np.array_equal(run(P, B), B[perm])


def test_deterministic_repeats():
    note("determinism 2048x1536x1000")
    A, B = inputs.make_operands(2048, 1536, 1000, seed=45)
    Ad, Bd = to_device(A), to_device(B)
    c1 = sg.sgemm(Ad, Bd)
    c2 = sg.sgemm(Ad, Bd)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


# ---- every compiled variant and tile order ---------------------------------------------

def _variants():
    return list(range(sg.sgemm_f32_num_variants()))


@pytest.mark.parametrize("vid", _variants())
def test_every_variant(vid):
    v = sg.sgemm_f32_variant(vid)
    for (M, N, K) in [(300, 200, 100), (512, 384, 200), (1, 1, 9)]:
        note(f"variant {vid} ({v.bm}x{v.bn}x{v.bk} w{v.waves_m}x{v.waves_n} "
             f"kernel={v.kernel}) M={M} N={N} K={K}")
        A, B = inputs.make_operands(M, N, K, seed=vid * 17 + K)
        check_full(run(A, B, cfg=forced(vid)), A, B)


@pytest.mark.parametrize("group_m", [0, 1, 3, 8, 64])
@pytest.mark.parametrize("xcd", [0, 1])
def test_tile_orders_cover_every_tile(group_m, xcd):
    """Tile counts not divisible by 8 or by the group height: any gap in the
    workgroup-to-tile mapping leaves NaN behind."""
    M, N, K = 1100, 1300, 40
    A, B = inputs.make_operands(M, N, K, seed=46)
    for vid in sorted({sg.sgemm_f32_plan(M, N, K, K, N, N, 256).id,
                       sg.sgemm_f32_plan(8192, 8192, 8192, 8192, 8192, 8192, 256).id}):
        note(f"tile order group_m={group_m} xcd={xcd} variant {vid}")
        out = torch.full((M, N), float("nan"), device="cuda")
        C = run(A, B, cfg=forced(vid, group_m, xcd), out=out)
        check_full(C, A, B)


@pytest.mark.parametrize("M,N,K,shift", [(520, 700, 300, 0), (517, 701, 303, 0),
                                          (300, 260, 200, 1), (257, 513, 4099, 1)])
def test_direct_load_kernels_on_every_fetch_path(M, N, K, shift):
    """Forced direct-load variants: 16-byte aligned operands with K and N
    multiples of 4 (direct path, zero chunks past the edge), K or N not a
    multiple of 4 (partial-chunk slices fetched through registers), and
    operands one float off 16-byte alignment (register fetch for every
    slice)."""
    A, B = inputs.make_operands(M, N, K, seed=49 + K)

    def place(x):
        if not shift:
            return to_device(x)
        flat = torch.empty(x.size + shift, dtype=torch.float32, device="cuda")
        v = flat[shift:].view(x.shape)
        v.copy_(torch.from_numpy(x))
        return v

    for vid in range(sg.sgemm_f32_num_variants()):
        v = sg.sgemm_f32_variant(vid)
        if v.kernel != sg.SGEMM_KERNEL_MFMA and (v.bm, v.bn) != (8, 8):
            continue  # the vector-FMA comparison kernel
        note(f"fetch paths variant {vid} M={M} N={N} K={K} shift={shift}")
        Ad, Bd = place(A), place(B)
        out = torch.full((M, N), float("nan"), device="cuda")
        sg.sgemm(Ad, Bd, out=out, cfg=forced(vid))
        torch.cuda.synchronize()
        check_full(out.cpu().numpy(), A, B)


def test_long_k_single_tile():
    """128 x 128 x 32768: the one-tile, long-K shape of the cuda-kernels README."""
    note("128x128x32768")
    A, B = inputs.make_operands(128, 128, 32768, seed=47)
    check_full(run(A, B), A, B)


def test_query_and_nondefault_stream():
    note("query + side stream 640x480x320")
    A, B = inputs.make_operands(640, 480, 320, seed=48)
    Ad, Bd = to_device(A), to_device(B)
    Cd = torch.empty((640, 480), device="cuda")
    q = sg.sgemm_f32_query(0, 0, 640, 480, 320, Ad.data_ptr(), 320, 0, Bd.data_ptr(), 480, 0,
                           Cd.data_ptr(), 480, 0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = sg.sgemm_f32_plan(640, 480, 320, 320, 480, 480, cus)
    assert (q.id, q.grid, q.group_m, q.xcd_remap, q.splits) == (p.id, p.grid, p.group_m, p.xcd_remap, 1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sg.sgemm(Ad, Bd, out=Cd, stream=s)
    s.synchronize()
    check_full(Cd.cpu().numpy(), A, B)
