"""GPU parity of the edge strips: the last few rows and columns of C computed
by the strip kernel while the tiles compute the block above and left of them,
and products of at most 4 rows or columns computed by the strip kernel alone.
Every result is compared element by element with the CPU reference's general
form on seeded inputs; exact cases compare bit for bit."""
import numpy as np
import pytest

import oracle
import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import inputs
from gpu_cases import check_general, forced, note, place, run_general, stored

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

LAYOUTS = [(0, 0), (1, 0), (0, 1), (1, 1)]


def with_strips(vid, sm, sn, splits=1):
    cfg = forced(vid)
    cfg.strip_m, cfg.strip_n, cfg.splits = sm, sn, splits
    return cfg


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_forced_strips_every_layout(ta, tb):
    """Forced strips of 1-4 rows and columns beside tiles of two families,
    on a shape with ragged tiles and K past one staged chunk of the small
    operand (4608) and not a multiple of 4, with padded strides and an
    unaligned start."""
    M, N, K = 517, 389, 4621
    A, B = inputs.make_operands(M, N, K, seed=300 + ta + 2 * tb)
    As, Bs = stored(A, ta), stored(B, tb)
    ref, absb = oracle.gemm_ref(As, Bs, ta, tb)
    for vid in (4, 11):
        for sm, sn in [(1, 0), (0, 3), (4, 4), (3, 1), (2, 2)]:
            for pad, shift in [((0, 0, 0), (0, 0, 0)), ((3, 1, 5), (1, 1, 1))]:
                note(f"strips ta={ta} tb={tb} variant {vid} sm={sm} sn={sn} pad={pad}")
                C = run_general(As, Bs, ta, tb, cfg=with_strips(vid, sm, sn), pad=pad,
                                shift=shift)
                rep = oracle.compare(C, ref, absb)
                assert rep["n_bad"] == 0, rep


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 1000, 4100), (3, 777, 9301), (4, 64, 4100),
                                   (1000, 1, 4100), (700, 3, 9301), (2, 2, 4100), (1, 1, 1),
                                   (4, 33, 4608)])
def test_strip_only_products(ta, tb, M, N, K):
    """Products with at most 4 rows or columns on the strip kernel alone (a
    forced strip-only plan), and through the default selector, which runs
    them on the strips or, without a workspace, on the 16 x 16 or 8 x 8
    tiles that split K inside the workgroup; K within one staged chunk of the small operand,
    exactly one, and past two."""
    A, B = inputs.make_operands(M, N, K, seed=310 + M + N)
    As, Bs = stored(A, ta), stored(B, tb)
    note(f"strip-only ta={ta} tb={tb} {M}x{N}x{K}")
    C = run_general(As, Bs, ta, tb, cfg=with_strips(4, M, 0) if M <= 4 else with_strips(4, 0, N))
    check_general(C, As, Bs, ta, tb)
    note(f"default plan ta={ta} tb={tb} {M}x{N}x{K}")
    C = run_general(As, Bs, ta, tb, workspace=False)
    check_general(C, As, Bs, ta, tb)
    if K >= 4096:
        q = sg.sgemm_f32_plan(M, N, K, M if ta else K, K if tb else N, N, 256, ta, tb)
        strips = q.grid == 0 and (q.strip_m == M or q.strip_n == N)
        assert strips or (q.bm in (8, 16) and q.splits == 1), q.as_dict()


@pytest.mark.parametrize("alpha,beta", [(1.5, -0.75), (-2.0, 0.0), (0.25, 2.0)])
def test_strips_alpha_beta(alpha, beta):
    M, N, K = 260, 259, 300
    A, B = inputs.make_operands(M, N, K, seed=320)
    C0 = inputs.make_operands(M, N, 1, seed=321)[0] @ np.ones((1, N), np.float32)
    C0 = np.ascontiguousarray(C0, dtype=np.float32)
    for ta, tb in LAYOUTS:
        As, Bs = stored(A, ta), stored(B, tb)
        note(f"strips alpha={alpha} beta={beta} ta={ta} tb={tb}")
        C = run_general(As, Bs, ta, tb, alpha, beta, C0.copy(), cfg=with_strips(4, 4, 3))
        check_general(C, As, Bs, ta, tb, alpha, beta, C0)


def test_strips_with_split_tiles():
    """The tiled block split along K (workspace) beside strips."""
    M, N, K = 131, 130, 6000
    A, B = inputs.make_operands(M, N, K, seed=330)
    for ta, tb in LAYOUTS:
        As, Bs = stored(A, ta), stored(B, tb)
        note(f"strips + split ta={ta} tb={tb}")
        C = run_general(As, Bs, ta, tb, cfg=with_strips(11, 3, 2, splits=4))
        check_general(C, As, Bs, ta, tb)


def test_strips_exact_and_deterministic():
    """Small integers: every partial sum is an exact integer in fp32, so the
    strips must give the integer product bit for bit; and two runs agree."""
    M, N, K = 1027, 1026, 3001
    rng = np.random.default_rng(340)
    A = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    B = rng.integers(-2, 3, size=(K, N)).astype(np.float32)
    # the reference's float64 sums of integers below 2^53 are the exact
    # integer product
    ref, _ = oracle.sgemm_ref(A, B)
    assert np.array_equal(ref, np.round(ref))
    want = ref.astype(np.float32)
    note("strips exact integers")
    cfg = with_strips(4, 3, 2)
    C1 = run_general(A, B, 0, 0, cfg=cfg)
    C2 = run_general(A, B, 0, 0, cfg=cfg)
    assert np.array_equal(C1, want)
    assert np.array_equal(C1, C2)
    # random values: reproducible bit for bit
    A, B = inputs.make_operands(M, N, K, seed=341)
    C1 = run_general(A, B, 0, 0, cfg=cfg)
    C2 = run_general(A, B, 0, 0, cfg=cfg)
    assert np.array_equal(C1, C2)
    check_general(C1, A, B, 0, 0)


def test_strips_batched():
    """Strided batches through the strip kernel: gaps between entries, a
    broadcast B, and a padded C whose padding stays untouched (NaN)."""
    batch, M, N, K = 5, 259, 131, 700
    rng = np.random.default_rng(350)
    for ta, tb in LAYOUTS:
        A = rng.uniform(-1, 1, size=(batch, M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, size=(1, K, N)).astype(np.float32)
        As = np.ascontiguousarray(np.swapaxes(A, 1, 2)) if ta else A
        Bs = np.ascontiguousarray(np.swapaxes(B, 1, 2)) if tb else B
        Ad = torch.zeros((batch, As.shape[1], As.shape[2] + 4), device="cuda")[:, :, :As.shape[2]]
        Ad.copy_(torch.from_numpy(As))
        Bd = torch.from_numpy(Bs).to("cuda")
        Cd = torch.full((batch, M, N + 3), float("nan"), device="cuda")
        out = Cd[:, :, :N]
        cfg = with_strips(11, 3, 3)
        note(f"strips batched ta={ta} tb={tb}")
        sg.sgemm_batched(Ad, Bd, out=out, transa=bool(ta), transb=bool(tb), cfg=cfg)
        torch.cuda.synchronize()
        C = Cd.cpu().numpy()
        assert np.isnan(C[:, :, N:]).all()
        ref, absb = oracle.gemm_ref_batched(As, Bs, ta, tb, 1.0, 0.0, None)
        rep = oracle.compare(C[:, :, :N], ref, absb)
        assert rep["n_bad"] == 0, rep


def test_ragged_4099_plan_full_rows():
    """4099^3 through sgemm_f32 (rows not 16-byte aligned): the selector's
    tiles on the 4096^2 block plus 3-wide strips; every element of the last 3 rows and
    columns and a seeded sample inside are checked."""
    n = 4099
    A, B = inputs.make_operands(n, n, n, seed=3)
    note("4099^3 default plan")
    Ad, Bd = place(A), place(B)
    Cd = torch.empty((n, n), dtype=torch.float32, device="cuda")
    q = sg.sgemm_f32_query(0, 0, n, n, n, Ad.data_ptr(), n, 0, Bd.data_ptr(), n, 0,
                           Cd.data_ptr(), n, 0)
    assert (q.strip_m, q.strip_n) == (3, 3) and q.grid * q.bm * q.bn == 4096 * 4096
    assert sg.sgemm_f32(n, n, n, Ad.data_ptr(), n, Bd.data_ptr(), n, Cd.data_ptr(), n,
                        torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    C = Cd.cpu().numpy()
    rows, cols = inputs.sample_indices(n, n, 103, last=3)
    ref, absb = oracle.sgemm_ref_sampled(A, B, rows, cols)
    rep = oracle.compare(C[rows, cols], ref, absb)
    assert rep["n_bad"] == 0, rep


def test_strip_only_batches_past_one_launch():
    """70,000 strip-only products (the strip grid's second dimension holds
    65,535 entries per launch): every entry checked."""
    batch, M, N, K = 70000, 2, 3, 37
    rng = np.random.default_rng(360)
    A = rng.uniform(-1, 1, size=(batch, M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, size=(batch, K, N)).astype(np.float32)
    note("strip-only batch 70000")
    q = sg.sgemm_f32_plan(M, N, K, K, N, N, 256, 0, 0, batch)
    assert q.grid == 0
    C = sg.sgemm_batched(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda())
    torch.cuda.synchronize()
    C = C.cpu().numpy()
    # every entry through the CPU reference (one thread per small product)
    ref, absb = oracle.gemm_ref_batched(A, B, nthreads=1)
    rep = oracle.compare(C, ref, absb)
    assert rep["n_bad"] == 0, rep


@pytest.mark.parametrize("vid", [14, 15, 16, 22, 23, 24])
def test_ksplit_tiles_with_outer_splits_batches_and_strips(vid):
    """The 32x32, 16x16 and 8x8 tiles that split K inside the workgroup, combined with a split
    across workgroups (workspace), batches with a broadcast operand, strips
    and alpha/beta, in every layout."""
    batch, M, N, K = 3, 67, 98, 1500
    rng = np.random.default_rng(370 + vid)
    for ta, tb in LAYOUTS:
        A = rng.uniform(-1, 1, size=(batch, M, K)).astype(np.float32)
        B = rng.uniform(-1, 1, size=(1, K, N)).astype(np.float32)
        C0 = rng.uniform(-1, 1, size=(batch, M, N)).astype(np.float32)
        As = np.ascontiguousarray(np.swapaxes(A, 1, 2)) if ta else A
        Bs = np.ascontiguousarray(np.swapaxes(B, 1, 2)) if tb else B
        cfg = with_strips(vid, 3, 2, splits=3)
        note(f"k-split tiles variant {vid} ta={ta} tb={tb} + split 3 + strips + batch")
        Cd = torch.from_numpy(C0.copy()).cuda()
        sg.sgemm_batched(torch.from_numpy(As).cuda(), torch.from_numpy(Bs).cuda(), out=Cd,
                         transa=bool(ta), transb=bool(tb), alpha=-0.5, beta=1.25, cfg=cfg)
        torch.cuda.synchronize()
        ref, absb = oracle.gemm_ref_batched(As, Bs, ta, tb, -0.5, 1.25, C0)
        rep = oracle.compare(Cd.cpu().numpy(), ref, absb)
        assert rep["n_bad"] == 0, rep


@pytest.mark.parametrize("ta,tb,M,N,K", [(0, 1, 4, 8192, 1000), (1, 1, 4, 8192, 1000),
                                         (0, 1, 8192, 3, 1000), (0, 0, 8192, 3, 1001)])
def test_wide_kc_strips_in_the_32_row_form(ta, tb, M, N, K):
    """Strip-only products whose k-contiguous strip has 256 workgroups of 32
    rows (as many as the CUs, so the launch keeps the 32-row form rather
    than the 16-row one it takes for fewer): the row strip with B
    transposed (NT, TT) and the column strip with A as stored (NT, NN)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    x = N if M <= 4 else M
    if -(-x // 32) < cus:
        pytest.skip(f"{cus} CUs: this strip would take the 16-row form")
    As, Bs = inputs.make_operands(M, N, K, seed=380 + M + ta + 2 * tb)
    As, Bs = stored(As, ta), stored(Bs, tb)
    # the strips forced to be the whole product
    cfg = with_strips(4, M, 0) if M <= 4 else with_strips(4, 0, N)
    q = sg.sgemm_f32_cfg_geometry(cfg, ta, tb, M, N, K, As.shape[1], Bs.shape[1], N)
    assert q.grid == 0, q.as_dict()
    note(f"wide KC strip ta={ta} tb={tb} {M}x{N}x{K}")
    C1 = run_general(As, Bs, ta, tb, cfg=cfg, workspace=False)
    C2 = run_general(As, Bs, ta, tb, cfg=cfg, workspace=False)
    assert np.array_equal(C1, C2)
    check_general(C1, As, Bs, ta, tb)
