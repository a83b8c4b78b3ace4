"""GPU parity at the size limits: operands and results of more than 2^31
elements (64-bit element offsets in every kernel family, the tile mapping
and the batch strides), and leading dimensions at the largest value the
library accepts and past the range of direct global -> LDS loads (where the
direct-load kernels fetch every slice through registers).

The large operands hold small integers drawn on the device by a seeded
generator, so every product is an exact integer below 2^24 and the check is
bit-exact in any summation order.  Only the sampled rows of op(A) and
columns of op(B) go back to the host, where the CPU reference forms their
full product; C is compared on that grid of rows and columns, which always
includes the first and the last ones.
"""
import numpy as np
import pytest

import oracle
import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import inputs
from gpu_cases import check_general, forced, note, place, stored

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

LAYOUTS = [(0, 0), (1, 0), (0, 1), (1, 1)]

# Leading-dimension limits (floats) declared with the C ABI: an operand whose
# contiguous index is k (A, or a transposed B) takes up to 2^22 - 64, one whose
# contiguous index is a row or column of C (B, or a transposed A) up to
# 2^25 - 512.  Direct global -> LDS loads take up to 2^20 and 2^24.
MAX_LD_K = (1 << 22) - 64
MAX_LD_X = (1 << 25) - 512
DIRECT_LD_K = 1 << 20
DIRECT_LD_X = 1 << 24
DEEP_LD_X = 1 << 23       # index-contiguous stride limit of the 64-deep-slice variants


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _op_rows(A, ta, rows):
    """Rows `rows` of op(A) on the host (A stored M x K, or K x M with ta)."""
    idx = torch.as_tensor(rows, device=A.device)
    sub = A[:, idx].t() if ta else A[idx, :]
    return np.ascontiguousarray(sub.cpu().numpy())


def _op_cols(B, tb, cols):
    """Columns `cols` of op(B) on the host (B stored K x N, or N x K with tb)."""
    idx = torch.as_tensor(cols, device=B.device)
    sub = B[idx, :].t() if tb else B[:, idx]
    return np.ascontiguousarray(sub.cpu().numpy())


def _check_grid(C, A, B, ta, tb, seed, alpha=1.0, beta=0.0, C0_grid=None):
    M, N = C.shape
    rows = inputs.grid_sample(M, seed)
    cols = inputs.grid_sample(N, seed + 1)
    a = _op_rows(A, ta, rows)
    b = _op_cols(B, tb, cols)
    ref, absb = oracle.gemm_ref(a, b, False, False, alpha, beta, C0_grid)
    ri = torch.as_tensor(rows, device=C.device)
    ci = torch.as_tensor(cols, device=C.device)
    got = C[ri][:, ci].cpu().numpy()
    rep = oracle.compare(got, ref, absb)
    assert rep["n_bad"] == 0, rep
    # exact integers: the result must be the reference itself
    assert np.array_equal(got.astype(np.float64), ref), rep
    return rep


@pytest.mark.parametrize("case", [
    # name,                ta, tb,     M,     N,     K
    ("C past 2^31 elements", 0, 0, 66000, 32800, 40),
    ("A past 2^31 elements", 0, 0, 33000, 96, 66000),
    ("B past 2^31 elements", 0, 0, 96, 33000, 66000),
    ("stored A^T past 2^31", 1, 0, 33000, 96, 66000),
    ("stored B^T past 2^31", 0, 1, 96, 33000, 66000),
], ids=lambda c: c[0].replace(" ", "_").replace("^", ""))
def test_operands_beyond_2_31_elements(case):
    name, ta, tb, M, N, K = case
    note(f"large: {name} ta={ta} tb={tb} {M}x{N}x{K}")
    seed = M + N + K
    A = inputs.small_integers_device((K, M) if ta else (M, K), seed)
    B = inputs.small_integers_device((N, K) if tb else (K, N), seed + 1)
    C = torch.full((M, N), float("nan"), device="cuda")
    sg.sgemm(A, B, out=C, transa=bool(ta), transb=bool(tb))
    torch.cuda.synchronize()
    _check_grid(C, A, B, ta, tb, seed)
    del A, B, C
    _free()


def test_batched_result_beyond_2_31_elements():
    """Three 27000 x 27000 results (2.19e9 elements in all) with alpha and
    beta: the last entry starts past element 2^31 of C."""
    M = N = 27000
    K, batch = 32, 3
    note(f"large: batched C {batch} x {M}x{N}x{K}")
    A = inputs.small_integers_device((batch, M, K), 11)
    B = inputs.small_integers_device((batch, K, N), 12)
    C = inputs.small_integers_device((batch, M, N), 13)
    rows = inputs.grid_sample(M, 14)
    cols = inputs.grid_sample(N, 15)
    ri = torch.as_tensor(rows, device="cuda")
    ci = torch.as_tensor(cols, device="cuda")
    C0 = [C[z][ri][:, ci].cpu().numpy() for z in range(batch)]
    sg.sgemm_batched(A, B, out=C, alpha=2.0, beta=-1.0)
    torch.cuda.synchronize()
    for z in range(batch):
        a = np.ascontiguousarray(A[z][ri].cpu().numpy())
        b = np.ascontiguousarray(B[z][:, ci].cpu().numpy())
        ref, absb = oracle.gemm_ref(a, b, False, False, 2.0, -1.0, C0[z])
        got = C[z][ri][:, ci].cpu().numpy()
        rep = oracle.compare(got, ref, absb)
        assert rep["n_bad"] == 0, (z, rep)
        assert np.array_equal(got.astype(np.float64), ref), (z, rep)
    del A, B, C
    _free()


def _variants_for(ta, tb):
    return [vid for vid in range(sg.sgemm_f32_num_variants())
            if sg.sgemm_f32_variant_ops(vid) & (1 << (ta + 2 * tb))]


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("which", ["past_direct", "maximum"])
def test_leading_dimension_limits_every_variant(ta, tb, which):
    """Every variant compiled for the layout, on operands whose row strides
    are just past the direct-load range or at the largest accepted value
    (a 300 x 200 x 100 product with ragged tiles, full check)."""
    M, N, K = 300, 200, 100
    if which == "past_direct":
        ld_k, ld_x = DIRECT_LD_K + 4, DIRECT_LD_X + 4
    else:
        ld_k, ld_x = MAX_LD_K, MAX_LD_X
    A, B = inputs.make_operands(M, N, K, seed=90 + ta + 2 * tb)
    As, Bs = stored(A, ta), stored(B, tb)
    lda = ld_x if ta else ld_k
    ldb = ld_k if tb else ld_x
    Ad = place(As, pad=lda - As.shape[1])
    Bd = place(Bs, pad=ldb - Bs.shape[1])
    assert Ad.stride(0) == lda and Bd.stride(0) == ldb
    # variants with 64-deep slices serve an index-contiguous operand (B, or a
    # transposed A) only up to DEEP_LD_X
    has_x = ta == 1 or tb == 0
    for vid in _variants_for(ta, tb) + [None]:
        note(f"ld limits {which} ta={ta} tb={tb} lda={lda} ldb={ldb} variant {vid}")
        C = torch.full((M, N), float("nan"), device="cuda")
        if vid is not None and sg.sgemm_f32_variant(vid).bk == 64 and has_x and ld_x > DEEP_LD_X:
            with pytest.raises(sg.SgemmError):
                sg.sgemm(Ad, Bd, out=C, cfg=forced(vid), transa=bool(ta), transb=bool(tb))
            continue
        sg.sgemm(Ad, Bd, out=C, cfg=None if vid is None else forced(vid),
                 transa=bool(ta), transb=bool(tb))
        torch.cuda.synchronize()
        check_general(C.cpu().numpy(), As, Bs, ta, tb)
    del Ad, Bd
    _free()



@pytest.mark.parametrize("case", [
    # name,                               ta, tb,  M,   N,   K,             lda,        ldb
    ("64x64xK lda 2^22+64 (packed A)",      0, 0,  64,  64, (1 << 22) + 64, None,      None),
    ("1x1xK lda 2^22+64 (strips)",          0, 0,   1,   1, (1 << 22) + 64, None,      None),
    ("300x200x8 ldb 2^25+4",                0, 0, 300, 200, 8,              None,      (1 << 25) + 4),
    ("300x200x4 stored A^T lda 2^26",       1, 0, 300, 200, 4,              1 << 26,   None),
    ("100x64x100 stored B^T ldb 2^23",      0, 1, 100,  64, 100,            None,      1 << 23),
], ids=lambda c: c[0].split(" ")[0] + "_" + str(c[1]) + str(c[2]))
def test_leading_dimensions_past_the_tiled_kernels(case):
    """Leading dimensions past the LDS-tiled kernels' 32-bit in-slice offsets,
    through the default plan (64-bit K-split tiles or strips), with and
    without a workspace; inputs in [-1, 1] integers, so every sum is exact
    (K < 2^24) and the result must equal the reference bit for bit."""
    name, ta, tb, M, N, K, lda, ldb = case
    seed = 500 + M + N
    gen = np.random.default_rng(seed)
    As = gen.integers(-1, 2, size=(K, M) if ta else (M, K)).astype(np.float32)
    Bs = gen.integers(-1, 2, size=(N, K) if tb else (K, N)).astype(np.float32)
    Ad = place(As, pad=0 if lda is None else lda - As.shape[1])
    Bd = place(Bs, pad=0 if ldb is None else ldb - Bs.shape[1])
    ref, absb = oracle.gemm_ref(As, Bs, ta, tb)
    for workspace in (False, True):
        note(f"large ld: {name} workspace={workspace} lda={Ad.stride(0)} ldb={Bd.stride(0)}")
        C = torch.full((M, N), float("nan"), device="cuda")
        sg.sgemm(Ad, Bd, out=C, transa=bool(ta), transb=bool(tb), workspace=workspace)
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        rep = oracle.compare(got, ref, absb)
        assert rep["n_bad"] == 0, rep
        assert np.array_equal(got.astype(np.float64), ref), rep
    del Ad, Bd
    _free()
