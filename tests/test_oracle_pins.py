"""Pins for the CPU reference: checks against facts fixed by mathematics and by
the pages, never against the reference itself or the HIP path.

* exact sums (fractions.Fraction and math.fsum) on small shapes, including the
  DD2360 workbook's lab shapes 64x64 and 100x50x70 (section 14.3);
* closed forms: identity, permutations, all-ones, rank-1, constant rows and
  columns, small integers;
* numpy's float64 matmul (a library routine with its own summation order);
* invariants: thread-count and sample-versus-full bit equality, leading
  dimensions, sign symmetry of absb.
A mutation check at the end shows that plausible mistakes (a dropped term, a
flipped sign, a transposed operand, a wrong row stride) fail these pins.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from fp32_gemm_sgemm_amd import inputs

U = 2.0 ** -53  # unit roundoff of binary64


def _sum_bound(K, absb):
    """Recursive-summation bound for K exact terms: gamma_{K-1} * sum|p|."""
    n = max(K - 1, 0)
    return (n * U / (1 - n * U)) * absb


def _rand(M, N, K, seed):
    return inputs.make_operands(M, N, K, seed)


# ---- exact sums ---------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 4), (7, 5, 3), (17, 13, 11)])
def test_fraction_brute_force(M, N, K):
    A, B = _rand(M, N, K, seed=M * 100 + N * 10 + K)
    ref, absb = oracle.sgemm_ref(A, B, nthreads=2)
    for i in range(M):
        for j in range(N):
            terms = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)]
            exact = sum(terms, Fraction(0))
            exact_abs = sum((abs(t) for t in terms), Fraction(0))
            bound = Fraction(_sum_bound(K, float(exact_abs)))
            assert abs(Fraction(ref[i, j]) - exact) <= bound
            assert abs(Fraction(absb[i, j]) - exact_abs) <= bound


def _fsum_reference(A, B):
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    P = A64[:, :, None] * B64[None, :, :]          # (M, K, N), products exact
    M, K, N = P.shape
    exact = np.empty((M, N))
    exact_abs = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            exact[i, j] = math.fsum(P[i, :, j])
            exact_abs[i, j] = math.fsum(np.abs(P[i, :, j]))
    return exact, exact_abs


def _within_exact(ref, absb, A, B):
    exact, exact_abs = _fsum_reference(A, B)
    K = A.shape[1]
    # fsum is the correctly rounded exact sum: one extra half-ulp of slack
    tol = _sum_bound(K, exact_abs) + U * np.abs(exact) + 1e-300
    return bool(np.all(np.abs(ref - exact) <= tol) and np.all(np.abs(absb - exact_abs) <= tol))


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (100, 70, 50), (33, 65, 129)])
def test_fsum_exact_sum(M, N, K):
    """Workbook lab shapes: 64x64 and A 100x50 times B 50x70."""
    A, B = _rand(M, N, K, seed=11)
    ref, absb = oracle.sgemm_ref(A, B)
    assert _within_exact(ref, absb, A, B)


def test_numpy_float64_matmul():
    A, B = _rand(257, 193, 311, seed=3)
    ref, absb = oracle.sgemm_ref(A, B)
    lib = A.astype(np.float64) @ B.astype(np.float64)
    K = A.shape[1]
    # both sides round K-1 additions, in different orders
    assert np.all(np.abs(ref - lib) <= 2.0 * _sum_bound(K, absb) + 1e-300)


# ---- closed forms -------------------------------------------------------------

def test_identity_gives_b_exactly():
    K, N = 37, 53
    _, B = _rand(K, N, K, seed=5)
    ref, absb = oracle.sgemm_ref(inputs.identity(K), B)
    assert np.array_equal(ref, B.astype(np.float64))
    assert np.array_equal(absb, np.abs(B).astype(np.float64))


def test_row_permutation():
    K, N = 41, 29
    _, B = _rand(K, N, K, seed=6)
    P, perm = inputs.permutation(K, seed=7)
    ref, _ = oracle.sgemm_ref(P, B)
    assert np.array_equal(ref, B[perm].astype(np.float64))


def test_column_permutation():
    M, K = 23, 31
    A, _ = _rand(M, K, K, seed=8)
    P, perm = inputs.permutation(K, seed=9)
    ref, _ = oracle.sgemm_ref(A, P)          # (A P)[:, perm[k]] = A[:, k]
    expect = np.empty((M, K))
    expect[:, perm] = A.astype(np.float64)
    assert np.array_equal(ref, expect)


@pytest.mark.parametrize("M,N,K", [(5, 7, 1), (19, 3, 1000), (64, 64, 4099)])
def test_all_ones_gives_k(M, N, K):
    ref, absb = oracle.sgemm_ref(inputs.ones((M, K)), inputs.ones((K, N)))
    assert np.all(ref == K) and np.all(absb == K)


def test_rank_one_k1_exact_outer_product():
    A, B = _rand(31, 47, 1, seed=12)
    ref, absb = oracle.sgemm_ref(A, B)
    outer = A.astype(np.float64) * B.astype(np.float64)   # (31,1)*(1,47)
    assert np.array_equal(ref, outer)
    assert np.array_equal(absb, np.abs(outer))


def test_constant_rows_and_columns():
    rng = np.random.default_rng(13)
    M, N, K = 17, 23, 301
    x = rng.integers(-3, 4, size=M).astype(np.float32)
    y = rng.integers(-3, 4, size=N).astype(np.float32)
    A = np.repeat(x[:, None], K, axis=1)
    B = np.repeat(y[None, :], K, axis=0)
    ref, _ = oracle.sgemm_ref(A, B)
    expect = K * np.outer(x.astype(np.int64), y.astype(np.int64))
    assert np.array_equal(ref, expect.astype(np.float64))


def test_small_integers_exact():
    rng = np.random.default_rng(14)
    A = inputs.small_integers(rng, (96, 112))
    B = inputs.small_integers(rng, (112, 80))
    ref, absb = oracle.sgemm_ref(A, B)
    ia, ib = A.astype(np.int64), B.astype(np.int64)
    assert np.array_equal(ref, (ia @ ib).astype(np.float64))
    assert np.array_equal(absb, (np.abs(ia) @ np.abs(ib)).astype(np.float64))


def test_empty_sum_and_empty_output():
    A = np.zeros((4, 0), dtype=np.float32)
    B = np.zeros((0, 6), dtype=np.float32)
    ref, absb = oracle.sgemm_ref(A, B)
    assert ref.shape == (4, 6) and np.all(ref == 0) and np.all(absb == 0)
    ref, _ = oracle.sgemm_ref(np.zeros((0, 3), np.float32), np.zeros((3, 5), np.float32))
    assert ref.shape == (0, 5)


# ---- invariants -----------------------------------------------------------------

def test_absb_properties():
    A, B = _rand(45, 39, 77, seed=15)
    ref, absb = oracle.sgemm_ref(A, B)
    assert np.all(absb >= np.abs(ref))
    ref_n, absb_n = oracle.sgemm_ref(-A, B)
    assert np.array_equal(ref_n, -ref) and np.array_equal(absb_n, absb)
    ref_p, absb_p = oracle.sgemm_ref(np.abs(A), np.abs(B))
    assert np.array_equal(ref_p, absb_p)


def test_thread_count_independent():
    A, B = _rand(67, 45, 93, seed=16)
    r1, s1 = oracle.sgemm_ref(A, B, nthreads=1)
    for t in (3, 8, 100):
        rt, st = oracle.sgemm_ref(A, B, nthreads=t)
        assert np.array_equal(r1, rt) and np.array_equal(s1, st)


def test_sampled_matches_full_bitwise():
    A, B = _rand(150, 170, 90, seed=17)
    ref, absb = oracle.sgemm_ref(A, B)
    rows, cols = inputs.sample_indices(150, 170, seed=17, n_uniform=300, n_edge=100, band=16, last=2)
    r, s = oracle.sgemm_ref_sampled(A, B, rows, cols, nthreads=3)
    assert np.array_equal(r, ref[rows, cols]) and np.array_equal(s, absb[rows, cols])


def test_leading_dimensions():
    A, B = _rand(20, 30, 40, seed=18)
    Abig = np.full((20, 47), np.nan, dtype=np.float32)
    Bbig = np.full((40, 35), np.nan, dtype=np.float32)
    Abig[:, :40] = A
    Bbig[:, :30] = B
    r1, s1 = oracle.sgemm_ref(A, B)
    r2, s2 = oracle.sgemm_ref(Abig[:, :40], Bbig[:, :30])   # padding is NaN, never read
    assert np.array_equal(r1, r2) and np.array_equal(s1, s2)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.sgemm_ref(np.zeros((3, 4), np.float32), np.zeros((5, 2), np.float32))
    with pytest.raises(TypeError):
        oracle.sgemm_ref(np.zeros((3, 4), np.float64), np.zeros((4, 2), np.float32))
    A = np.zeros((3, 4), np.float32)
    B = np.zeros((4, 2), np.float32)
    with pytest.raises(RuntimeError):
        oracle.sgemm_ref_sampled(A, B, [3], [0])     # row out of range


# ---- the acceptance check -----------------------------------------------------------

def test_compare_accepts_float32_product_and_flags_planted_errors():
    A, B = _rand(128, 96, 256, seed=19)
    ref, absb = oracle.sgemm_ref(A, B)
    c32 = np.zeros((128, 96), dtype=np.float32)
    # a float32 dot product in plain sequential order: error <= ~K*2^-24*absb
    for k in range(256):
        c32 += np.outer(A[:, k], B[k, :]).astype(np.float32)
    rep = oracle.compare(c32, ref, absb)
    assert rep["n_bad"] == 0 and rep["max_norm_err"] < 1e-4
    bad = c32.copy()
    bad[3, 4] = np.float32(ref[3, 4] + 2e-4 * absb[3, 4])
    rep = oracle.compare(bad, ref, absb)
    assert rep["n_bad"] == 1 and rep["first_bad"] == 3 * 96 + 4
    nan = c32.copy()
    nan[7, 7] = np.nan
    assert oracle.compare(nan, ref, absb)["n_bad"] == 1
    inf = c32.copy()
    inf[0, 0] = np.inf
    assert oracle.compare(inf, ref, absb)["n_bad"] == 1
    # an element whose terms are all zero must come out exactly zero
    z = np.zeros((1, 1)), np.zeros((1, 1))
    assert oracle.compare(np.array([[1e-30]]), *z)["n_bad"] == 1
    assert oracle.compare(np.array([[0.0]]), *z)["n_bad"] == 0


def test_sample_indices_deterministic_and_in_range():
    r1, c1 = inputs.sample_indices(4099, 4099, seed=3, last=3)
    r2, c2 = inputs.sample_indices(4099, 4099, seed=3, last=3)
    assert np.array_equal(r1, r2) and np.array_equal(c1, c2)
    assert r1.min() >= 0 and r1.max() < 4099 and c1.min() >= 0 and c1.max() < 4099
    edge_r, edge_c = r1[3584:4096], c1[3584:4096]
    assert np.all((edge_r >= 4099 - 256) | (edge_c >= 4099 - 256))
    assert len(r1) == 4096 + 3 * 4099 * 2
    assert set(r1[4096:4096 + 3 * 4099].tolist()) == {4096, 4097, 4098}


# ---- the pins catch plausible mistakes --------------------------------------------------

def _mutants():
    def dropped_last_term(A, B):
        a, b = A.astype(np.float64), B.astype(np.float64)
        return a[:, :-1] @ b[:-1], np.abs(a[:, :-1]) @ np.abs(b[:-1])

    def flipped_sign(A, B):
        a, b = A.astype(np.float64), B.astype(np.float64).copy()
        b[0] = -b[0]
        return a @ b, np.abs(a) @ np.abs(b)

    def transposed_b(A, B):
        a, b = A.astype(np.float64), B.astype(np.float64)
        bt = b.T if b.shape[0] == b.shape[1] else b[::-1]
        return a @ bt, np.abs(a) @ np.abs(bt)

    def wrong_row_stride(A, B):
        # reads B as if its rows were one element longer
        a = A.astype(np.float64)
        flat = np.concatenate([B.reshape(-1), np.zeros(B.shape[0], np.float32)])
        K, N = B.shape
        b = np.stack([flat[k * (N + 1): k * (N + 1) + N] for k in range(K)]).astype(np.float64)
        return a @ b, np.abs(a) @ np.abs(b)

    return [dropped_last_term, flipped_sign, transposed_b, wrong_row_stride]


def _pins_pass(fn):
    """The pin suite in miniature, applied to a candidate reference."""
    A, B = _rand(33, 33, 33, seed=21)
    ref, absb = fn(A, B)
    if not _within_exact(ref, absb, A, B):
        return False
    P, perm = inputs.permutation(33, seed=22)
    ref, _ = fn(P, B)
    if not np.array_equal(ref, B[perm].astype(np.float64)):
        return False
    ref, _ = fn(inputs.ones((9, 33)), inputs.ones((33, 11)))
    return bool(np.all(ref == 33))


def test_pins_accept_oracle_and_reject_mutants():
    assert _pins_pass(lambda A, B: oracle.sgemm_ref(A, B))
    for m in _mutants():
        assert not _pins_pass(m), m.__name__


# ---- the general form: op(), alpha, beta, batches ------------------------------------
# Pinned by closed forms that a dropped or doubled transpose, a scalar applied
# to the wrong term or a batch entry taken from the wrong place would break.

def test_general_transposed_permutations():
    """op(A) = P^T for a stored permutation P gives the inverse row
    permutation of B; op(B) = P^T gives a column gather of A (exact)."""
    P, perm = inputs.permutation(37, seed=61)
    _, B = _rand(37, 23, 37, seed=62)
    ref, _ = oracle.gemm_ref(P, B, transa=True)
    assert np.array_equal(ref, B[np.argsort(perm)].astype(np.float64))
    ref, _ = oracle.gemm_ref(P, B, transa=False)
    assert np.array_equal(ref, B[perm].astype(np.float64))
    A, _ = _rand(19, 37, 37, seed=63)
    ref, _ = oracle.gemm_ref(A, P, transb=True)
    assert np.array_equal(ref, A[:, perm].astype(np.float64))
    ref, _ = oracle.gemm_ref(A, P, transb=False)
    assert np.array_equal(ref, A[:, np.argsort(perm)].astype(np.float64))


@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True), (True, True)])
def test_general_transposes_of_stored_transposes(ta, tb):
    """Storing an operand transposed and asking for its transpose is the
    plain product, on non-square shapes (a missed transpose changes the
    shapes or the values)."""
    A, B = _rand(21, 13, 17, seed=64)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    ref, absb = oracle.gemm_ref(As, Bs, ta, tb)
    want = np.array([[math.fsum(float(A[i, k]) * float(B[k, j]) for k in range(17))
                      for j in range(13)] for i in range(21)])
    assert np.all(np.abs(ref - want) <= _sum_bound(17, absb))
    assert ref.shape == (21, 13)


def test_general_alpha_beta_closed_forms():
    A, B = _rand(12, 9, 7, seed=65)
    C0 = inputs.make_operands(12, 9, 1, seed=66)[0][:, :1] * np.ones((1, 9), np.float32)
    ref1, absb1 = oracle.gemm_ref(A, B)
    # a power-of-two alpha scales exactly
    ref, absb = oracle.gemm_ref(A, B, alpha=-0.5)
    assert np.array_equal(ref, -0.5 * ref1) and np.array_equal(absb, 0.5 * absb1)
    # alpha = 0: beta * C0 exactly, A and B not used (NaN operands are ignored)
    nanA = np.full_like(A, np.nan)
    ref, absb = oracle.gemm_ref(nanA, B, alpha=0.0, beta=-2.0, C0=C0)
    assert np.array_equal(ref, -2.0 * C0.astype(np.float64))
    assert np.array_equal(absb, 2.0 * np.abs(C0.astype(np.float64)))
    # beta = 0: C0 not used (NaN is ignored)
    ref, _ = oracle.gemm_ref(A, B, beta=0.0, C0=np.full((12, 9), np.nan, np.float32))
    assert np.array_equal(ref, ref1)
    # K = 0: beta * C0
    Z, Zb = np.zeros((12, 0), np.float32), np.zeros((0, 9), np.float32)
    ref, _ = oracle.gemm_ref(Z, Zb, alpha=3.0, beta=0.25, C0=C0)
    assert np.array_equal(ref, 0.25 * C0.astype(np.float64))
    # identity: alpha * I x B + beta * C0 with small integers is exact
    rng = np.random.default_rng(67)
    Bi = inputs.small_integers(rng, (12, 9))
    Ci = inputs.small_integers(rng, (12, 9))
    ref, _ = oracle.gemm_ref(inputs.identity(12), Bi, alpha=3.0, beta=-1.0, C0=Ci)
    assert np.array_equal(ref, 3.0 * Bi.astype(np.float64) - Ci.astype(np.float64))


def test_general_batched_entries_and_broadcast():
    rng = np.random.default_rng(68)
    A = rng.uniform(-1, 1, (3, 5, 4)).astype(np.float32)
    B = rng.uniform(-1, 1, (1, 4, 6)).astype(np.float32)    # broadcast
    ref, absb = oracle.gemm_ref_batched(A, B)
    assert ref.shape == (3, 5, 6)
    for z in range(3):
        r, s = oracle.gemm_ref(A[z], B[0])
        assert np.array_equal(ref[z], r) and np.array_equal(absb[z], s)
    # entries are independent: permuting A's stack permutes the results
    ref2, _ = oracle.gemm_ref_batched(A[::-1].copy(), B)
    assert np.array_equal(ref2, ref[::-1])
    with pytest.raises(ValueError):
        oracle.gemm_ref_batched(A, np.zeros((2, 4, 6), np.float32))


def _general_mutants():
    def transpose_ignored(A, B, ta, tb):
        a = A if not ta else A.reshape(A.shape[1], A.shape[0])
        b = B if not tb else B.reshape(B.shape[1], B.shape[0])
        return oracle.gemm_ref(np.ascontiguousarray(a), np.ascontiguousarray(b))

    def transposes_swapped(A, B, ta, tb):
        return oracle.gemm_ref(A, B, tb, ta) if A.shape[0] == B.shape[1] else (None, None)

    return [transpose_ignored, transposes_swapped]


def test_general_pins_reject_mutants():
    P, perm = inputs.permutation(37, seed=61)
    _, B = _rand(37, 37, 37, seed=62)
    want = B[np.argsort(perm)].astype(np.float64)
    for m in _general_mutants():
        ref, _ = m(P, B, True, False)
        assert ref is None or not np.array_equal(ref, want), m.__name__
