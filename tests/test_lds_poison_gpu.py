"""LDS race check: parity cases run through the LDS-poisoned build
(libsgemm_lds_poison.so, the same sources compiled with SGEMM_LDS_POISON=1,
where every LDS word is set to a quiet NaN before it is refilled).  A read
that came before its fill landed, or after its words were released to the
next fill, would return NaN and spread it into C.  Each case must therefore
give the normal build's result bit for bit (and no NaN), and match the CPU
reference element by element.

Covered: every variant in every operand layout on ragged multi-tile shapes,
with direct loads and with the register fetch (odd strides, 4-byte shifted
starts); long K (many reuses of each LDS stage) for the tile families and the
K-split 32x32 tiles; K split across workgroups; edge strips and strip-only
products past one staged chunk; strided batches."""
import numpy as np
import pytest

import oracle
import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import inputs
from gpu_cases import check_general, forced, forced_split, note, run_general, stored

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

LAYOUTS = [(0, 0), (1, 0), (0, 1), (1, 1)]


@pytest.fixture(scope="module", autouse=True)
def poisoned_build():
    if not __import__("os").path.exists(sg.POISON_LIB_PATH):
        pytest.fail(f"{sg.POISON_LIB_PATH} is not built (python -m fp32_gemm_sgemm_amd.build)")
    sg.load(sg.POISON_LIB_PATH)


def both(fn):
    """fn() with the normal build, then with the LDS-poisoned build."""
    normal = fn()
    with sg.library(sg.POISON_LIB_PATH):
        poisoned = fn()
    return normal, poisoned


def assert_race_free(normal, poisoned):
    assert not np.isnan(poisoned).any(), "NaN from the poisoned build: an LDS read raced"
    assert np.array_equal(normal.view(np.uint32), poisoned.view(np.uint32)), \
        "the poisoned build's result differs from the normal build's"


def variants_for(ta, tb):
    return [v for v in range(sg.sgemm_f32_num_variants())
            if sg.sgemm_f32_variant_ops(v) & (1 << (ta + 2 * tb))]


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_every_variant_race_free(ta, tb):
    M, N, K = 517, 389, 261
    A, B = inputs.make_operands(M, N, K, seed=500 + ta + 2 * tb)
    As, Bs = stored(A, ta), stored(B, tb)
    for vid in variants_for(ta, tb):
        for pad, shift in [((0, 0, 0), (0, 0, 0)), ((3, 1, 5), (1, 1, 1))]:
            note(f"lds poison ta={ta} tb={tb} variant {vid} pad={pad} shift={shift}")
            n, p = both(lambda: run_general(As, Bs, ta, tb, cfg=forced(vid), pad=pad,
                                            shift=shift))
            assert_race_free(n, p)
            check_general(p, As, Bs, ta, tb)


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 1)])
def test_long_k_race_free(ta, tb):
    """K = 4099: every LDS stage of the tile loops is refilled many times;
    the K-split 32x32 tiles sum many partial ranges through LDS."""
    M, N, K = 200, 130, 4099
    A, B = inputs.make_operands(M, N, K, seed=510 + ta + 2 * tb)
    As, Bs = stored(A, ta), stored(B, tb)
    ids = [v for v in variants_for(ta, tb)
           if sg.sgemm_f32_variant(v).bm in (32, 64, 128) or v == 4]
    for vid in ids:
        note(f"lds poison long K ta={ta} tb={tb} variant {vid}")
        n, p = both(lambda: run_general(As, Bs, ta, tb, cfg=forced(vid)))
        assert_race_free(n, p)
        check_general(p, As, Bs, ta, tb)


@pytest.mark.parametrize("vid,splits", [(4, 3), (11, 5), (16, 4)])
def test_split_k_race_free(vid, splits):
    M, N, K = 300, 260, 3001
    A, B = inputs.make_operands(M, N, K, seed=520 + vid)
    note(f"lds poison split K variant {vid} splits {splits}")
    n, p = both(lambda: run_general(A, B, 0, 0, alpha=0.75, beta=-0.5, C0=np.ones((M, N), np.float32),
                                    cfg=forced_split(vid, splits)))
    assert_race_free(n, p)
    check_general(p, A, B, 0, 0, alpha=0.75, beta=-0.5, C0=np.ones((M, N), np.float32))


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_strips_race_free(ta, tb):
    """Edge strips beside tiles, and strip-only products of 3 rows and of 3
    columns, with K past two staged chunks of the small operand (4608)."""
    for (M, N, K, sm, sn) in [(517, 389, 9301, 3, 2), (3, 777, 9301, 3, 0), (700, 3, 9301, 0, 3)]:
        A, B = inputs.make_operands(M, N, K, seed=530 + M + ta + 2 * tb)
        As, Bs = stored(A, ta), stored(B, tb)
        cfg = forced(4)
        cfg.strip_m, cfg.strip_n = sm, sn
        note(f"lds poison strips ta={ta} tb={tb} {M}x{N}x{K} sm={sm} sn={sn}")
        n, p = both(lambda: run_general(As, Bs, ta, tb, cfg=cfg, workspace=False))
        assert_race_free(n, p)
        check_general(p, As, Bs, ta, tb)


def test_batched_race_free():
    batch, M, N, K = 5, 130, 70, 300
    A = np.stack([inputs.make_operands(M, N, K, seed=540 + z)[0] for z in range(batch)])
    B = np.stack([inputs.make_operands(M, N, K, seed=540 + z)[1] for z in range(batch)])

    def call():
        C = torch.empty((batch, M, N), device="cuda")
        sg.sgemm_batched(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), out=C)
        torch.cuda.synchronize()
        return C.cpu().numpy()

    note("lds poison batched")
    n, p = both(call)
    assert_race_free(n, p)
    ref, absb = oracle.gemm_ref_batched(A, B, 0, 0)
    rep = oracle.compare(p, ref, absb)
    assert rep["n_bad"] == 0, rep
