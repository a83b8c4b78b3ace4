"""The entry point that allocates nothing (sgemm_f32_ex_noalloc), through the
C ABI: its K splits keep their partials in the library's static per-GPU
scratch.  Each case runs the same product through sgemm_f32_ex with a
workspace as large as the scratch (the same plan, so the same bits) and
checks both against the CPU reference; two calls in a row, the second on a
smaller product, so the scratch holds the first call's partials when the
second starts."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import fp32_gemm_sgemm_amd as sg  # noqa: E402
from fp32_gemm_sgemm_amd import inputs  # noqa: E402

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from gpu_cases import forced_split, note, stored  # noqa: E402

HIP_ERROR_OUT_OF_MEMORY = 2


def _product(M, N, K, ta, tb, seed, batch=1):
    rng = np.random.default_rng(seed)
    A = rng.uniform(-1, 1, size=(batch, M, K)).astype(np.float32)
    B = rng.uniform(-1, 1, size=(batch, K, N)).astype(np.float32)
    C0 = rng.uniform(-1, 1, size=(batch, M, N)).astype(np.float32)
    As = np.stack([stored(a, ta) for a in A])
    Bs = np.stack([stored(b, tb) for b in B])
    return As, Bs, C0


def _run(fn, As, Bs, C0, ta, tb, alpha, beta, cfg):
    """One call through the raw binding; returns (hipError_t, C as numpy)."""
    batch = As.shape[0]
    M = As.shape[2] if ta else As.shape[1]
    K = As.shape[1] if ta else As.shape[2]
    N = Bs.shape[1] if tb else Bs.shape[2]
    A = torch.from_numpy(As).cuda()
    B = torch.from_numpy(Bs).cuda()
    C = torch.from_numpy(C0.copy()).cuda()
    h = torch.cuda.current_stream().cuda_stream
    args = (ta, tb, M, N, K, alpha, A.data_ptr(), As.shape[2], As[0].size,
            B.data_ptr(), Bs.shape[2], Bs[0].size, beta, C.data_ptr(), N, M * N, batch)
    code = fn(*args, h, cfg)
    torch.cuda.synchronize()
    return code, C.cpu().numpy()


def _with_workspace(ws):
    def fn(*args):
        h, cfg = args[-2], args[-1]
        return sg.sgemm_f32_ex(*args[:-2], ws.data_ptr(), ws.numel(), h, cfg)
    return fn


def _noalloc(*args):
    h, cfg = args[-2], args[-1]
    return sg.sgemm_f32_ex_noalloc(*args[:-2], h, cfg)


# (M, N, K, ta, tb, batch, alpha, beta, forced (variant, splits) or None)
CASES = [
    # the selector splits K 64 ways (4 MiB of partials), then a smaller split
    [(128, 128, 32768, 0, 0, 1, 1.0, 0.0, None), (96, 80, 20000, 1, 0, 1, -0.5, 1.5, None)],
    # forced splits through the 64 x 64 tile, then a smaller product in another layout
    [(200, 190, 3000, 0, 1, 2, 1.0, 0.0, (11, 6)), (70, 45, 1001, 1, 1, 3, 2.0, -1.0, (11, 3))],
    # no split (a product that fills the chip), then a small split product
    [(512, 512, 512, 0, 0, 1, 1.0, 0.0, None), (64, 64, 8192, 0, 0, 1, 1.0, 0.0, None)],
]


@pytest.mark.parametrize("pair", CASES)
def test_noalloc_matches_workspace_entry_point(pair):
    ws = torch.empty(sg.SGEMM_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    for i, (M, N, K, ta, tb, batch, alpha, beta, force) in enumerate(pair):
        cfg = None if force is None else forced_split(*force)
        note(f"noalloc call {i}: {batch} x {M}x{N}x{K} ta={ta} tb={tb} alpha={alpha} "
             f"beta={beta} cfg={force}")
        As, Bs, C0 = _product(M, N, K, ta, tb, 900 + 10 * i + M, batch)
        code_ws, C_ws = _run(_with_workspace(ws), As, Bs, C0, ta, tb, alpha, beta, cfg)
        code_na, C_na = _run(_noalloc, As, Bs, C0, ta, tb, alpha, beta, cfg)
        assert code_ws == 0 and code_na == 0, (code_ws, code_na)
        # the same plan with the same scratch size: the same bits
        assert np.array_equal(C_na, C_ws)
        ref, absb = oracle.gemm_ref_batched(As, Bs, ta, tb, alpha, beta, C0)
        rep = oracle.compare(C_na, ref, absb)
        assert rep["n_bad"] == 0, rep


def test_noalloc_plan_splits_within_the_scratch():
    """The selector's plan for the first case splits K, and its partials fit."""
    q = sg.sgemm_f32_plan(128, 128, 32768, 32768, 128, 128, 0, 0, 0, 1, sg.SGEMM_SCRATCH_BYTES)
    assert q.splits > 1 and 0 < q.workspace_bytes <= sg.SGEMM_SCRATCH_BYTES


def test_noalloc_refuses_a_split_larger_than_the_scratch():
    """A forced split whose partials exceed the scratch is refused before any
    launch, and C is left as it was."""
    M = N = 2048
    K = 4096
    cfg = forced_split(4, 8)
    need = sg.sgemm_f32_cfg_geometry(cfg, 0, 0, M, N, K, K, N, N).workspace_bytes
    assert need > sg.SGEMM_SCRATCH_BYTES
    note("noalloc refusal 2048x2048x4096 split 8")
    A, B = inputs.make_operands(M, N, K, seed=950)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    C = torch.full((M, N), 7.0, device="cuda")
    code = sg.sgemm_f32_ex_noalloc(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, 0, Bd.data_ptr(), N, 0,
                                   0.0, C.data_ptr(), N, 0, 1,
                                   torch.cuda.current_stream().cuda_stream, cfg)
    torch.cuda.synchronize()
    assert code == HIP_ERROR_OUT_OF_MEMORY
    assert bool((C == 7.0).all())


def test_noalloc_under_graph_capture():
    """The point of the entry point: a K-split product captured in a HIP graph
    with nothing allocated on the way.  The graph is replayed three times with
    an eager call of the same entry point (sharing the scratch, in stream
    order) and a synchronisation between replays; every replay must equal the
    eager result bit for bit, and that result must match the reference."""
    M, N, K = 96, 128, 24000
    q = sg.sgemm_f32_plan(M, N, K, K, N, N, 0, 0, 0, 1, sg.SGEMM_SCRATCH_BYTES)
    assert q.splits > 1, q.as_dict()
    A, B = inputs.make_operands(M, N, K, seed=960)
    Ad, Bd = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()

    def call(out, stream):
        code = sg.sgemm_f32_ex_noalloc(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, 0, Bd.data_ptr(), N,
                                       0, 0.0, out.data_ptr(), N, 0, 1, stream.cuda_stream, None)
        assert code == 0

    note(f"noalloc graph capture {M}x{N}x{K} split {q.splits}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    eager = torch.empty((M, N), device="cuda")
    with torch.cuda.stream(side):
        call(eager, side)          # first call on the device: the scratch lookup, outside capture
    torch.cuda.synchronize()
    want = eager.cpu().numpy()
    ref, absb = oracle.sgemm_ref(A, B)
    rep = oracle.compare(want, ref, absb)
    assert rep["n_bad"] == 0, rep
    Cg = torch.full((M, N), float("nan"), device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(Cg, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(3):
        graph.replay()
        again = torch.full((M, N), float("nan"), device="cuda")
        call(again, torch.cuda.current_stream())      # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(Cg.cpu().numpy(), want), f"replay {r}"
        assert np.array_equal(again.cpu().numpy(), want), f"eager call after replay {r}"
    del graph
