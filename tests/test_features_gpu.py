"""GPU parity for the BLAS-style paths: transposed operands, alpha/beta,
K split across workgroups with a fixed-order reduction, and strided batches.
Every result is compared element by element with the CPU reference's general
form (oracle.gemm_ref / gemm_ref_batched) on seeded inputs."""
import numpy as np
import pytest

import oracle
import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import inputs
from gpu_cases import (check_general, forced, forced_split, note, place, run_general,
                       stored)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

LAYOUTS = [(0, 0), (1, 0), (0, 1), (1, 1)]


def variants_for(ta, tb, selectable_only=False):
    out = []
    for vid in range(sg.sgemm_f32_num_variants()):
        if sg.sgemm_f32_variant_ops(vid) & (1 << (ta + 2 * tb)):
            out.append(vid)
    return out


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(300, 200, 100), (257, 513, 129), (64, 96, 33), (1, 1, 1),
                                   (520, 390, 700)])
def test_transposed_layouts_default(ta, tb, M, N, K):
    note(f"layout ta={ta} tb={tb} {M}x{N}x{K}")
    A, B = inputs.make_operands(M, N, K, seed=70 + ta + 2 * tb)
    As, Bs = stored(A, ta), stored(B, tb)
    check_general(run_general(As, Bs, ta, tb), As, Bs, ta, tb)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_transposed_layouts_every_variant(ta, tb):
    """Each variant compiled for the layout, on a shape spanning several
    tiles with ragged edges in M, N and K; aligned (direct loads) and with
    padded, odd row strides and a 4-byte shifted start (register fetch)."""
    M, N, K = 517, 389, 261
    A, B = inputs.make_operands(M, N, K, seed=80 + ta + 2 * tb)
    As, Bs = stored(A, ta), stored(B, tb)
    for vid in variants_for(ta, tb):
        for pad, shift in [((0, 0, 0), (0, 0, 0)), ((4, 8, 0), (0, 0, 0)),
                           ((3, 1, 5), (1, 1, 1))]:
            note(f"layout ta={ta} tb={tb} variant {vid} pad={pad} shift={shift}")
            C = run_general(As, Bs, ta, tb, cfg=forced(vid), pad=pad, shift=shift)
            check_general(C, As, Bs, ta, tb)


def _ksplit_variants():
    return [v for v in range(sg.sgemm_f32_num_variants())
            if (sg.sgemm_f32_variant(v).bm, sg.sgemm_f32_variant(v).bk) in ((32, 8), (16, 16), (8, 32))]


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_ksplit_tiles_k_ranges(ta, tb):
    """The tiles that split K over their W waves (32 x 32 tiles in 8-deep
    groups, 16 x 16 ones in 16-deep groups, the 8 x 8 vector-FMA ones in
    32-deep groups, one k per lane pair): each wave takes a range of whole
    G-deep groups and keeps four groups of loads in flight (prefetch clamped
    to its last whole group); the last wave may end in a ragged group.  K
    values cover a single k, one ragged group, exactly one group per wave, one
    k more or less, waves left with no range (K below G (W - 1)), whole
    prefetch blocks plus a remainder, and ragged M and N."""
    for vid in _ksplit_variants():
        W = sg.sgemm_f32_variant(vid).waves_m
        G = sg.sgemm_f32_variant(vid).bk
        ks = sorted({1, 3, G - 1, G, G + 1, G * W - 1, G * W, G * W + 1, G * (W - 1) - 3,
                     G * W * 4 * 2 + 5, G * W * 4 * 3 + G * 3, G * W * 5 + 17} - {0})
        for K in ks:
            if K <= 0:
                continue
            M, N = 70, 45
            note(f"k-split variant {vid} (W={W}) ta={ta} tb={tb} {M}x{N}x{K}")
            A, B = inputs.make_operands(M, N, K, seed=700 + K + vid)
            As, Bs = stored(A, ta), stored(B, tb)
            check_general(run_general(As, Bs, ta, tb, cfg=forced(vid)), As, Bs, ta, tb)


def test_vector_fma_ksplit_tile_both_k_contiguous():
    """The 8 x 8 vector-FMA K-split tile in the NT layout (both operands
    k-contiguous), whose lanes each take 4 successive k of 256-deep steps:
    K below one step, exactly one and one more, steps that leave waves
    without a range, an odd number of whole steps per wave (the loop and its
    tail) with and without a ragged step, and outputs of fewer than 8 rows
    or columns."""
    vid = next(v for v in range(sg.sgemm_f32_num_variants())
               if (sg.sgemm_f32_variant(v).bm, sg.sgemm_f32_variant(v).bk) == (8, 32))
    W = sg.sgemm_f32_variant(vid).waves_m
    for M, N in [(70, 45), (5, 3), (8, 8)]:
        for K in (1, 255, 256, 257, 256 * (W - 1) + 3, 3 * 256 * W, 3 * 256 * W + 77,
                  5 * 256 * W + 1):
            note(f"vector-FMA k-split NT variant {vid} {M}x{N}x{K}")
            A, B = inputs.make_operands(M, N, K, seed=720 + K + M)
            Bs = stored(B, 1)
            check_general(run_general(A, Bs, 0, 1, cfg=forced(vid)), A, Bs, 0, 1)


def test_random_problems_through_the_selector():
    """100 seeded random problems through the default plan: small, medium,
    skinny with long K and wide with short K, half with sizes that are
    multiples of 4; random layout, alpha/beta, workspace or none, padded
    strides and 4-byte shifted starts.  The plans this reaches include the
    K-split 32 x 32 tiles (with and without an outer split), the K-split
    16 x 16 and 8 x 8 tiles, the 64 x 64 tiles with 32- and 64-deep slices and edge
    strips."""
    rng = np.random.default_rng(20261202)
    for case in range(100):
        kind = rng.integers(0, 4)
        if kind == 0:
            M, N, K = (int(x) for x in rng.integers(1, 200, size=3))
        elif kind == 1:
            M, N, K = (int(x) for x in rng.integers(1, 1100, size=3))
        elif kind == 2:
            M, N = (int(x) for x in rng.integers(1, 300, size=2))
            K = int(rng.integers(500, 9000))
        else:
            M, N = (int(x) for x in rng.integers(500, 1500, size=2))
            K = int(rng.integers(1, 700))
        if rng.random() < 0.5:
            M, N, K = [max(1, (x // 4) * 4) for x in (M, N, K)]
        ta, tb = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        alpha = float(rng.choice([1.0, -0.5, 2.0]))
        beta = float(rng.choice([0.0, 0.0, 1.0, -1.5]))
        ws = bool(rng.random() < 0.5)
        pad = tuple(int(x) for x in rng.choice([0, 0, 3, 4], size=3))
        shift = tuple(int(x) for x in rng.choice([0, 0, 1], size=3))
        A, B = inputs.make_operands(M, N, K, seed=3000 + case)
        C0 = inputs.make_operands(M, N, 1, seed=5000 + case)[0] if beta != 0 else None
        if C0 is not None:
            C0 = np.ascontiguousarray(np.repeat(C0[:, :1], N, axis=1))
        As, Bs = stored(A, ta), stored(B, tb)
        note(f"random case {case}: {M}x{N}x{K} ta={ta} tb={tb} alpha={alpha} beta={beta} "
             f"ws={ws} pad={pad} shift={shift}")
        C = run_general(As, Bs, ta, tb, alpha=alpha, beta=beta, C0=C0, workspace=ws, pad=pad,
                        shift=shift)
        check_general(C, As, Bs, ta, tb, alpha=alpha, beta=beta, C0=C0)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_transposed_exact_cases(ta, tb):
    """Closed forms through the transposed paths: a stored permutation
    matrix used transposed gathers rows (or columns) by the inverse
    permutation, exactly."""
    n = 131
    P, perm = inputs.permutation(n, seed=90)
    _, X = inputs.make_operands(n, 77, n, seed=91)
    note(f"permutation ta={ta} tb={tb}")
    if tb == 0:
        # op(A) = P or P^T; B = X (stored transposed when ta... only A varies)
        C = run_general(P, stored(X, 0), ta, 0)
        want = X[np.argsort(perm)] if ta else X[perm]
        assert np.array_equal(C, want)
    else:
        Y = np.ascontiguousarray(X.T)                 # 77 x n
        C = run_general(stored(Y, ta), P, ta, 1)
        want = Y[:, perm]
        assert np.array_equal(C, want)


@pytest.mark.parametrize("alpha,beta", [(1.5, -0.75), (-2.0, 0.0), (0.0, 0.5), (0.0, 0.0),
                                        (1.0, 1.0), (0.25, 2.0)])
def test_alpha_beta(alpha, beta):
    M, N, K = 333, 222, 150
    A, B = inputs.make_operands(M, N, K, seed=100)
    C0 = inputs.make_operands(M, N, 1, seed=101)[0][:, :1] * np.linspace(-1, 1, N, dtype=np.float32)
    C0 = np.ascontiguousarray(C0.astype(np.float32))
    for vid in (None, 1, 2, 3, 4, 5, 6, 14, 15, 16, 17, 18, 22, 23, 24):
        note(f"alpha={alpha} beta={beta} variant {vid}")
        cfg = None if vid is None else forced(vid)
        C = run_general(A, B, 0, 0, alpha, beta, C0, cfg=cfg)
        check_general(C, A, B, 0, 0, alpha, beta, C0)
        if alpha == 0.0:
            assert np.array_equal(C, (np.float32(beta) * C0).astype(np.float32))


def test_beta_zero_ignores_nan_and_k_zero_scales():
    M, N = 100, 60
    A, B = inputs.make_operands(M, N, 40, seed=102)
    note("beta 0 over NaN C")
    nan = np.full((M, N), np.nan, np.float32)
    C = run_general(A, B, 0, 0, 1.0, 0.0, nan)
    check_general(C, A, B, 0, 0)
    note("K = 0 with beta")
    C0 = inputs.make_operands(M, N, 1, seed=103)[0][:, :1] * np.ones((1, N), np.float32)
    Z, Zb = np.zeros((M, 0), np.float32), np.zeros((0, N), np.float32)
    C = run_general(Z, Zb, 0, 0, 3.0, -0.5, np.ascontiguousarray(C0))
    assert np.array_equal(C, (np.float32(-0.5) * C0).astype(np.float32))


SPLIT_VARIANTS = [1, 2, 3, 4, 5, 6, 14, 15, 16, 17, 18, 22, 23, 24]


@pytest.mark.parametrize("K", [1000, 1001, 130])
def test_split_k_forced(K):
    """Every kernel family with forced K splits (ragged last split, K not a
    multiple of 4), reduced in fixed order: within the bound, and bitwise the
    same on a second run."""
    M, N = 300, 203
    A, B = inputs.make_operands(M, N, K, seed=110 + K)
    for vid in SPLIT_VARIANTS:
        for splits in (2, 3, 8):
            note(f"split-K variant {vid} splits {splits} K={K}")
            cfg = forced_split(vid, splits)
            C1 = run_general(A, B, 0, 0, cfg=cfg)
            check_general(C1, A, B, 0, 0)
            C2 = run_general(A, B, 0, 0, cfg=cfg)
            assert np.array_equal(C1, C2)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_split_k_with_layouts_and_scalars(ta, tb):
    M, N, K = 190, 170, 1500
    A, B = inputs.make_operands(M, N, K, seed=120 + ta + 2 * tb)
    As, Bs = stored(A, ta), stored(B, tb)
    C0 = np.ascontiguousarray(inputs.make_operands(M, N, 1, seed=121)[0][:, :1] *
                              np.ones((1, N), np.float32))
    for vid in (4, 5, 15):
        note(f"split-K layout ta={ta} tb={tb} variant {vid}")
        C = run_general(As, Bs, ta, tb, -1.25, 0.5, C0, cfg=forced_split(vid, 5))
        check_general(C, As, Bs, ta, tb, -1.25, 0.5, C0)


def test_split_k_long_k_single_tile_auto():
    """128 x 128 x 32768 (one output tile): with a workspace the selector
    splits K; the result is checked in full and is reproducible."""
    M, N, K = 128, 128, 32768
    A, B = inputs.make_operands(M, N, K, seed=47)
    Ad, Bd = place(A), place(B)
    Cd = torch.empty((M, N), device="cuda")
    ws_bytes = sg.sgemm_f32_workspace_size(0, 0, M, N, K, K, N, N, 1)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    q = sg.sgemm_f32_query(0, 0, M, N, K, Ad.data_ptr(), K, 0, Bd.data_ptr(), N, 0,
                           Cd.data_ptr(), N, 0, 1, ws.data_ptr(), ws_bytes)
    note(f"auto split 128x128x32768: variant {q.id} splits {q.splits} ws {ws_bytes}")
    assert q.splits > 1 and q.workspace_bytes == ws_bytes
    code = sg.sgemm_f32_gemm(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0,
                             Cd.data_ptr(), N, ws.data_ptr(), ws_bytes,
                             torch.cuda.current_stream().cuda_stream)
    assert code == 0
    torch.cuda.synchronize()
    C1 = Cd.cpu().numpy()
    check_general(C1, A, B, 0, 0)
    sg.sgemm_f32_gemm(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, Bd.data_ptr(), N, 0.0,
                      Cd.data_ptr(), N, ws.data_ptr(), ws_bytes,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(C1, Cd.cpu().numpy())


def test_small_config_with_workspace():
    """512^3 (the small configuration) through the workspace entry point."""
    A, B = inputs.make_operands(512, 512, 512, seed=0)
    note("512^3 with workspace")
    C = run_general(A, B, 0, 0)
    check_general(C, A, B, 0, 0)


def _batched_stack(batch, rows, cols, seed, gap):
    """A (batch, rows, cols) device view whose entries are rows*cols + gap
    floats apart, and the host copy."""
    rng = np.random.default_rng(seed)
    host = rng.uniform(-1, 1, (batch, rows, cols)).astype(np.float32)
    stride = rows * cols + gap
    buf = torch.zeros(max(batch * stride, 1), dtype=torch.float32, device="cuda")
    view = torch.as_strided(buf, (batch, rows, cols), (stride, cols, 1))
    view.copy_(torch.from_numpy(host))
    return view, host


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_strided_batched(ta, tb):
    batch, M, N, K = 5, 70, 90, 130
    Ar = (K, M) if ta else (M, K)
    Br = (N, K) if tb else (K, N)
    A, Ah = _batched_stack(batch, *Ar, seed=130, gap=37)
    B, Bh = _batched_stack(batch, *Br, seed=131, gap=0)
    C0h = np.random.default_rng(132).uniform(-1, 1, (batch, M, N)).astype(np.float32)
    C = torch.zeros((batch, M, N + 3), device="cuda")[:, :, :N]
    C.copy_(torch.from_numpy(C0h))
    note(f"strided batched ta={ta} tb={tb}")
    sg.sgemm_batched(A, B, out=C, transa=ta, transb=tb, alpha=0.5, beta=-1.0)
    torch.cuda.synchronize()
    ref, absb = oracle.gemm_ref_batched(Ah, Bh, ta, tb, 0.5, -1.0, C0h)
    rep = oracle.compare(C.cpu().numpy(), ref, absb)
    assert rep["n_bad"] == 0, rep


def test_strided_batched_broadcast_and_split():
    """Stride 0 reuses one B for every entry; a forced split over a batch."""
    batch, M, N, K = 7, 100, 64, 900
    A, Ah = _batched_stack(batch, M, K, seed=140, gap=5)
    B, Bh = _batched_stack(1, K, N, seed=141, gap=0)
    for cfg in (None, forced_split(5, 3), forced_split(1, 4)):
        note(f"batched broadcast cfg={None if cfg is None else (cfg.id, cfg.splits)}")
        C = sg.sgemm_batched(A, B, cfg=cfg)
        torch.cuda.synchronize()
        ref, absb = oracle.gemm_ref_batched(Ah, Bh)
        rep = oracle.compare(C.cpu().numpy(), ref, absb)
        assert rep["n_bad"] == 0, rep


def test_batched_many_small_entries():
    batch, M, N, K = 3000, 8, 12, 20
    A, Ah = _batched_stack(batch, M, K, seed=150, gap=0)
    B, Bh = _batched_stack(batch, K, N, seed=151, gap=0)
    note("3000 small entries")
    C = sg.sgemm_batched(A, B)
    torch.cuda.synchronize()
    ref, absb = oracle.gemm_ref_batched(Ah, Bh)
    rep = oracle.compare(C.cpu().numpy(), ref, absb)
    assert rep["n_bad"] == 0, rep


def test_batch_beyond_one_launch():
    """More entries than one reduction launch's second grid dimension holds
    (65535) and, for the GEMM, more workgroups than one dispatch holds
    (2^32 work-items): the host splits the launches.  A and B are broadcast
    (stride 0), so every entry must equal the one reference."""
    M, N, K = 4, 4, 128
    A, B = inputs.make_operands(M, N, K, seed=160)
    Ad, Bd = place(A), place(B)
    ref, absb = oracle.gemm_ref(A, B)
    for batch, cfg in [(70000, forced_split(1, 2)), (8_500_000, forced(0))]:
        note(f"batch {batch} cfg ({cfg.id}, {cfg.splits})")
        C = torch.empty((batch, M, N), device="cuda")
        ws_bytes = sg.sgemm_f32_cfg_geometry(cfg, 0, 0, M, N, K, K, N, N, batch).workspace_bytes
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        code = sg.sgemm_f32_ex(0, 0, M, N, K, 1.0, Ad.data_ptr(), K, 0, Bd.data_ptr(), N, 0,
                               0.0, C.data_ptr(), N, M * N, batch, ws.data_ptr(), ws_bytes,
                               torch.cuda.current_stream().cuda_stream, cfg)
        assert code == 0
        torch.cuda.synchronize()
        Ch = C.cpu().numpy()
        rep = oracle.compare(Ch[0], ref, absb)
        assert rep["n_bad"] == 0, rep
        assert np.all(Ch == Ch[0][None])
        del C, ws
        torch.cuda.empty_cache()


def test_batch_zero_and_empty():
    A = torch.zeros((0, 4, 4), device="cuda")
    B = torch.zeros((0, 4, 4), device="cuda")
    note("batch 0")
    C = sg.sgemm_batched(A, B)
    torch.cuda.synchronize()
    assert C.shape == (0, 4, 4)


def test_hip_graph_capture_and_replay():
    """The library's launches (GEMM, split-K reduction, alpha/beta) can be
    captured in a HIP graph on torch's capture stream: it records no memset
    and allocates nothing.  The graph is replayed several times with eager
    work and synchronisations in between, and every replay is compared with
    the eager result bit for bit."""
    M, N, K = 300, 200, 1000
    A, B = inputs.make_operands(M, N, K, seed=170)
    Ad, Bd = place(A), place(B)
    C0 = np.ascontiguousarray(inputs.make_operands(M, N, 1, seed=171)[0][:, :1] *
                              np.ones((1, N), np.float32))
    for cfg, alpha, beta in [(None, 1.0, 0.0), (forced_split(8, 4), 1.0, 0.0),
                             (forced_split(4, 3), -0.5, 2.0)]:
        wsb = 0 if cfg is None else sg.sgemm_f32_cfg_geometry(cfg, 0, 0, M, N, K, K, N, N).workspace_bytes
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        Cd = place(C0)
        eager = place(C0)
        note(f"graph capture cfg={None if cfg is None else (cfg.id, cfg.splits)} alpha={alpha} beta={beta}")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())

        def call(out, stream):
            code = sg.sgemm_f32_ex(0, 0, M, N, K, alpha, Ad.data_ptr(), K, 0, Bd.data_ptr(), N, 0,
                                   beta, out.data_ptr(), N, 0, 1, ws.data_ptr(), wsb,
                                   stream.cuda_stream, cfg)
            assert code == 0
        with torch.cuda.stream(s):
            call(eager, s)           # warm-up on the side stream, outside capture
        torch.cuda.synchronize()
        want_once = eager.cpu().numpy()
        check_general(want_once, A, B, 0, 0, alpha, beta, C0)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call(Cd, torch.cuda.current_stream())
        # beta != 0 accumulates: the eager reference repeats the same calls
        ref = place(C0)
        Cd.copy_(torch.from_numpy(C0))
        torch.cuda.synchronize()
        for rep in range(3):
            graph.replay()
            call(ref, torch.cuda.current_stream())     # eager work between replays
            torch.cuda.synchronize()
            assert np.array_equal(Cd.cpu().numpy(), ref.cpu().numpy()), f"replay {rep}"
        del graph


def _stack(host, pad, sh):
    """A (batch, rows, cols) device view of `host` with row stride cols + pad,
    entries 3*pad floats apart, starting `sh` floats into its buffer."""
    b, r, c = host.shape
    ld = c + pad
    stride = r * ld + 3 * pad
    buf = torch.zeros(sh + b * stride + 4, dtype=torch.float32, device="cuda")
    view = torch.as_strided(buf, (b, r, c), (stride, ld, 1), storage_offset=sh)
    view.copy_(torch.from_numpy(host))
    return view


def test_random_configurations_with_strips():
    """40 seeded random problems whose M and N are a multiple of 32 plus 0-4
    (or at most 4), each through the selector and through a forced variant
    with forced strips of 0-4 rows and columns and a forced K split, in any
    layout, with alpha/beta, batches, padded strides and shifted starts."""
    rng = np.random.default_rng(4242)
    nvar = sg.sgemm_f32_num_variants()

    def dim():
        if rng.random() < 0.2:
            return int(rng.integers(1, 5))
        return 32 * int(rng.integers(1, 9)) + int(rng.integers(0, 5))

    for case in range(40):
        M, N = dim(), dim()
        K = int(rng.integers(1, 700))
        ta, tb = (int(x) for x in rng.integers(0, 2, size=2))
        batch = int(rng.choice([1, 1, 2]))
        alpha = float(rng.choice([1.0, -0.75, 2.5]))
        beta = float(rng.choice([0.0, 0.0, -0.5]))
        pads = [int(x) for x in rng.integers(0, 6, size=3)]
        shift = [int(x) for x in rng.integers(0, 2, size=3)]
        ops = [v for v in range(nvar) if sg.sgemm_f32_variant_ops(v) & (1 << (ta + 2 * tb))]
        Ar, Br = ((K, M) if ta else (M, K)), ((N, K) if tb else (K, N))
        Ah = rng.uniform(-1, 1, (batch,) + Ar).astype(np.float32)
        Bh = rng.uniform(-1, 1, (batch,) + Br).astype(np.float32)
        C0 = rng.uniform(-1, 1, (batch, M, N)).astype(np.float32)
        ref, absb = oracle.gemm_ref_batched(Ah, Bh, ta, tb, alpha, beta, C0)
        vid = int(rng.choice(ops))
        sm = int(rng.integers(0, min(4, M) + 1))
        sn = int(rng.integers(0, min(4, N) + 1))
        splits = int(rng.choice([1, 2, 3]))
        for cfg in (None, "forced"):
            if cfg == "forced":
                cfg = forced_split(vid, splits)
                cfg.strip_m, cfg.strip_n = sm, sn
            note(f"random strips case {case}: {M}x{N}x{K} ta={ta} tb={tb} batch={batch} "
                 f"alpha={alpha} beta={beta} cfg={'selector' if cfg is None else (vid, splits, sm, sn)} "
                 f"pads={pads} shift={shift}")
            A, B, C = _stack(Ah, pads[0], shift[0]), _stack(Bh, pads[1], shift[1]), \
                _stack(C0, pads[2], shift[2])
            sg.sgemm_batched(A, B, out=C, transa=ta, transb=tb, alpha=alpha, beta=beta, cfg=cfg)
            torch.cuda.synchronize()
            rep = oracle.compare(C.cpu().numpy(), ref, absb)
            assert rep["n_bad"] == 0, (case, rep)


def test_random_configurations():
    """40 seeded random problems mixing every feature: layout, alpha/beta,
    batch with gaps between entries, a forced variant compiled for the layout
    (or the selector), a forced K split, padded row strides and 4-byte
    shifted starts; each compared in full with the general reference."""
    rng = np.random.default_rng(31337)
    nvar = sg.sgemm_f32_num_variants()
    for case in range(40):
        M, N, K = (int(x) for x in rng.integers(1, 260, size=3))
        ta, tb = (int(x) for x in rng.integers(0, 2, size=2))
        batch = int(rng.choice([1, 1, 2, 3]))
        alpha = float(rng.choice([1.0, -0.75, 0.0, 2.5]))
        beta = float(rng.choice([0.0, 0.0, 1.0, -0.5]))
        pads = [int(x) for x in rng.integers(0, 6, size=3)]
        shift = [int(x) for x in rng.integers(0, 2, size=3)]
        ops = [v for v in range(nvar) if sg.sgemm_f32_variant_ops(v) & (1 << (ta + 2 * tb))]
        vid = None if rng.random() < 0.3 else int(rng.choice(ops))
        splits = int(rng.choice([1, 1, 2, 3, 8]))
        note(f"random case {case}: {M}x{N}x{K} ta={ta} tb={tb} batch={batch} alpha={alpha} "
             f"beta={beta} variant={vid} splits={splits} pads={pads} shift={shift}")
        Ar, Br = ((K, M) if ta else (M, K)), ((N, K) if tb else (K, N))
        Ah = rng.uniform(-1, 1, (batch,) + Ar).astype(np.float32)
        Bh = rng.uniform(-1, 1, (batch,) + Br).astype(np.float32)
        C0 = rng.uniform(-1, 1, (batch, M, N)).astype(np.float32)

        def stack(host, pad, sh):
            b, r, c = host.shape
            ld = c + pad
            stride = r * ld + 3 * pad
            buf = torch.zeros(sh + b * stride + 4, dtype=torch.float32, device="cuda")
            view = torch.as_strided(buf, (b, r, c), (stride, ld, 1), storage_offset=sh)
            view.copy_(torch.from_numpy(host))
            return view
        A, B, C = stack(Ah, pads[0], shift[0]), stack(Bh, pads[1], shift[1]), stack(C0, pads[2], shift[2])
        cfg = None
        if vid is not None:
            cfg = forced_split(vid, splits)
        sg.sgemm_batched(A, B, out=C, transa=ta, transb=tb, alpha=alpha, beta=beta, cfg=cfg)
        torch.cuda.synchronize()
        ref, absb = oracle.gemm_ref_batched(Ah, Bh, ta, tb, alpha, beta, C0)
        rep = oracle.compare(C.cpu().numpy(), ref, absb)
        assert rep["n_bad"] == 0, (case, rep)
