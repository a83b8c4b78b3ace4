"""The timeline build (libsgemm_timeline.so, SGEMM_TIMELINE=1) on the GPU.

It computes what the normal build computes: bit for bit on the same plan, and
within the oracle's bound.  Its readings are consistent: in every workgroup of
a call the clock readings are in order (entry, loop start, loop end, stores
done); the main loop takes at least its MFMA time at the FP32 matrix rate;
every slice of the first workgroups carries its two readings and the slots
past the last slice stay empty; and a plan on another kernel records nothing."""
import numpy as np
import pytest

import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import inputs, timeline
from gpu_cases import check_general, forced, note, run_general

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)


@pytest.fixture(scope="module", autouse=True)
def timeline_build():
    if not __import__("os").path.exists(sg.TIMELINE_LIB_PATH):
        pytest.fail(f"{sg.TIMELINE_LIB_PATH} is not built (python -m fp32_gemm_sgemm_amd.build)")
    sg.load(sg.TIMELINE_LIB_PATH)


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 1)])
def test_timeline_build_computes_the_same_results(ta, tb):
    M, N, K = 517, 389, 261
    A, B = inputs.make_operands(M, N, K, seed=600 + ta + 2 * tb)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    for vid in [4, 6, 7, 11, 12, 20, 25]:
        if not sg.sgemm_f32_variant_ops(vid) & (1 << (ta + 2 * tb)):
            continue
        note(f"timeline build ta={ta} tb={tb} variant {vid}")
        normal = run_general(As, Bs, ta, tb, cfg=forced(vid))
        with sg.library(sg.TIMELINE_LIB_PATH):
            timed = run_general(As, Bs, ta, tb, cfg=forced(vid))
        assert np.array_equal(normal.view(np.uint32), timed.view(np.uint32)), vid
        check_general(timed, As, Bs, ta, tb)


@pytest.mark.parametrize("M,N,K,vid", [(640, 384, 1000, 7), (520, 300, 777, 4), (256, 256, 96, 20),
                                       (300, 200, 64, 11)])
def test_readings_are_consistent(M, N, K, vid):
    note(f"timeline readings {M}x{N}x{K} variant {vid}")
    cfg, phase, sl, khz, (normal_us, timed_us) = timeline.measure(M, N, K, vid, warm_ms=5.0, seed=vid)
    assert normal_us > 0 and timed_us > 0
    nwg = cfg.grid
    ph = phase[:nwg].astype(np.int64)
    assert (ph[:, 0] > 0).all(), "a workgroup left no readings"
    assert (np.diff(ph[:, :4], axis=1) >= 0).all(), "readings out of order"
    assert (ph[:, 5] > ph[:, 4]).all() and khz > 0
    ghz = (ph[:, 3] - ph[:, 0]) / ((ph[:, 5] - ph[:, 4]) / khz * 1e6)
    assert ((ghz > 0.3) & (ghz < 3.0)).all(), ghz
    assert not phase[nwg:].any(), "readings past the grid"
    nk = -(-K // cfg.bk)
    ideal = cfg.bm * cfg.bn * nk * cfg.bk * 2 / timeline.FLOP_PER_CYCLE_PER_CU
    assert (ph[:, 2] - ph[:, 1] >= 0.95 * ideal).all(), "a loop ran faster than the matrix cores"
    waves = cfg.threads // 64
    for w in range(min(nwg, sl.shape[0])):
        rec = sl[w, :waves, :nk]
        assert (rec != 0).any(axis=-1).all(), f"workgroup {w}: a slice without readings"
        wait = (rec[..., 1].astype(np.int64) - rec[..., 0].astype(np.int64)) % (1 << 32)
        assert (wait < 10_000_000).all()
        assert not sl[w, waves:].any() and not sl[w, :, nk:].any()
    assert not sl[nwg:].any()
    s = timeline.summarize(cfg, K, phase, sl, khz)
    assert s["workgroups"] == nwg and 0 < s["loop_efficiency"] <= 1.05
    assert s["call_span_us"] > 0
    assert s["slice_period"][1] > 0


def test_other_kernels_record_nothing():
    """The register-staged tiles (variants 0, 1, 3, 8 and 9), the K-split
    32 x 32 and 16 x 16 tiles and the vector-FMA kernel carry no readings."""
    lib = sg.load(sg.TIMELINE_LIB_PATH)
    others = [0, 1, 3, 8, 9] + [v for v in range(sg.sgemm_f32_num_variants())
                                if sg.sgemm_f32_variant(v).kernel == sg.SGEMM_KERNEL_VALU
                                or (sg.sgemm_f32_variant(v).bm <= 32
                                    and sg.sgemm_f32_variant(v).waves_n == 1)]
    A, B = inputs.make_operands(200, 150, 300, seed=610)
    for vid in others:
        note(f"timeline build, no readings from variant {vid}")
        assert lib.sgemm_f32_timeline_clear() == 0
        with sg.library(sg.TIMELINE_LIB_PATH):
            C = run_general(A, B, 0, 0, cfg=forced(vid))
        check_general(C, A, B, 0, 0)
        phase, sl = timeline.read(lib)
        assert not phase.any() and not sl.any(), vid


def test_command_line_summary(tmp_path):
    """python -m fp32_gemm_sgemm_amd.timeline writes a summary with both tables
    for a forced plan, a batched and transposed default plan, and a plan on
    the K-split 32 x 32 tiles (a row without readings)."""
    out = tmp_path / "summary.md"
    note("timeline command line")
    assert timeline.main(["--out", str(out), "--shape", "256", "256", "96", "20",
                          "--shape", "640", "384", "512", "-1", "4", "0", "1",
                          "--shape", "300", "200", "64", "16"]) == 0
    md = out.read_text()
    assert "| 256x256x96 | v20 64x64x32, 4 waves" in md
    assert "| 4 x 640x384x512 NT | v20 64x64x32" in md
    assert "| 300x200x64 | v16 32x32x8 (no readings" in md
    assert "call us, normal / timeline build" in md
    assert "--shape 256 256 96 20 --shape 640 384 512 -1 4 0 1 --shape 300 200 64 16" in md
