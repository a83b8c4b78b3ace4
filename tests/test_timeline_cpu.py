"""Host logic of the timeline report (fp32_gemm_sgemm_amd.timeline) on
synthetic readings: phase durations, the loop's ideal and efficiency, the
shader clock's rate and the call's span from the real-time counter, the slice
period from the last wave arrivals, the waits, and 32-bit wrap of the
per-slice counts."""
import numpy as np

import fp32_gemm_sgemm_amd as sg
from fp32_gemm_sgemm_amd import timeline


def cfg(bm=128, bn=128, bk=32, threads=512, grid=4, splits=1, k_chunk=0):
    c = sg.SgemmCfg()
    c.bm, c.bn, c.bk, c.threads, c.grid, c.splits, c.k_chunk = bm, bn, bk, threads, grid, splits, k_chunk
    return c


def test_phases_and_ideal():
    c = cfg(grid=3)
    phase = np.zeros((4096, 6), np.uint64)
    for w in range(3):  # prologue 1000, loop 5000 + 10 w, stores 300
        t0 = 10_000_000 * (w + 1)
        phase[w, :4] = [t0, t0 + 1000, t0 + 6000 + 10 * w, t0 + 6300 + 10 * w]
        # real time (100 MHz): starts 0, 1, 2 us after the first; 6300 + 10 w
        # cycles at 2.1 GHz take 3 us (+ 10 w / 2100 us)
        r0 = 5_000 + 100 * w
        phase[w, 4:] = [r0, r0 + round((6300 + 10 * w) / 21)]
    phase[3] = [1, 2, 3, 4, 5, 6]  # past the grid: ignored
    sl = np.zeros((16, 16, 256, 2), np.uint32)
    K = 96  # 3 slices of 32
    s = timeline.summarize(c, K, phase, sl, khz=100_000)
    assert s["workgroups"] == 3 and s["slices"] == 3
    assert all(abs(g - 2.1) < 0.01 for g in s["clock_ghz"])
    assert s["start_us"] == [1.0, 1.8, 2.0]
    assert s["call_span_us"] == round((200 + round(6320 / 21)) / 100, 2)
    assert "clock_ghz" not in timeline.summarize(c, K, phase, sl)  # no rate given
    assert s["prologue"] == [1000, 1000, 1000] and s["stores"] == [300, 300, 300]
    assert s["loop"][1] == 5010
    ideal = 128 * 128 * 96 * 2 / 256
    assert s["loop_ideal"] == ideal == 12288
    assert s["loop_efficiency"] == round(ideal / 5010, 4)
    assert "slice_period" not in s  # no per-slice readings


def test_slice_statistics_with_wrap():
    c = cfg(grid=1, threads=128)  # two waves
    phase = np.zeros((4096, 6), np.uint64)
    phase[0] = [5, 10, 20, 30, 0, 0]
    sl = np.zeros((16, 16, 256, 2), np.uint32)
    base = (1 << 32) - 1500  # the 32-bit counter wraps during the loop
    # wave 0 arrives at base + 1000 s, wave 1 at base + 1000 s + 100; each
    # waits 40 (s = 0, 1) or 60 (s = 2) for its own loads
    for v in range(2):
        for k in range(3):
            t1 = (base + 1000 * k + 100 * v) % (1 << 32)
            w = 60 if k == 2 else 40
            sl[0, v, k] = [(t1 - w) % (1 << 32), t1]
    s = timeline.summarize(c, 96, phase, sl)
    assert s["slice_period"] == [1000, 1000, 1000]
    assert s["slice_ideal"] == 4096
    assert s["wait_own_loads"] == [40, 40, 60]  # percentiles of [40] * 4 + [60] * 2
    # the last wave (1) waits 0 at each barrier, wave 0 waits 100
    assert s["wait_barrier"] == [0, 50, 100]


def test_k_split_uses_the_split_range():
    c = cfg(grid=2, splits=4, k_chunk=64)
    phase = np.zeros((4096, 6), np.uint64)
    phase[:2] = [[1, 2, 1002, 1003, 0, 0], [1, 2, 1002, 1003, 0, 0]]
    s = timeline.summarize(c, 256, phase, np.zeros((16, 16, 256, 2), np.uint32))
    assert s["slices"] == 2 and s["loop_ideal"] == 128 * 128 * 64 * 2 // 256


def test_markdown_names_batches_and_layouts():
    row = {"shape": [1024, 1024, 128], "batch": 64, "layout": "NT", "variant": 4,
           "tile": "256x256x32", "waves": 8, "grid": 1024, "strips": [0, 0], "workgroups": 1024,
           "prologue": [1, 2, 3], "loop": [4, 5, 6], "loop_ideal": 5, "loop_efficiency": 1.0,
           "stores": [7, 8, 9], "slice_period": [1, 1, 1], "slice_ideal": 1,
           "wait_own_loads": [40, 40, 40], "wait_barrier": [0, 0, 0]}
    md = timeline.markdown([row], "python -m fp32_gemm_sgemm_amd.timeline")
    assert "| 64 x 1024x1024x128 NT | v4 256x256x32, 8 waves" in md
