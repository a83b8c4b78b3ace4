#!/usr/bin/env python3
"""Benchmark: single-precision GEMM TFLOP/s on one MI355X, and its fraction of
the FP32 matrix peak.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one C = A x B call through the library's C ABI at the headline
workload, M = N = K = 8192, row-major, A and B i.i.d. U[-1, 1] drawn with seed
4 (synthetic data; inputs are resident in HBM before timing starts).  W
untimed warm-up steps are followed by exactly K timed steps back to back,
bracketed by device synchronisation, with one pair of HIP events recorded on
the launch stream around them; a second pass of K steps, each between its
own events, gives the per-step distribution (median, min, p90) and the
roofline's mean launch time.  TFLOP/s = 2*M*N*K / t ("4.1 CUDA GEMM operator
performance optimization", section 1.3).  By default the operands stay cached
between steps (warm); --cold writes 512 MiB between steps, outside the step's
events, and takes the value from the per-step events.  A second workload, 3072^3 with N(0, 1) inputs
(seed 2), is timed the same way and reported under "secondary"; its launches
are only ~0.45 ms, so it is warmed for at least --secondary-warm-ms of GPU
time (the chip takes about 0.1 s of sustained load to reach its full clock;
with 3 warm-up launches the same kernel reads ~15% slower).

One JSON line is printed.  Besides the driver's fields it holds:
  roofline      the dominant (only) kernel against the FP32 matrix peak
                (157.3 TFLOP/s): achieved = 2*M*N*K / mean launch time;
                traffic = HBM bytes per launch from rocprofv3 counters stored
                under profiles/, or null if the kernel sources changed since.
  cpu_baseline  the CPU reference (oracle/) timed on this host on a bounded
                sample of the same product (whole rows of C, about
                --cpu-seconds of work), in TFLOP/s, with the threads used and
                the host's core count, and on one thread over a smaller
                sample; the sampled rows are also compared with the GPU result
                (n, n_bad, max normalised error, RRMSE).
  configs       every configuration of the measured workload set through
                sgemm_f32 (the plain C ABI, no workspace): 512^3, 2048^3 (and
                its identity-A run), 3072^3, 8192x8192x4096, 4096x4096x8192,
                the ragged 4099^3 and 8192^3, each after a time-based warm-up:
                mean time per call over back-to-back calls, and the median,
                min and p90 of per-call times.  Unless --no-cpu-baseline, each
                carries `check`, its accuracy against the CPU reference (part
                of the CPU-reference leg): full at 512^3 and for the
                identity-A run (which must also equal B exactly), the seeded
                4096-output sample otherwise, plus the last 3 rows and
                columns of 4099^3 in full.
  metric_figures  which numbers are the metric's 8192^3 and 3072^3 figures.
  meta          device, HIP runtime and driver, ROCm and hipcc versions, the
                power mode, and the host's cores.
  vendor        context only: torch.matmul in float32 (the ROCm BLAS libraries,
                TF32 disabled) timed the same way on the square shapes from
                512^3 to 8192^3 and on 128 x 128 x 32768 in every layout, and
                torch.bmm on the two batched attention products.
  extras        the library's other paths, each timed the same way after a
                time-based warm-up (--extra-warm-ms): the small 512^3
                configuration and the one-tile 128 x 128 x 32768 product with
                and without a workspace (K split across workgroups), the same
                product in every layout on each form of tile that splits K
                inside the workgroup (forced: 32 x 32, 16 x 16, 8 x 8), the
                transposed-operand layouts at 8192^3 and 3072^3, strided
                batches of attention-like products, the 1024 x 8192 x 8192
                row band one GPU would run if 8192^3 were split over 8 GPUs,
                1024^3 (one 64 x 64 tile per CU), three shapes the selector
                gives 32 x 64 tiles (beside the tile it would use without
                them, forced), shapes whose few edge rows or columns (or all of them, for
                products of 1 row or column) go to the strip kernel, and the
                vector-FMA comparison kernel forced at 8192^3 and 3072^3
                (with its fraction of valu_probe).
  mfma_probe    the sustained v_mfma_f32_32x32x2_f32 rate on register operands
                (the matrix-core ceiling at the chip's actual clock), and the
                headline's fraction of it.
  valu_probe    the sustained non-packed v_fma_f32 rate on register operands
                (the vector-ALU ceiling the comparison kernel is bound by).
  launch_floor  an empty launch with the 512^3 plan's grid (256 workgroups of
                512 threads), timed like the configurations: the part of a
                small product's time that is not its work.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SGEMM TFLOP/s and % of FP32 matrix peak at 3072³ and 8192³, 1×MI355X"
HEADLINE = "sgemm_8192x8192x8192_uniform_seed4"
SECONDARY = "sgemm_3072x3072x3072_normal_seed2"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sgemm_8192x8192x8192_traffic.txt")
KERNEL_SOURCES = ["sgemm_mfma.hpp", "sgemm_mfma_dl.hpp", "common.hpp"]


def kernel_code(text):
    """Kernel source with // comments and blank lines removed: what the
    counters depend on (editing a comment does not change the kernel)."""
    lines = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code.strip():
            lines.append(code)
    return "\n".join(lines)


def kernel_source_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp32_gemm_sgemm_amd", "csrc", name)) as f:
            h.update(kernel_code(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE,
    if they were taken on the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# Bytes written between timed steps with --cold: twice the 256 MB last-level
# cache (MALL), so no operand byte stays cached from the previous step.
COLD_FLUSH_BYTES = 512 << 20


def time_workload(torch, sg, w, steps, warmup, cfg=None, cold=False):
    from fp32_gemm_sgemm_amd import inputs
    A_np, B_np = inputs.workload_operands(w)
    A = torch.from_numpy(A_np).to("cuda")
    B = torch.from_numpy(B_np).to("cuda")
    C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    flush = torch.empty(COLD_FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") \
        if cold else None
    for _ in range(warmup):
        sg.sgemm(A, B, out=C, stream=stream, cfg=cfg)
    torch.cuda.synchronize()
    # the timed region: `steps` calls back to back between two synchronisations,
    # one event pair around all of them (events between the calls would put a
    # barrier packet between the kernels); with --cold each step is bracketed
    # by its own events instead, so that the cache flush stays outside them
    region_ms, wall_s = None, None
    if flush is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            sg.sgemm(A, B, out=C, stream=stream, cfg=cfg)
        e1.record(stream)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - t0
        region_ms = e0.elapsed_time(e1)
    # the per-step distribution: a second pass of `steps` calls, each between
    # its own pair of events
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush.fill_(float(i))  # outside the step's events
        starts[i].record(stream)
        sg.sgemm(A, B, out=C, stream=stream, cfg=cfg)
        ends[i].record(stream)
    torch.cuda.synchronize()
    if wall_s is None:
        wall_s = time.perf_counter() - t0
        region_ms = starts[0].elapsed_time(ends[-1])
    del flush
    per_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return {
        "A": A_np, "B": B_np, "C": C,
        "region_ms": region_ms, "wall_s": wall_s,
        "mean_ms": sum(per_ms) / len(per_ms), "min_ms": per_ms[0],
        "median_ms": per_ms[len(per_ms) // 2], "p90_ms": per_ms[min(len(per_ms) - 1, int(0.9 * len(per_ms)))],
    }


_SLEEP_CYCLES = [0]


def _queue_ahead(torch, ms=3.0):
    """Enqueue a GPU sleep of about `ms` so that the launches queued after it
    start back to back: the host's per-call cost (Python, ctypes, argument
    checks) then does not pace small kernels."""
    if not _SLEEP_CYCLES[0]:
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(10 ** 5)
        e0.record(s)
        torch.cuda._sleep(10 ** 6)
        e1.record(s)
        torch.cuda.synchronize()
        _SLEEP_CYCLES[0] = max(1, int(10 ** 6 / max(e0.elapsed_time(e1), 1e-3)))
    torch.cuda._sleep(int(_SLEEP_CYCLES[0] * ms))


def time_calls(torch, fn, steps, warm_ms, min_steps=20):
    """GPU time per call of fn() on the current stream, after at least warm_ms
    of warm-up calls.  Two passes, each queued behind a GPU sleep:
      mean_ms  HIP events around max(steps, min_steps) back-to-back calls,
               divided by the count (the throughput figure);
      median_ms, min_ms, p90_ms  over per-call HIP event pairs of a second
               pass of the same length (each pair brackets one call)."""
    n = max(steps, min_steps)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(max(3, int(warm_ms / one))):
        fn()
    torch.cuda.synchronize()
    _queue_ahead(torch, min(20.0, 0.02 * n + 1.0))
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / n
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    _queue_ahead(torch, min(20.0, 0.03 * n + 1.0))
    for i in range(n):
        ev[2 * i].record(stream)
        fn()
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n))
    return {"mean_ms": mean, "median_ms": per[n // 2], "min_ms": per[0],
            "p90_ms": per[min(n - 1, int(0.9 * n))], "calls": n}


def time_call(torch, fn, steps, warm_ms):
    """Mean ms per call of fn() (see time_calls)."""
    return time_calls(torch, fn, steps, warm_ms)["mean_ms"]


def _timing_fields(t):
    return {k: round(t[k], 5) for k in ("median_ms", "min_ms", "p90_ms")}


CONFIG_WORKLOADS = [
    "sgemm_512x512x512_uniform_seed0",
    "sgemm_2048x2048x2048_uniform_seed1",
    "sgemm_2048x2048x2048_identityA_seed1",
    "sgemm_3072x3072x3072_normal_seed2",
    "sgemm_8192x8192x4096_uniform_seed3",
    "sgemm_4096x4096x8192_uniform_seed3",
    "sgemm_4099x4099x4099_uniform_seed3",
    "sgemm_8192x8192x8192_uniform_seed4",
]


def configs(torch, sg, steps, warm_ms, cus, peak, checker=None):
    """TFLOP/s of each workload configuration through sgemm_f32, with the
    distribution of per-call times (at least 20 calls, 100 at the small
    512^3).  `checker(w, A_np, B_np, C)`, when given, returns the accuracy
    block of one configuration (the CPU-reference leg, cpu_config_check)."""
    from fp32_gemm_sgemm_amd import inputs
    out = []
    stream = torch.cuda.current_stream()
    for name in CONFIG_WORKLOADS:
        w = inputs.WORKLOADS[name]
        A_np, B_np = inputs.workload_operands(w)
        A = torch.from_numpy(A_np).to("cuda")
        B = torch.from_numpy(B_np).to("cuda")
        C = torch.empty((w.M, w.N), device="cuda")
        h = stream.cuda_stream

        def call():
            code = sg.sgemm_f32(w.M, w.N, w.K, A.data_ptr(), w.K, B.data_ptr(), w.N,
                                C.data_ptr(), w.N, h)
            if code != 0:
                raise RuntimeError(f"sgemm_f32 failed with hipError_t {code}")
        t = time_calls(torch, call, steps, warm_ms, min_steps=100 if w.flops < 1e9 else 20)
        ms = t["mean_ms"]
        plan = sg.sgemm_f32_plan(w.M, w.N, w.K, w.K, w.N, w.N, cus)
        tf = w.flops / (ms * 1e-3) / 1e12
        entry = dict(workload=name, value=round(tf, 3), unit="TFLOP/s", ms=round(ms, 5),
                     **_timing_fields(t), calls=t["calls"],
                     frac_of_fp32_matrix_peak=round(tf / peak, 4), variant=plan.id,
                     tile=f"{plan.bm}x{plan.bn}x{plan.bk}",
                     strips=[plan.strip_m, plan.strip_n])
        if checker is not None:
            torch.cuda.synchronize()
            entry["check"] = checker(w, A_np, B_np, C)
        out.append(entry)
        del A, B, C, A_np, B_np
    torch.cuda.empty_cache()
    return out


def extras(torch, sg, steps, warm_ms, cus, peak):
    """Throughput of the split-K, transposed-layout and batched paths."""
    from fp32_gemm_sgemm_amd import inputs
    out = []
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)

    def operand(shape):
        return torch.rand(shape, device="cuda", generator=gen) * 2 - 1

    def chk(code):
        if code != 0:
            raise RuntimeError(f"libsgemm call failed with hipError_t {code}")

    def record(name, flops, ms, plan, **kw):
        tf = flops / (ms * 1e-3) / 1e12
        out.append(dict(name=name, value=round(tf, 3), unit="TFLOP/s", ms=round(ms, 5),
                        frac_of_fp32_matrix_peak=round(tf / peak, 4), variant=plan.id,
                        tile=f"{plan.bm}x{plan.bn}x{plan.bk}" if plan.grid else "none",
                        splits=plan.splits,
                        strips=[plan.strip_m, plan.strip_n], **kw))

    # K split across workgroups: the small configuration and one tile with long K
    w = inputs.WORKLOADS["sgemm_512x512x512_uniform_seed0"]
    A_np, B_np = inputs.workload_operands(w)
    for name, (A, B) in [("512x512x512 (seed 0)", (torch.from_numpy(A_np).cuda(),
                                                     torch.from_numpy(B_np).cuda())),
                         ("128x128x32768", (operand((128, 32768)), operand((32768, 128))))]:
        M, K = A.shape
        N = B.shape[1]
        C = torch.empty((M, N), device="cuda")
        wsb = sg.sgemm_f32_workspace_size(0, 0, M, N, K, K, N, N, 1)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        h = stream.cuda_stream
        plan_ws = sg.sgemm_f32_plan(M, N, K, K, N, N, cus, 0, 0, 1, wsb)
        plan_no = sg.sgemm_f32_plan(M, N, K, K, N, N, cus)
        ms_no = time_call(torch, lambda: chk(sg.sgemm_f32(M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                                      C.data_ptr(), N, h)), steps, warm_ms)
        ms_ws = time_call(torch, lambda: chk(sg.sgemm_f32_gemm(0, 0, M, N, K, 1.0, A.data_ptr(), K,
                                                           B.data_ptr(), N, 0.0, C.data_ptr(), N,
                                                           ws.data_ptr(), wsb, h)), steps, warm_ms)
        flops = 2.0 * M * N * K
        record(f"{name} sgemm_f32 (no workspace)", flops, ms_no, plan_no)
        record(f"{name} with workspace", flops, ms_ws, plan_ws, workspace_bytes=wsb,
               speedup=round(ms_no / ms_ws, 3))
        del A, B, C, ws

    # the tiles that split K inside the workgroup (32 x 32 and 16 x 16 MFMA
    # tiles over 8 waves, 8 x 8 vector-FMA tiles over lane pairs and 4 waves),
    # each forced, on the one-tile long-K product in every layout
    forms = {(32, 32, 8, 8), (16, 16, 16, 8), (8, 8, 32, 4)}
    ksplit = [i for i in range(sg.sgemm_f32_num_variants())
              if (sg.sgemm_f32_variant(i).bm, sg.sgemm_f32_variant(i).bn, sg.sgemm_f32_variant(i).bk,
                  sg.sgemm_f32_variant(i).waves_m) in forms]
    M = N = 128
    K = 32768
    for ta, tb in ((0, 0), (1, 0), (0, 1), (1, 1)):
        A = operand((K, M) if ta else (M, K))
        B = operand((N, K) if tb else (K, N))
        C = torch.empty((M, N), device="cuda")
        lda, ldb = A.shape[1], B.shape[1]
        lay = ("T" if ta else "N") + ("T" if tb else "N")
        h = stream.cuda_stream
        for vid in ksplit:
            cfg = sg.SgemmCfg()
            cfg.id, cfg.group_m, cfg.xcd_remap, cfg.splits = vid, 8, 1, 1
            plan = sg.sgemm_f32_cfg_geometry(cfg, ta, tb, M, N, K, lda, ldb, N)
            ms = time_call(torch, lambda: chk(sg.sgemm_f32_ex(ta, tb, M, N, K, 1.0, A.data_ptr(), lda, 0,
                                                          B.data_ptr(), ldb, 0, 0.0, C.data_ptr(), N, 0,
                                                          1, 0, 0, h, cfg)), steps, warm_ms)
            record(f"128x128x32768 {lay} forced K-split tile v{vid}", 2.0 * M * N * K, ms, plan)
        del A, B, C
    torch.cuda.empty_cache()

    # transposed operands (loaded as stored)
    for n in (8192, 3072):
        for ta, tb in ((1, 0), (0, 1), (1, 1)):
            A = operand((n, n))
            B = operand((n, n))
            C = torch.empty((n, n), device="cuda")
            plan = sg.sgemm_f32_plan(n, n, n, n, n, n, cus, ta, tb)
            h = stream.cuda_stream
            ms = time_call(torch, lambda: chk(sg.sgemm_f32_gemm(ta, tb, n, n, n, 1.0, A.data_ptr(), n,
                                                            B.data_ptr(), n, 0.0, C.data_ptr(), n,
                                                            0, 0, h)), steps, warm_ms)
            lay = ("T" if ta else "N") + ("T" if tb else "N")
            record(f"{n}^3 {lay}", 2.0 * n ** 3, ms, plan)
            del A, B, C
    torch.cuda.empty_cache()

    # the vector-FMA comparison kernel (the register-blocked design carried to
    # 64-wide waves), forced, on the two shapes the metric names; its bound is
    # the vector-ALU rate, reported beside it as frac_of_valu_probe
    valu = next(i for i in range(sg.sgemm_f32_num_variants())
                if sg.sgemm_f32_variant(i).kernel == sg.SGEMM_KERNEL_VALU)
    for n in (8192, 3072):
        A, B = operand((n, n)), operand((n, n))
        C = torch.empty((n, n), device="cuda")
        cfg = sg.SgemmCfg()
        cfg.id, cfg.group_m, cfg.xcd_remap, cfg.splits = valu, 8, 1, 1
        plan = sg.sgemm_f32_cfg_geometry(cfg, 0, 0, n, n, n, n, n, n)
        h = stream.cuda_stream
        ms = time_call(torch, lambda: chk(sg.sgemm_f32_ex(0, 0, n, n, n, 1.0, A.data_ptr(), n, 0,
                                                      B.data_ptr(), n, 0, 0.0, C.data_ptr(), n, 0,
                                                      1, 0, 0, h, cfg)), steps, warm_ms)
        record(f"valu comparison {n}^3 (forced vector-FMA kernel)", 2.0 * n ** 3, ms, plan,
               kernel="valu_fma")
        del A, B, C
    torch.cuda.empty_cache()

    # strided batches: per-head products of attention (sequence 1024, head 128)
    for name, batch, M, N, K, ta, tb in [("64 x QK^T 1024x1024x128 NT", 64, 1024, 1024, 128, 0, 1),
                                         ("64 x PV 1024x128x1024 NN", 64, 1024, 128, 1024, 0, 0)]:
        A = operand((batch,) + ((K, M) if ta else (M, K)))
        B = operand((batch,) + ((N, K) if tb else (K, N)))
        C = torch.empty((batch, M, N), device="cuda")
        lda, ldb = A.shape[2], B.shape[2]
        wsb = sg.sgemm_f32_workspace_size(ta, tb, M, N, K, lda, ldb, N, batch)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        plan = sg.sgemm_f32_plan(M, N, K, lda, ldb, N, cus, ta, tb, batch, wsb)
        h = stream.cuda_stream
        ms = time_call(torch, lambda: chk(sg.sgemm_f32_strided_batched(
            ta, tb, M, N, K, 1.0, A.data_ptr(), lda, A.stride(0), B.data_ptr(), ldb, B.stride(0),
            0.0, C.data_ptr(), N, C.stride(0), batch, ws.data_ptr(), wsb, h)), steps, warm_ms)
        record(name, 2.0 * batch * M * N * K, ms, plan, batch=batch)
        del A, B, C, ws
    torch.cuda.empty_cache()

    # one GPU's share of 8192^3 split by rows of C over 8 GPUs (a 1024-row band
    # of A times all of B), the shape each GPU would run in a row-band sharding;
    # and 1024^3, one 64x64 tile per CU
    for name, M, N, K in [("row-band shard 1024x8192x8192 (8192^3 over 8 GPUs)", 1024, 8192, 8192),
                          ("1024^3", 1024, 1024, 1024)]:
        A, B = operand((M, K)), operand((K, N))
        C = torch.empty((M, N), device="cuda")
        plan = sg.sgemm_f32_plan(M, N, K, K, N, N, cus)
        h = stream.cuda_stream
        ms = time_call(torch, lambda: chk(sg.sgemm_f32(M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                                    C.data_ptr(), N, h)), steps, warm_ms)
        record(name, 2.0 * M * N * K, ms, plan)
        del A, B, C
    torch.cuda.empty_cache()

    # outputs between one and three rounds of 64x64 tiles (or fewer 32x32
    # tiles than CUs), which the selector gives 32x64 tiles, three per CU:
    # the default plan, and forced beside it the tile it would use without them
    for M, N, K, before in [(1536, 1024, 4096, 20), (1024, 384, 1024, 16), (3072, 384, 4096, 16)]:
        A, B = operand((M, K)), operand((K, N))
        C = torch.empty((M, N), device="cuda")
        h = stream.cuda_stream
        plan = sg.sgemm_f32_plan(M, N, K, K, N, N, cus)
        ms = time_call(torch, lambda: chk(sg.sgemm_f32(M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                                    C.data_ptr(), N, h)), steps, warm_ms)
        cfg = sg.SgemmCfg()
        cfg.id, cfg.group_m, cfg.xcd_remap, cfg.splits = before, 8, 1, 1
        plan_b = sg.sgemm_f32_cfg_geometry(cfg, 0, 0, M, N, K, K, N, N)
        ms_b = time_call(torch, lambda: chk(sg.sgemm_f32_ex(0, 0, M, N, K, 1.0, A.data_ptr(), K, 0,
                                                         B.data_ptr(), N, 0, 0.0, C.data_ptr(), N, 0,
                                                         1, 0, 0, h, cfg)), steps, warm_ms)
        record(f"{M}x{N}x{K}", 2.0 * M * N * K, ms, plan)
        record(f"{M}x{N}x{K} forced v{before}", 2.0 * M * N * K, ms_b, plan_b,
               default_speedup=round(ms_b / ms, 3))
        del A, B, C
    torch.cuda.empty_cache()

    # edge strips: a few rows or columns past the last full tile, and products
    # of at most 4 rows (the strip kernel alone; reported with its HBM rate:
    # the streamed operand's bytes over the call time)
    for name, M, N, K in [("8196x8192x8192 (4-row edge strip)", 8196, 8192, 8192),
                          ("2051^3 (3-row and 3-column strips, ld 2051)", 2051, 2051, 2051),
                          ("513x8192x1023 (lda 1023)", 513, 8192, 1023),
                          ("1x8192x8192 (vector-shaped)", 1, 8192, 8192),
                          ("8192x1x8192 (vector-shaped)", 8192, 1, 8192)]:
        A, B = operand((M, K)), operand((K, N))
        C = torch.empty((M, N), device="cuda")
        plan = sg.sgemm_f32_plan(M, N, K, K, N, N, cus)
        h = stream.cuda_stream
        ms = time_call(torch, lambda: chk(sg.sgemm_f32(M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                                    C.data_ptr(), N, h)), steps, warm_ms)
        kw = {}
        if plan.grid == 0:
            kw["GB_per_s"] = round(4.0 * K * max(M, N) / (ms * 1e-3) / 1e9, 1)
        record(name, 2.0 * M * N * K, ms, plan, **kw)
        del A, B, C
    torch.cuda.empty_cache()
    return out


def vendor(torch, steps, warm_ms, peak):
    """torch.matmul (rocBLAS / hipBLASLt) in float32 on the same shapes, and
    torch.bmm on the two batched attention products, for context."""
    out = []
    torch.backends.cuda.matmul.allow_tf32 = False

    def rec(shape, flops, ms):
        tf = flops / (ms * 1e-3) / 1e12
        out.append(dict(shape=shape, value=round(tf, 3), unit="TFLOP/s", ms=round(ms, 5),
                        frac_of_fp32_matrix_peak=round(tf / peak, 4)))

    for n in (8192, 3072, 4096, 2048, 1024, 512):
        A = torch.rand((n, n), device="cuda") * 2 - 1
        B = torch.rand((n, n), device="cuda") * 2 - 1
        C = torch.empty((n, n), device="cuda")
        rec(f"{n}^3", 2.0 * n ** 3, time_call(torch, lambda: torch.matmul(A, B, out=C), steps, warm_ms))
        del A, B, C
    # float32 operands: B of the NT product is passed as a transposed view
    for shape, batch, M, N, K, tb in [("64 x QK^T 1024x1024x128 NT (torch.bmm)", 64, 1024, 1024, 128, 1),
                                      ("64 x PV 1024x128x1024 NN (torch.bmm)", 64, 1024, 128, 1024, 0)]:
        A = torch.rand((batch, M, K), device="cuda") * 2 - 1
        B = torch.rand((batch, N, K) if tb else (batch, K, N), device="cuda") * 2 - 1
        Bv = B.transpose(1, 2) if tb else B
        C = torch.empty((batch, M, N), device="cuda")
        rec(shape, 2.0 * batch * M * N * K,
            time_call(torch, lambda: torch.bmm(A, Bv, out=C), steps, warm_ms))
        del A, B, Bv, C
    # one 128 x 128 output with K = 32768 in every layout (a transposed
    # operand passed as a transposed view of its stored form)
    M = N = 128
    K = 32768
    for ta, tb in ((0, 0), (1, 0), (0, 1), (1, 1)):
        A = torch.rand((K, M) if ta else (M, K), device="cuda") * 2 - 1
        B = torch.rand((N, K) if tb else (K, N), device="cuda") * 2 - 1
        Av, Bv = (A.t() if ta else A), (B.t() if tb else B)
        C = torch.empty((M, N), device="cuda")
        lay = ("T" if ta else "N") + ("T" if tb else "N")
        rec(f"128x128x32768 {lay}", 2.0 * M * N * K,
            time_call(torch, lambda: torch.matmul(Av, Bv, out=C), steps, warm_ms))
        del A, B, Av, Bv, C
    torch.cuda.empty_cache()
    return out


def host_cores():
    """Cores of this host: all of them, and the ones this process may use."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        affinity = os.cpu_count() or 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"os_cpu_count": os.cpu_count(), "affinity": affinity, "model": model}


def cpu_baseline(w, A_np, B_np, C_gpu, seconds):
    """The CPU reference on whole rows of the same product, about `seconds` of
    work; its rows are also checked against the GPU result."""
    import numpy as np
    import oracle
    nt = oracle.default_threads()
    rows = 0
    spent = 0.0
    n_bad = 0
    max_err = 0.0
    sq_err = sq_ref = 0.0
    while rows < w.M and (spent < seconds or rows == 0):
        r1 = min(w.M, rows + nt)
        t0 = time.perf_counter()
        ref, absb = oracle.sgemm_ref(A_np[rows:r1], B_np, nthreads=nt)
        spent += time.perf_counter() - t0
        rep = oracle.compare(C_gpu[rows:r1], ref, absb)
        n_bad += rep["n_bad"]
        max_err = max(max_err, rep["max_norm_err"])
        sq_err += float(np.sum((C_gpu[rows:r1].astype(np.float64) - ref) ** 2))
        sq_ref += float(np.sum(ref * ref))
        rows = r1
    flops = 2.0 * rows * w.N * w.K
    # the same reference on one thread, over whole rows for about a sixth as long
    rows1, spent1 = 0, 0.0
    while rows1 < w.M and (spent1 < seconds / 6 or rows1 == 0):
        t0 = time.perf_counter()
        oracle.sgemm_ref(A_np[rows1:rows1 + 1], B_np, nthreads=1)
        spent1 += time.perf_counter() - t0
        rows1 += 1
    flops1 = 2.0 * rows1 * w.N * w.K
    return {
        "value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": nt, "kind": "oracle",
        "threads": nt, "host_cores": host_cores(),
        "sample": f"rows 0..{rows - 1} of C ({rows} x {w.N} outputs, K = {w.K}, "
                  f"{flops / 1e9:.1f} GFLOP) in {spent:.1f} s on {nt} threads",
        "single_thread": {"value": flops1 / spent1 / 1e12, "unit": "TFLOP/s",
                          "sample": f"rows 0..{rows1 - 1} in {spent1:.1f} s"},
        "check": {"n": rows * w.N, "n_bad": n_bad, "max_norm_err": max_err,
                  "rrmse": (sq_err / sq_ref) ** 0.5 if sq_ref > 0 else 0.0,
                  "tol": oracle.TOL},
    }


def cpu_config_check(w, A_np, B_np, C):
    """Part of the CPU-reference leg: the accuracy of one configuration's GPU
    result against the CPU reference.  Full comparison when the workload asks
    for it (512^3, and the identity-A run, which must also equal B exactly);
    otherwise the seeded sample of 4096 outputs (3584 uniform, 512 from the
    256-wide edge band), plus every element of the last 3 rows and columns for
    the ragged 4099^3."""
    import numpy as np
    import oracle
    from fp32_gemm_sgemm_amd import inputs
    import torch
    t0 = time.perf_counter()
    out = {}
    if w.check == "full":
        C_np = C.cpu().numpy()
        ref, absb = oracle.sgemm_ref(A_np, B_np)
        rep = oracle.compare(C_np, ref, absb)
        out["mode"] = "full"
        if w.variant == "identity":
            out["exact_equal_B"] = bool(np.array_equal(C_np, B_np))
    else:
        last = 3 if w.M % 4 or w.N % 4 else 0
        rows, cols = inputs.sample_indices(w.M, w.N, w.seed, last=last)
        vals = C[torch.from_numpy(rows).to(C.device), torch.from_numpy(cols).to(C.device)]
        ref, absb = oracle.sgemm_ref_sampled(A_np, B_np, rows, cols)
        rep = oracle.compare(vals.cpu().numpy(), ref, absb)
        out["mode"] = "sampled 4096 (3584 uniform + 512 edge band)" + \
            (f", last {last} rows and columns in full" if last else "")
    out.update({k: rep[k] for k in ("n", "n_bad", "max_norm_err", "rrmse")})
    out["tol"] = oracle.TOL
    out["cpu_s"] = round(time.perf_counter() - t0, 3)
    return out


def run_meta(torch):
    """Where the numbers were taken: device, runtime and toolchain versions,
    host (the workbook's rule for trustworthy timings: name the GPU, driver,
    toolkit and power mode)."""
    import ctypes
    import subprocess
    p = torch.cuda.get_device_properties(0)
    meta = {"device": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "hbm_bytes": p.total_memory, "torch": torch.__version__,
            "torch_hip": torch.version.hip}
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
        v = ctypes.c_int(0)
        if hip.hipRuntimeGetVersion(ctypes.byref(v)) == 0:
            meta["hip_runtime_version"] = v.value
        if hip.hipDriverGetVersion(ctypes.byref(v)) == 0:
            meta["hip_driver_version"] = v.value
    except OSError:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            meta["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        r = subprocess.run(["/opt/rocm/bin/hipcc", "--version"], capture_output=True,
                           text=True, timeout=30)
        meta["hipcc"] = " | ".join(l.strip() for l in r.stdout.splitlines()
                                   if "version" in l.lower())[:300]
    except (OSError, subprocess.SubprocessError):
        pass
    for card in sorted(os.listdir("/sys/class/drm")) if os.path.isdir("/sys/class/drm") else []:
        path = f"/sys/class/drm/{card}/device/power_dpm_force_performance_level"
        if card.startswith("card") and "-" not in card and os.path.exists(path):
            try:
                with open(path) as f:
                    meta["power_dpm_force_performance_level"] = f.read().strip()
                break
            except OSError:
                pass
    meta["host"] = host_cores()
    return meta


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--secondary", default=SECONDARY, help="'' to skip")
    ap.add_argument("--secondary-warm-ms", type=float, default=200.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variant", type=int, default=-1, help="force a compiled variant id")
    ap.add_argument("--group-m", type=int, default=8)
    ap.add_argument("--xcd-remap", type=int, default=1)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing every workload configuration")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the torch.matmul context measurement")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the split-K, transposed-layout and batched measurements")
    ap.add_argument("--extra-warm-ms", type=float, default=150.0)
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the MFMA- and VALU-peak probes (the measured ceilings)")
    ap.add_argument("--cold", action="store_true",
                    help="write 512 MiB between timed steps (no operand left in L2 or MALL); "
                         "the value is then the mean of the per-step event times")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB, a "
                         "known-size kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library has no multi-GPU path.", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import fp32_gemm_sgemm_amd as sg
    from fp32_gemm_sgemm_amd import inputs, metrics
    if not os.path.exists(sg.LIB_PATH):
        from fp32_gemm_sgemm_amd import build
        build.build()
    sg.load()

    cfg = None
    if args.variant >= 0:
        cfg = sg.SgemmCfg()
        cfg.id, cfg.group_m, cfg.xcd_remap = args.variant, args.group_m, args.xcd_remap

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = inputs.WORKLOADS[args.workload]
    r = time_workload(torch, sg, w, args.steps, args.warmup, cfg, cold=args.cold)
    flops = w.flops
    # (with --cold the region also holds the cache flushes between steps)
    ms_per_step = r["mean_ms"] if args.cold else r["region_ms"] / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (r["mean_ms"] * 1e-3) / 1e12
    peak = metrics.MI355X_FP32_MATRIX_PEAK_TFLOPS
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plan = sg.sgemm_f32_plan(w.M, w.N, w.K, w.K, w.N, w.N, cus) \
        if cfg is None else sg.sgemm_f32_variant(cfg.id)

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "M": w.M, "N": w.N, "K": w.K, "layout": "row-major",
            "inputs": f"{w.dist} seed {w.seed}",
            "variant": plan.id, "tile": f"{plan.bm}x{plan.bn}x{plan.bk}",
            "waves": f"{plan.waves_m}x{plan.waves_n}",
            "kernel": "mfma_f32_32x32x2" if plan.kernel == 0 else "valu_fma",
            "parallelism": "single GPU",
            "cache": "cold" if args.cold else "warm",
        },
        "frac_of_fp32_matrix_peak": round(value / peak, 4),
        "timing_ms": {k: round(r[k], 4) for k in ("mean_ms", "median_ms", "min_ms", "p90_ms")},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": read_traffic() if w.name == HEADLINE else None,
            "compulsory_bytes": metrics.compulsory_bytes(w.M, w.N, w.K),
            "kernel_source_sha256_16": kernel_source_hash(),
        },
    }

    if args.secondary:
        w2 = inputs.WORKLOADS[args.secondary]
        # warm-up launches for about --secondary-warm-ms, at the headline's rate
        # scaled by work (never fewer than --warmup)
        est_ms = r["mean_ms"] * w2.flops / flops
        warm2 = max(args.warmup, int(args.secondary_warm_ms / max(est_ms, 1e-3)))
        r2 = time_workload(torch, sg, w2, args.steps, warm2, cfg)
        v2 = w2.flops / (r2["region_ms"] / args.steps * 1e-3) / 1e12
        result["secondary"] = {
            "workload": w2.name, "value": round(v2, 3), "unit": "TFLOP/s",
            "ms_per_step": round(r2["region_ms"] / args.steps, 4),
            "frac_of_fp32_matrix_peak": round(v2 / peak, 4),
            "mean_kernel_ms": round(r2["mean_ms"], 4),
            "warmup": warm2,
        }
        del r2

    if not args.no_configs:
        result["configs"] = configs(torch, sg, args.steps, args.extra_warm_ms, cus, peak,
                                    checker=None if args.no_cpu_baseline else cpu_config_check)
    if not args.no_extras:
        result["extras"] = extras(torch, sg, args.steps, args.extra_warm_ms, cus, peak)
    if not args.no_vendor:
        result["vendor"] = vendor(torch, args.steps, args.extra_warm_ms, peak)

    if not args.no_probe:
        from fp32_gemm_sgemm_amd import probes
        ceil = probes.mfma_peak_tflops()
        result["mfma_probe"] = {
            "tflops": round(ceil, 3),
            "frac_of_published_peak": round(ceil / peak, 4),
            "gemm_frac_of_probe": round(value / ceil, 4),
            "what": "sustained v_mfma_f32_32x32x2_f32 rate, register operands only",
        }
        vceil = probes.valu_peak_tflops()
        result["valu_probe"] = {
            "tflops": round(vceil, 3),
            "frac_of_published_peak": round(vceil / peak, 4),
            "what": "sustained non-packed v_fma_f32 rate, register operands only (the "
                    "instruction of the vector-FMA comparison kernel)",
        }
        for e in result.get("extras", []):
            if e.get("kernel") == "valu_fma":
                e["frac_of_valu_probe"] = round(e["value"] / vceil, 4)
        # the floor of a launch with the small products' grid: 256 empty
        # workgroups of 512 threads, timed like the configurations
        t = time_calls(torch, probes.empty_launch(256), args.steps, args.extra_warm_ms,
                       min_steps=100)
        result["launch_floor"] = {
            "mean_ms": round(t["mean_ms"], 5), **_timing_fields(t),
            "what": "empty launch of 256 workgroups x 512 threads (the 512^3 grid), HIP "
                    "events like configs: back-to-back mean and per-call distribution",
        }

    if not args.no_cpu_baseline:
        C_host = r["C"].cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(w, r["A"], r["B"], C_host, args.cpu_seconds)

    # the metric's two figures: 8192^3 is `value` (the timed steps above),
    # 3072^3 is `secondary` (the same protocol); the configs entries of those
    # shapes are the same products timed by the per-configuration protocol
    result["metric_figures"] = {
        "8192^3": {"value": result["value"], "from": "value"},
        "3072^3": ({"value": result["secondary"]["value"], "from": "secondary"}
                   if "secondary" in result and args.secondary == SECONDARY else None),
    }
    result["meta"] = run_meta(torch)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
