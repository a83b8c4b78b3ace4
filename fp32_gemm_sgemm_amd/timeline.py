"""Where the direct-load kernel's time goes, from the timeline build
(libsgemm_timeline.so; its functions are declared in include/sgemm_timeline.h).

    python -m fp32_gemm_sgemm_amd.timeline [--out FILE]
        [--shape M N K [VARIANT [BATCH [TRANSA TRANSB]]]] ...

For each product (the default plan without a workspace, or a forced variant;
VARIANT -1 is the default plan; BATCH > 1 is a strided batch of packed
matrices; TRANSA, TRANSB 1 pass that operand stored transposed) one call is
measured after identical calls have kept the GPU busy for 200 ms (the chip
needs about 0.1 s of load to reach its full clock).  Per workgroup: the
shader-clock cycles of the prologue (entry until the first slice has landed in
LDS), of the main loop and of the stores of C, against the loop's ideal, the
cycles its MFMAs take at the FP32 matrix rate (256 FLOP per cycle per compute
unit: 157.3 TFLOP/s over 256 CUs at 2.4 GHz); from the device's real-time
counter, each workgroup's shader-clock rate and when it started and ended
against the call's first start (the call's span).  Per K slice, over the first
workgroups: the period from one slice's last wave arrival at the barrier to
the next, how long a wave waits for its own loads of the next slice, and how
long it then waits at the barrier for the other waves.

Needs a GPU.  The timeline build computes the same results as libsgemm.so:
its readings add a few scalar instructions per slice and none to the
arithmetic.
"""
import argparse
import ctypes
import json
import sys
import time

import numpy as np

from . import binding

FLOP_PER_CYCLE_PER_CU = 256  # 157.3e12 / (256 CUs * 2.4e9 cycles/s)

DEFAULT_SHAPES = [  # (M, N, K[, variant, batch, transa, transb]): the benchmark's shapes
    (8192, 8192, 8192), (8192, 8192, 4096), (4096, 4096, 8192), (3072, 3072, 3072),
    (2048, 2048, 2048), (1024, 1024, 1024), (4099, 4099, 4099),
    (1024, 1024, 128, -1, 64, 0, 1), (1024, 128, 1024, -1, 64, 0, 0),
]


def layout(lib):
    vals = [ctypes.c_int() for _ in range(4)]
    binding._check(lib.sgemm_f32_timeline_layout(*[ctypes.byref(v) for v in vals]),
                   "sgemm_f32_timeline_layout")
    return tuple(v.value for v in vals)  # phase_wgs, slice_wgs, waves, slices


def clock_khz(lib):
    """Rate of the real-time counter (kHz)."""
    v = ctypes.c_int()
    binding._check(lib.sgemm_f32_timeline_clock_khz(ctypes.byref(v)), "sgemm_f32_timeline_clock_khz")
    return v.value


def read(lib):
    """(phase[wg, 6] uint64, slice[wg, wave, slice, 2] uint32) of the build."""
    phase_wgs, slice_wgs, waves, slices = layout(lib)
    phase = np.zeros((phase_wgs, 6), np.uint64)
    sl = np.zeros((slice_wgs, waves, slices, 2), np.uint32)
    binding._check(lib.sgemm_f32_timeline_read(phase.ctypes.data, phase.nbytes,
                                               sl.ctypes.data, sl.nbytes),
                   "sgemm_f32_timeline_read")
    return phase, sl


def _q(x, ps=(10, 50, 90)):
    return [int(round(float(np.percentile(x, p)))) for p in ps]


def summarize(cfg, K, phase, sl, khz=0):
    """Statistics of one call's readings for the plan `cfg` (khz: the
    real-time counter's rate; 0 skips the real-time figures)."""
    nwg = min(cfg.grid, phase.shape[0])
    ph = phase[:nwg].astype(np.int64)
    ph = ph[ph[:, 0] != 0]
    kk = cfg.k_chunk if cfg.splits > 1 else K
    nk = -(-kk // cfg.bk)
    ideal = cfg.bm * cfg.bn * nk * cfg.bk * 2 / FLOP_PER_CYCLE_PER_CU
    if not len(ph):  # a plan on another kernel: no readings
        return {"workgroups": 0, "slices": nk}
    pro, loop, epi = ph[:, 1] - ph[:, 0], ph[:, 2] - ph[:, 1], ph[:, 3] - ph[:, 2]
    out = {
        "workgroups": int(len(ph)), "slices": nk,
        "prologue": _q(pro), "loop": _q(loop), "stores": _q(epi), "total": _q(ph[:, 3] - ph[:, 0]),
        "loop_ideal": int(round(ideal)),
        "loop_efficiency": round(ideal / float(np.median(loop)), 4),
    }
    if khz > 0 and len(ph) and (ph[:, 5] > ph[:, 4]).all():
        us = 1e3 / khz  # microseconds per real-time tick
        t0 = ph[:, 4].min()
        span = (ph[:, 5] - ph[:, 4]) * us
        out.update(
            clock_ghz=[round(float(v), 3) for v in np.percentile(
                (ph[:, 3] - ph[:, 0]) / (span * 1e3), (10, 50, 90))],
            call_span_us=round(float((ph[:, 5].max() - t0) * us), 2),
            start_us=[round(float(v), 2) for v in np.percentile((ph[:, 4] - t0) * us, (50, 90, 100))],
            end_us=[round(float(v), 2) for v in np.percentile((ph[:, 5] - t0) * us, (0, 50, 100))])
    waves = cfg.threads // 64
    ns = min(nk, sl.shape[2])
    per, own, bar = [], [], []
    for w in range(min(nwg, sl.shape[0])):
        t = sl[w, :waves, :ns].astype(np.int64)
        if not t.any():
            continue
        t0, t1 = t[..., 0], t[..., 1]
        # 32-bit counts: differences modulo 2^32, read as signed
        rel = ((t1 - t1[0, 0] + (1 << 31)) % (1 << 32)) - (1 << 31)
        last = rel.max(axis=0)  # the last wave's arrival at each barrier
        per += list(np.diff(last))
        own += list(((t1 - t0) % (1 << 32)).ravel())
        bar += list((last[None, :] - rel).ravel())
    if per:
        out.update(slice_period=_q(per), slice_ideal=int(round(ideal / nk)),
                   wait_own_loads=_q(own), wait_barrier=_q(bar))
    return out


def measure(M, N, K, variant=None, warm_ms=200.0, seed=0, batch=1, transa=0, transb=0):
    """Readings of one call through the timeline build (packed row-major
    operands, op(A) M x K and op(B) K x N, `batch` of them; no workspace),
    after identical calls for about warm_ms.  variant None or < 0: the
    default plan."""
    import torch
    lib = binding.load(binding.TIMELINE_LIB_PATH)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    sa, sb = ((K, M) if transa else (M, K)), ((N, K) if transb else (K, N))
    A = torch.rand((batch,) + sa, device="cuda", generator=gen) * 2 - 1
    B = torch.rand((batch,) + sb, device="cuda", generator=gen) * 2 - 1
    C = torch.empty((batch, M, N), device="cuda")
    lda, ldb = sa[1], sb[1]
    st = (A.stride(0), B.stride(0), C.stride(0)) if batch > 1 else (0, 0, 0)
    with binding.library(binding.TIMELINE_LIB_PATH):
        if variant is None or variant < 0:
            cfg = binding.sgemm_f32_query(transa, transb, M, N, K, A.data_ptr(), lda, st[0],
                                          B.data_ptr(), ldb, st[1], C.data_ptr(), N, st[2], batch)
        else:
            cfg = binding.SgemmCfg()
            cfg.id, cfg.group_m, cfg.xcd_remap, cfg.splits = variant, 8, 1, 1
            cfg = binding.sgemm_f32_cfg_geometry(cfg, transa, transb, M, N, K, lda, ldb, N, batch)

        def call():
            binding.sgemm_batched(A, B, out=C, cfg=cfg, transa=transa, transb=transb,
                                  workspace=False)
        end, n = time.perf_counter() + warm_ms / 1e3, 0
        while n < 3 or time.perf_counter() < end:
            call()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()  # keep the queue short: the time is GPU time
        torch.cuda.synchronize()
        binding._check(lib.sgemm_f32_timeline_clear(), "sgemm_f32_timeline_clear")
        call()
        torch.cuda.synchronize()
        phase, sl = read(lib)
        timed_us = call_us(torch, call)
    with binding.library(binding.LIB_PATH):  # the same plan through the normal build
        normal_us = call_us(torch, call, warm_ms)
    return cfg, phase, sl, clock_khz(lib), (normal_us, timed_us)


def call_us(torch, call, warm_ms=0.0, n=50):
    """Mean time of n back-to-back calls (HIP events), after about warm_ms of
    calls."""
    end = time.perf_counter() + warm_ms / 1e3
    while time.perf_counter() < end:
        call()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def report(M, N, K, variant=None, batch=1, transa=0, transb=0):
    cfg, phase, sl, khz, (normal_us, timed_us) = measure(M, N, K, variant, batch=batch,
                                                         transa=transa, transb=transb)
    lay = ("T" if transa else "N") + ("T" if transb else "N")
    r = {"shape": [M, N, K], "batch": batch, "layout": lay, "variant": cfg.id,
         "tile": f"{cfg.bm}x{cfg.bn}x{cfg.bk}",
         "waves": cfg.threads // 64, "grid": cfg.grid, "strips": [cfg.strip_m, cfg.strip_n],
         "call_us_normal": round(normal_us, 2), "call_us_timeline": round(timed_us, 2)}
    r.update(summarize(cfg, K, phase, sl, khz))
    return r


def markdown(rows, command):
    out = ["# Inside the direct-load kernel: prologue, loop and stores (timeline build)", "",
           "Command (from the repository root, on the MI355X; committed files only):", "",
           "```", command, "```", "",
           "One call per product after 200 ms of identical warm-up calls (operands warm in the",
           "caches, the clock ramped up),",
           "default plan without a workspace.  Shader-clock cycles (s_memtime) per workgroup, as",
           "10th / 50th / 90th percentiles over the call's workgroups (at most 4096); the loop's",
           "ideal is its MFMA cycles at 256 FLOP per cycle per CU.  Per-slice figures come from",
           "the first 16 workgroups: the period between the last wave arrivals at two successive",
           "barriers, and per wave the wait for its own loads of the next slice and the wait at",
           "the barrier.  Where several workgroups share a CU (more workgroups than CUs in one",
           "round, when registers and LDS allow it) each one's loop cycles include the others'",
           "share of the matrix cores, so its efficiency reads low.", "",
           "| product | plan | workgroups | prologue | main loop | loop ideal | loop efficiency | stores of C | slice period (ideal) | wait for own loads | wait at barrier |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    f = lambda q: " / ".join(f"{v:,}" for v in q)

    def name(r):
        m = "x".join(map(str, r["shape"]))
        if r["batch"] > 1:
            m = f"{r['batch']} x {m}"
        return m if r["layout"] == "NN" else f"{m} {r['layout']}"
    for r in rows:
        if not r["workgroups"]:
            out.append(f"| {name(r)} | v{r['variant']} {r['tile']} (no readings: not the direct-load "
                       "kernel) | 0 | | | | | | | | |")
            continue
        per = f"{f(r['slice_period'])} ({r['slice_ideal']:,})" if "slice_period" in r else ""
        out.append(
            f"| {name(r)} | v{r['variant']} {r['tile']}, "
            f"{r['waves']} waves, strips {r['strips'][0]}, {r['strips'][1]} | {r['workgroups']} | "
            f"{f(r['prologue'])} | {f(r['loop'])} | {r['loop_ideal']:,} | {r['loop_efficiency']} | "
            f"{f(r['stores'])} | {per} | {f(r.get('wait_own_loads', []))} | "
            f"{f(r.get('wait_barrier', []))} |")
    rt = [r for r in rows if "call_span_us" in r]
    if rt:
        g = lambda q: " / ".join(f"{v:g}" for v in q)
        out += ["", "From the device's real-time counter (microseconds after the call's first",
                "workgroup started; the shader clock's rate is each workgroup's cycles over its",
                "real time), and the mean time of 50 back-to-back calls of the same plan through",
                "the normal build and through the timeline build (the readings' own cost):", "",
                "| product | shader clock GHz (10th / 50th / 90th) | call span us | workgroup starts (median / 90th / last) | workgroup ends (first / median / last) | call us, normal / timeline build |",
                "|---|---|---|---|---|---|"]
        for r in rt:
            cu = (f"{r['call_us_normal']:g} / {r['call_us_timeline']:g}"
                  if "call_us_normal" in r else "")
            out.append(f"| {name(r)} | {g(r['clock_ghz'])} | {r['call_span_us']:g} | "
                       f"{g(r['start_us'])} | {g(r['end_us'])} | {cu} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shape", nargs="+", type=int, action="append",
                    help="M N K [VARIANT [BATCH [TRANSA TRANSB]]] (repeatable; default: the "
                         "benchmark's shapes)")
    ap.add_argument("--out", default=None, help="write a markdown summary here")
    args = ap.parse_args(argv)
    shapes = [tuple(s) for s in args.shape] if args.shape else DEFAULT_SHAPES
    rows = []
    for s in shapes:
        if len(s) not in (3, 4, 5, 7):
            ap.error("--shape takes M N K [VARIANT [BATCH [TRANSA TRANSB]]]")
        print(f"[timeline] {s}", flush=True)
        r = report(*s)
        rows.append(r)
        print(json.dumps(r), flush=True)
    if args.out:
        cmd = "python -m fp32_gemm_sgemm_amd.timeline --out <summary.md>" + "".join(
            " --shape " + " ".join(map(str, s)) for s in (args.shape or []))
        with open(args.out, "w") as fh:
            fh.write(markdown(rows, cmd))
    return 0


if __name__ == "__main__":
    sys.exit(main())
