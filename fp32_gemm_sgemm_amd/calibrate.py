"""Measure the figures the selector's cost model uses, on the GPU at hand.

    python -m fp32_gemm_sgemm_amd.calibrate [--variants 4,6,...] [--ms 150]

First the launch floor: what every launch costs beyond the model (dispatch,
completion, the events), from one-tile products of the small-tile reference
variant.  It is the same for every variant and so left out of the model, and
taken off each measured time below.

For each selectable variant (or the ones listed) three shapes are timed with
the variant forced, no K split and no strips, K = 4096 (4099 for the last):

  full       32 BM x 32 BN      four rounds of full tiles on 256 CUs, rows
                                16-byte aligned
  one        16 BM x 16 BN      one round, one workgroup per CU
  unaligned  (32 BM - 5) x (32 BN - 5), K = 4099: rows not 16-byte aligned

and the cost model of select.hpp,

  t = rounds * (2.5 us + slices * 2 BM BN BK / (614.4 FLOP/ns * eff)),

is inverted for eff (x1000), the three numbers each variant carries in the
table of sgemm.hip (printed at the end as table lines).  With --fit-fixed the
listed variants get their own fixed cost in place of the 2.5 us (fit_fixed),
a fourth number in their table line.  The variants that split K inside the
workgroup (32 x 32, 16 x 16 and 8 x 8 tiles, whose L2 spill the model prices)
also get their own fixed cost and spill factors (one round, several rounds),
and are measured at K where the operands one XCD reads fit in its L2
(calibrate_ksplit); several of their
workgroups share a CU, and the model charges their fixed cost once per wave
of co-resident workgroups.  The strip kernel is timed alone on 4-row products
in both storage orders of its streamed operand: two sizes that fill the chip
give its fixed cost and the chip's streaming rates (kStripFixedNs,
kStripBytesPerNs, kStripBytesPerNsXc), and a narrow product with long K the
rate of one workgroup (kStripWgBytesPerNsXc, kStripWgBytesPerNsKcNarrow).

Each timing is the median of HIP events around single launches queued behind
a GPU sleep, after a time-based warm-up (the chip needs about 0.1 s of load
to reach its clock).
Prints one JSON line per measurement and, at the end, the table lines.
"""
import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

CU_FLOP_PER_NS = 157.3e3 / 256.0
TILE_FIXED_NS = 2500.0
CUS = 256
REF_VARIANT = 11  # 64 x 64 x 32 tiles, direct loads: the launch-floor reference


_SLEEP = [0]


def _sleep_cycles(torch, ms=2.0):
    """GPU sleep cycles for about `ms` milliseconds (measured once)."""
    if not _SLEEP[0]:
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(10 ** 5)
        torch.cuda.synchronize()
        e0.record(s)
        torch.cuda._sleep(10 ** 6)
        e1.record(s)
        torch.cuda.synchronize()
        _SLEEP[0] = int(10 ** 6 * ms / max(e0.elapsed_time(e1), 1e-3))
    return _SLEEP[0]


def _time(torch, fn, warm_ms, reps=15):
    """Median GPU time of one launch of fn (ns).  The timed launches are
    queued behind a GPU sleep, so the host's per-call cost does not pace
    them."""
    torch.cuda.synchronize()
    t0 = time.time()
    while (time.time() - t0) * 1000 < warm_ms:
        fn()
        torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda._sleep(_sleep_cycles(torch))
    ev[0].record(s)
    for i in range(reps):
        fn()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    return t[reps // 2] * 1e6  # ns


def _operands(torch, M, N, K, ld_pad):
    lda, ldb = K + ld_pad, N + ld_pad
    A = torch.empty(M * lda, device="cuda").uniform_(-1, 1).view(M, lda)[:, :K]
    B = torch.empty(K * ldb, device="cuda").uniform_(-1, 1).view(K, ldb)[:, :N]
    C = torch.empty((M, N), device="cuda")
    return A, B, C


def _forced(torch, sg, vid, M, N, K, warm_ms):
    """GPU time (ns) of an M x N x K product with variant vid, no split or strips."""
    A, B, C = _operands(torch, M, N, K, 0)
    cfg = sg.SgemmCfg()
    cfg.id, cfg.group_m, cfg.xcd_remap, cfg.splits = vid, 8, 1, 1
    t = _time(torch, lambda: sg.sgemm(A, B, out=C, cfg=cfg, workspace=False), warm_ms)
    del A, B, C
    return t


def slice_ns(bm, bn, bk, eff):
    return 2.0 * bm * bn * bk / (CU_FLOP_PER_NS * eff / 1000.0)


def eff_from_time(t_ns, bm, bn, bk, M, N, K, fixed_ns=TILE_FIXED_NS, coresident=1):
    """t_ns: the launch's time less the launch floor.  Co-resident workgroups
    pay the fixed cost once per wave of CUS * coresident tiles."""
    tiles = -(-M // bm) * -(-N // bn)
    rounds = -(-tiles // CUS)
    waves = -(-tiles // (CUS * coresident)) if coresident > 1 else rounds
    slices = -(-K // bk)
    per_round = (t_ns - waves * fixed_ns) / rounds
    return 1000.0 * slices * 2.0 * bm * bn * bk / (CU_FLOP_PER_NS * per_round)


def launch_floor(torch, sg, warm_ms, ref=REF_VARIANT):
    """Time every launch takes beyond the cost model (dispatch, completion,
    the events): a one-tile product under the small-tile reference variant,
    one slice deep, less the model's fixed cost and that slice (the time one
    more slice adds, measured over 32 more)."""
    v = sg.sgemm_f32_variant(ref)
    t1 = _forced(torch, sg, ref, 8, 8, v.bk, warm_ms)
    t33 = _forced(torch, sg, ref, 8, 8, 33 * v.bk, warm_ms)
    floor = t1 - TILE_FIXED_NS - (t33 - t1) / 32.0
    print(json.dumps({"floor": "launch", "variant": ref, "us": [round(t1 / 1e3, 2), round(t33 / 1e3, 2)],
                      "floor_ns": round(floor)}), flush=True)
    return max(floor, 0.0)


def _record(vid, v, name, M, N, K, t, e):
    print(json.dumps({"variant": vid, "tile": f"{v.bm}x{v.bn}x{v.bk}", "shape": name,
                      "M": M, "N": N, "K": K, "us": round(t / 1e3, 2),
                      "tflops": round(2.0 * M * N * K / t / 1e3, 2), "eff": round(e)}),
          flush=True)


def fit_fixed(torch, sg, vid, warm_ms, floor):
    """Fixed cost per tile (ns) of a variant whose pipeline fill differs from
    the common 2.5 us: its one-round shape (16 BM x 16 BN) as many slices deep
    as it has LDS stages (at least two: the pipeline full) and at K = 2048,
    the line through them taken back to K = 0."""
    v = sg.sgemm_f32_variant(vid)
    stages = max(2, round(v.lds_bytes / (4.0 * (v.bm + v.bn) * v.bk)))
    M1, N1, k1 = 16 * v.bm, 16 * v.bn, stages * v.bk
    t1 = _forced(torch, sg, vid, M1, N1, k1, warm_ms)
    t2 = _forced(torch, sg, vid, M1, N1, 2048, warm_ms)
    fixed = max(t1 - (t2 - t1) / (2048.0 - k1) * k1 - floor, 0.0)
    print(json.dumps({"variant": vid, "fit": "fixed", "K": [k1, 2048],
                      "us": [round(t1 / 1e3, 2), round(t2 / 1e3, 2)], "fixed_ns": round(fixed)}),
          flush=True)
    return fixed


def calibrate_variant(torch, sg, vid, warm_ms, floor, fixed=TILE_FIXED_NS):
    v = sg.sgemm_f32_variant(vid)
    bm, bn, bk = v.bm, v.bn, v.bk
    shapes = {
        "full": (32 * bm, 32 * bn, 4096),
        "one": (16 * bm, 16 * bn, 4096),
        # odd leading dimensions: rows not 16-byte aligned
        "unaligned": (32 * bm - 5, 32 * bn - 5, 4099),
    }
    out = {}
    for name, (M, N, K) in shapes.items():
        t = _forced(torch, sg, vid, M, N, K, warm_ms)
        e = eff_from_time(t - floor, bm, bn, bk, M, N, K, fixed)
        out[name] = round(e)
        _record(vid, v, name, M, N, K, t, e)
    return out


def calibrate_ksplit(torch, sg, vid, warm_ms, floor):
    """A variant that splits K over its waves (spill modelled):

    - its fixed cost and one-round rate from its one-round shape (16 BM x 16
      BN) one slice deep and at K = 2048, where the operands one XCD reads
      stay in its L2;
    - its rate over four rounds (32 BM x 32 BN, K = 1024) with that fixed cost;
    - its spill factors from the one-round and four-round shapes at
      K = 4096 * 32 / BM (4096, 8192 and 16384 for 32 x 32, 16 x 16 and
      8 x 8 tiles), where those operands do not fit: the operand rows and
      columns one XCD's tiles read are then as many bytes for every tile;
    - its rate on unaligned rows where these tiles serve: a few tiles with
      long K (4 BM - 5 x 4 BN - 5, 16 tiles, K = 16384 * 32 / BM + 3, spilled
      as above), the spill factor taken out, stored scaled by full / one as
      the model scales it back for one round."""
    v = sg.sgemm_f32_variant(vid)
    bm, bn, bk = v.bm, v.bn, v.bk
    co = v.coresident
    M1, N1 = 16 * bm, 16 * bn
    t1 = _forced(torch, sg, vid, M1, N1, bk, warm_ms)
    t2k = _forced(torch, sg, vid, M1, N1, 2048, warm_ms)
    fixed = max(t1 - (t2k - t1) / (2048.0 - bk) * bk - floor, 0.0)
    out = {"fixed": round(fixed)}
    e_one = eff_from_time(t2k - floor, bm, bn, bk, M1, N1, 2048, fixed)
    out["one"] = round(e_one)
    _record(vid, v, "one", M1, N1, 2048, t2k, e_one)
    M, N, K = 32 * bm, 32 * bn, 1024
    t = _forced(torch, sg, vid, M, N, K, warm_ms)
    e_full = eff_from_time(t - floor, bm, bn, bk, M, N, K, fixed, co)
    out["full"] = round(e_full)
    _record(vid, v, "full", M, N, K, t, e_full)
    k_spill = 4096 * 32 // bm
    slices = -(-k_spill // bk)
    t4k = _forced(torch, sg, vid, M1, N1, k_spill, warm_ms)
    spill = (t4k - floor - fixed) / (slices * slice_ns(bm, bn, bk, e_one))
    out["spill"] = round(1000.0 * spill)
    M4, N4 = 32 * bm, 32 * bn
    tiles4 = (M4 // bm) * (N4 // bn)
    rounds = -(-tiles4 // CUS)
    waves = -(-tiles4 // (CUS * co)) if co > 1 else rounds
    t4k_full = _forced(torch, sg, vid, M4, N4, k_spill, warm_ms)
    out["spill_full"] = round(1000.0 * ((t4k_full - floor - waves * fixed) / rounds) /
                              (slices * slice_ns(bm, bn, bk, e_full)))
    print(json.dumps({"variant": vid, "shape": "spill", "M": [M1, M4], "N": [N1, N4], "K": k_spill,
                      "us": [round(t4k / 1e3, 2), round(t4k_full / 1e3, 2)],
                      "fixed_ns": out["fixed"], "spill_permille": out["spill"],
                      "spill_full_permille": out["spill_full"]}), flush=True)
    M, N, K = 4 * bm - 5, 4 * bn - 5, 16384 * 32 // bm + 3
    t = _forced(torch, sg, vid, M, N, K, warm_ms)
    e = eff_from_time(t - floor, bm, bn, bk, M, N, K, fixed, co) * spill
    out["unaligned"] = round(e * e_full / e_one)
    _record(vid, v, "unaligned (16 tiles, spill taken out)", M, N, K, t, e)
    return out


def _strip_only(torch, sg, M, N, K, tb, warm_ms):
    """GPU time (ns) of a product of M <= 4 rows run by the strip kernel alone
    (a row strip streaming op(B): x-contiguous, k-contiguous when B is
    transposed)."""
    A = torch.empty((M, K), device="cuda").uniform_(-1, 1)
    B = torch.empty((N, K) if tb else (K, N), device="cuda").uniform_(-1, 1)
    C = torch.empty((M, N), device="cuda")
    cfg = sg.SgemmCfg()
    cfg.id, cfg.group_m, cfg.xcd_remap, cfg.strip_m = 4, 8, 1, M
    t = _time(torch, lambda: sg.sgemm(A, B, out=C, cfg=cfg, transb=bool(tb), workspace=False),
              warm_ms)
    del A, B, C
    return t


def calibrate_strips(torch, sg, warm_ms):
    """The strip kernel's cost model: fixed cost (ns, the launch floor
    included), the chip's streaming rate per order (bytes/ns) and the rate of
    one workgroup when a strip has too few of them.  4-row products streaming
    op(B): the chip's rates from N = 8192 and 16384 (256 and 512 workgroups,
    K = 4096); the fixed cost is the larger of the two orders' intercepts.
    The per-workgroup rates from N = 256 with K = 262144: 8 x-contiguous
    workgroups, or 16 narrow k-contiguous ones."""
    fits = {}
    for tb in (0, 1):
        pts = []
        for n in (8192, 16384):
            M, N, K = 4, n, 4096
            t = _strip_only(torch, sg, M, N, K, tb, warm_ms)
            nbytes = 4.0 * K * N
            pts.append((nbytes, t))
            print(json.dumps({"strip": "row", "transb": tb, "M": M, "N": N, "K": K,
                              "us": round(t / 1e3, 2), "GB/s": round(nbytes / t, 1)}),
                  flush=True)
        (b0, t0), (b1, t1) = pts
        rate = (b1 - b0) / (t1 - t0)
        fits[tb] = (t0 - b0 / rate, rate)
    fixed = max(f for f, _ in fits.values())
    per_wg = {}
    for tb in (0, 1):
        M, N, K = 4, 256, 262144
        t = _strip_only(torch, sg, M, N, K, tb, warm_ms)
        wgs = N // 16 if tb else N // 32
        nbytes = 4.0 * K * N
        per_wg[tb] = nbytes / (t - fixed) / wgs
        print(json.dumps({"strip": "row", "transb": tb, "M": M, "N": N, "K": K, "workgroups": wgs,
                          "us": round(t / 1e3, 2), "GB/s per workgroup": round(per_wg[tb], 1)}),
              flush=True)
    return {"fixed": fixed, "kc": fits[1][1], "xc": fits[0][1], "wg_xc": per_wg[0],
            "wg_kc_narrow": per_wg[1]}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--variants", default="",
                    help="comma-separated variant ids (default: every selectable one)")
    ap.add_argument("--ms", type=float, default=150.0, help="warm-up per measurement, ms")
    ap.add_argument("--no-strips", action="store_true")
    ap.add_argument("--strips-only", action="store_true",
                    help="measure only the strip kernel's figures")
    ap.add_argument("--fit-fixed", default="",
                    help="comma-separated tile variants whose fixed cost is fitted instead "
                         "of taken as 2.5 us")

    args = ap.parse_args(argv)
    import torch
    import fp32_gemm_sgemm_amd as sg
    if not torch.cuda.is_available():
        raise SystemExit("calibration needs a GPU")
    sg.load()
    if args.strips_only:
        vids = []
    elif args.variants:
        vids = [int(x) for x in args.variants.split(",")]
    else:
        vids = [i for i in range(sg.sgemm_f32_num_variants()) if _is_rated(sg, i)]
    floor = launch_floor(torch, sg, args.ms) if vids else 0.0
    fit = {int(x) for x in args.fit_fixed.split(",") if x}
    table = {}
    for vid in vids:
        if sg.sgemm_f32_variant(vid).spill_full_permille > 0:
            table[vid] = calibrate_ksplit(torch, sg, vid, args.ms, floor)
        elif vid in fit:
            fixed = fit_fixed(torch, sg, vid, args.ms, floor)
            table[vid] = calibrate_variant(torch, sg, vid, args.ms, floor, fixed)
            table[vid]["fit"] = round(fixed)
        else:
            table[vid] = calibrate_variant(torch, sg, vid, args.ms, floor)
    for vid, e in table.items():
        co = sg.sgemm_f32_variant(vid).coresident
        extra = f", {e['fixed']}, {e['spill']}, {e['spill_full']}, {co}" if "spill" in e else ""
        if "fit" in e:
            extra = f", {e['fit']}"
        print(f"variant {vid}: ({e['full']}, {e['one']}, {e['unaligned']}{extra})", flush=True)
    if not args.no_strips:
        st = calibrate_strips(torch, sg, args.ms)
        print(f"strips: kStripFixedNs = {st['fixed']:.0f}, kStripBytesPerNs = {st['kc']:.0f}, "
              f"kStripBytesPerNsXc = {st['xc']:.0f}, kStripWgBytesPerNsXc = {st['wg_xc']:.1f}, "
              f"kStripWgBytesPerNsKcNarrow = {st['wg_kc_narrow']:.1f}", flush=True)
    return 0


def _is_rated(sg, vid):
    """The variants the table rates: the matrix-core ones and the vector-FMA
    tiles that split K (the vector-FMA comparison kernel is measured only
    when named with --variants)."""
    v = sg.sgemm_f32_variant(vid)
    return v.kernel == sg.binding.SGEMM_KERNEL_MFMA or v.spill_full_permille > 0


if __name__ == "__main__":
    sys.exit(main())
