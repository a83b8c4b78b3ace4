// Variant description and the shape-aware selector: pure host integer logic,
// no HIP calls, so it can be exercised without a device.
//
// Geometry uses round-up-and-guard sizing (DD2360 workbook "Applied GPU
// Programming", Module 6, section 6.3): tiles_m = ceil(M/BM),
// tiles_n = ceil(N/BN), one workgroup per tile.  The selector weighs per-tile
// efficiency against wave quantisation: on S compute units a grid of n equal
// tiles takes ceil(n/S) rounds ("4.1 CUDA GEMM operator performance
// optimization", section 12.5 on launching at least as many blocks as SMs and
// tuning per shape; the workbook's Module 17 on the tail effect).
#pragma once

#include <limits.h>

#include "sgemm.h"

namespace sgemm {

struct Variant {
    int kernel;
    int bm, bn, bk;
    int waves_m, waves_n;
    int stage_at;      // register-staged kernel: LDS write after this k group
    int stages;        // direct-load kernel: LDS stages (0 = register-staged kernel)
    int threads;
    int lds_bytes;
    const void *fn;
    int eff_permille;  // measured steady-state fraction of the FP32 matrix peak
                       // (x1000) at 8192^3; 0 = never chosen by the selector
};

// Largest sizes accepted: k0 + BK and similar sums stay in int, and the byte
// offsets of a thread inside one slice ((BM-1)*lda + BK floats of A,
// (BK-1)*ldb + BN floats of B) stay below 2^32.
constexpr int kMaxDim = INT_MAX - 1024;
constexpr int kMaxLda = (1 << 22) - 64;
constexpr int kMaxLdb = (1 << 25) - 512;

inline bool leading_dims_ok(int M, int N, int K, int lda, int ldb, int ldc)
{
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return false;
    const int mk = K > 1 ? K : 1, mn = N > 1 ? N : 1;
    return lda >= mk && ldb >= mn && ldc >= mn && lda <= kMaxLda && ldb <= kMaxLdb;
}

inline long long ceil_div_ll(long long a, long long b) { return (a + b - 1) / b; }

inline void describe(const Variant &v, int id, sgemm_cfg *out)
{
    out->id = id;
    out->kernel = v.kernel;
    out->bm = v.bm;
    out->bn = v.bn;
    out->bk = v.bk;
    out->waves_m = v.waves_m;
    out->waves_n = v.waves_n;
    out->group_m = 0;
    out->xcd_remap = 0;
    out->grid = 0;
    out->threads = v.threads;
    out->lds_bytes = v.lds_bytes;
    out->tiles_m = 0;
    out->tiles_n = 0;
}

// Default tile order: groups of 8 tile rows and the XCD remap.
constexpr int kDefaultGroupM = 8;
constexpr int kDefaultXcdRemap = 1;

inline bool finish_cfg(const Variant &v, int id, int M, int N, sgemm_cfg *out)
{
    describe(v, id, out);
    const long long tm = ceil_div_ll(M, v.bm), tn = ceil_div_ll(N, v.bn);
    if (tm * tn > INT_MAX) return false;
    out->tiles_m = (int)tm;
    out->tiles_n = (int)tn;
    out->grid = (int)(tm * tn);
    out->group_m = kDefaultGroupM;
    out->xcd_remap = kDefaultXcdRemap;
    return true;
}

// Per-tile overhead (prologue fetch, epilogue stores, pipeline fill), in
// 16-deep slices of the same tile.
constexpr long long kTileOverhead = 24;

// Estimated cost of running variant v on M x N x K (arbitrary units):
// rounds * tile area * (K slices + overhead) / efficiency.
inline long long estimate(const Variant &v, int M, int N, int K, int cus)
{
    const long long tiles = ceil_div_ll(M, v.bm) * ceil_div_ll(N, v.bn);
    const long long rounds = ceil_div_ll(tiles, cus);
    long long slices = ceil_div_ll(K, v.bk);
    if (v.stages == 0 && v.stage_at >= 0) slices += slices & 1;  // register pipeline takes pairs
    const long long kpad = slices * v.bk;
    const long long area = (long long)v.bm * v.bn;
    const long long work = area * (kpad / 16 + kTileOverhead);
    return rounds * work * 1000 / v.eff_permille;
}

// direct_ok: the operands allow direct global -> LDS loads (16-byte aligned
// rows); otherwise the direct-load variants would fetch every slice through
// registers and are left out.
inline int select_variant(const Variant *vs, int n, int M, int N, int K, int cus, bool direct_ok)
{
    int best = -1;
    long long best_cost = 0;
    for (int i = 0; i < n; ++i) {
        if (vs[i].kernel != SGEMM_KERNEL_MFMA || vs[i].eff_permille <= 0) continue;
        if (vs[i].stages > 0 && !direct_ok) continue;
        const long long c = estimate(vs[i], M, N, K, cus);
        if (best < 0 || c < best_cost) {
            best = i;
            best_cost = c;
        }
    }
    return best < 0 ? 0 : best;
}

}  // namespace sgemm
