// Variant description and the shape-aware selector: pure host integer logic,
// no HIP calls, so it can be exercised without a device.
//
// Geometry uses round-up-and-guard sizing (DD2360 workbook "Applied GPU
// Programming", Module 6, section 6.3): tiles_m = ceil(M/BM),
// tiles_n = ceil(N/BN), one workgroup per tile.  The selector weighs per-tile
// efficiency against wave quantisation: a grid of n workgroups on S resident
// slots takes ceil(n/S) rounds ("4.1 CUDA GEMM operator performance
// optimization", section 12.5 on launching at least as many blocks as SMs;
// the workbook's Module 17 on the tail effect).
#pragma once

#include <limits.h>

#include "sgemm.h"

namespace sgemm {

struct Variant {
    int kernel;
    int bm, bn, bk;
    int waves_m, waves_n;
    int vec;
    int threads;
    int lds_bytes;
    const void *fn;
};

// Largest size accepted, so that k0 + BK and similar sums stay in int.
constexpr int kMaxDim = INT_MAX - 1024;

inline bool leading_dims_ok(int M, int N, int K, int lda, int ldb, int ldc)
{
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return false;
    const int mk = K > 1 ? K : 1, mn = N > 1 ? N : 1;
    return lda >= mk && ldb >= mn && ldc >= mn;
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
    out->vec = v.vec;
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

// Index of the MFMA variant with the given tile and path, or -1.
inline int find_variant(const Variant *vs, int n, int bm, int bn, int bk, int waves, int vec)
{
    for (int i = 0; i < n; ++i)
        if (vs[i].kernel == SGEMM_KERNEL_MFMA && vs[i].bm == bm && vs[i].bn == bn &&
            vs[i].bk == bk && vs[i].waves_m * vs[i].waves_n == waves && vs[i].vec == vec)
            return i;
    return -1;
}

inline int select_variant(const Variant *vs, int n, int M, int N, int K, bool vec, int cus)
{
    (void)K;
    const int v = vec ? 1 : 0;
    const long long big = ceil_div_ll(M, 256) * ceil_div_ll(N, 256);
    int id = -1;
    if (big >= cus) id = find_variant(vs, n, 256, 256, 16, 8, v);
    if (id < 0) id = find_variant(vs, n, 128, 128, 16, 4, v);
    if (id < 0) id = 0;
    return id;
}

}  // namespace sgemm
