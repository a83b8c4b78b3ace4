// libsgemm: the C ABI of include/sgemm.h, the table of compiled variants, the
// shape-aware selector and argument validation.
//
// Host workflow conventions (asynchronous launch on the caller's stream,
// launch errors returned by the call, execution faults at the next
// synchronisation) follow the DD2360 workbook "Applied GPU Programming",
// Module 5, sections 5.5-5.6.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "sgemm.h"
#include "sgemm_mfma.hpp"
#include "sgemm_mfma_dl.hpp"
#include "sgemm_valu.hpp"
#include "select.hpp"

namespace {

using sgemm::Variant;

template <int BM, int BN, int BK, int WM, int WN, int STAGE_AT>
Variant mfma_variant(int eff_permille)
{
    typedef sgemm::MfmaTraits<BM, BN, BK, WM, WN, STAGE_AT> T;
    return Variant{SGEMM_KERNEL_MFMA, BM, BN, BK, WM, WN, STAGE_AT, 0,
                   T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
                   reinterpret_cast<const void *>(
                       &sgemm::sgemm_mfma_kernel<BM, BN, BK, WM, WN, STAGE_AT>),
                   eff_permille};
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES>
Variant dl_variant(int eff_permille)
{
    typedef sgemm::DlTraits<BM, BN, BK, WM, WN, STAGES> T;
    return Variant{SGEMM_KERNEL_MFMA, BM, BN, BK, WM, WN, -1, STAGES,
                   T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
                   reinterpret_cast<const void *>(
                       &sgemm::sgemm_mfma_dl_kernel<BM, BN, BK, WM, WN, STAGES>),
                   eff_permille};
}

Variant valu_variant()
{
    typedef sgemm::ValuTraits T;
    return Variant{SGEMM_KERNEL_VALU, T::BM, T::BN, T::BK, 1, 1, -1, 0,
                   T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
                   reinterpret_cast<const void *>(&sgemm::sgemm_valu_kernel), 0};
}

// The compiled variants.  Indices are part of the ABI of sgemm_f32_ex.  The
// last argument is the fraction of the FP32 matrix peak (x1000) the variant
// sustains per round of full tiles on MI355X, which the selector's cost model
// uses: measured at 8192^3 for the 256 x 256 and 128 x 128 tiles, at 3072^3
// (exactly one 192 x 192 tile per CU) for the 192 x 192 tiles.  0 keeps a
// variant out of automatic selection (comparison kernels, dominated tiles).
const Variant kVariants[] = {
    mfma_variant<256, 256, 16, 4, 2, 0>(894),   // 0: 8 waves of 64x128
    mfma_variant<128, 128, 16, 2, 2, 0>(861),   // 1: 4 waves of 64x64
    mfma_variant<128, 128, 32, 2, 2, 1>(0),     // 2: 4 waves of 64x64, BK 32
    mfma_variant<128, 256, 16, 2, 2, 0>(0),     // 3: 4 waves of 64x128
    mfma_variant<256, 128, 16, 4, 1, 0>(0),     // 4: 4 waves of 64x128
    mfma_variant<256, 256, 16, 4, 2, -1>(0),    // 5: plain order (comparison)
    mfma_variant<128, 128, 16, 2, 2, -1>(0),    // 6: plain order (comparison)
    valu_variant(),                             // 7: vector-FMA comparison
    mfma_variant<192, 192, 16, 2, 6, 0>(0),     // 8: 12 waves of 96x32
    mfma_variant<192, 192, 32, 2, 6, 1>(869),   // 9: 12 waves of 96x32, BK 32
    dl_variant<256, 256, 16, 4, 2, 4>(0),       // 10: direct loads, 4 stages
    dl_variant<256, 256, 32, 4, 2, 2>(912),     // 11: direct loads, 2 stages of BK 32
    dl_variant<128, 128, 32, 2, 2, 3>(775),     // 12: direct loads
    dl_variant<192, 192, 32, 2, 6, 3>(854),     // 13: direct loads
    dl_variant<256, 256, 16, 4, 2, 3>(0),       // 14: direct loads, 3 stages
};
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

// ---- device properties, queried once per device ----------------------------
constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
int g_dev_cus[kMaxDevices];  // 0 = not queried yet

hipError_t device_cus(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    if (g_dev_cus[dev] == 0) {
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        g_dev_cus[dev] = n > 0 ? n : 1;
    }
    *cus = g_dev_cus[dev];
    return hipSuccess;
}

// ---- validation ---------------------------------------------------------------
bool misaligned4(const void *p) { return ((uintptr_t)p & 3u) != 0; }

// Address range [lo, hi) spanned by a rows x cols row-major matrix with stride ld.
void span(const void *p, int rows, int cols, int ld, uintptr_t &lo, uintptr_t &hi)
{
    lo = (uintptr_t)p;
    hi = lo + ((uint64_t)(rows - 1) * (uint64_t)ld + (uint64_t)cols) * sizeof(float);
}

bool overlaps(const void *a, int ar, int ac, int lda, const void *c, int cr, int cc, int ldc)
{
    if (ar == 0 || ac == 0 || cr == 0 || cc == 0) return false;
    uintptr_t alo, ahi, clo, chi;
    span(a, ar, ac, lda, alo, ahi);
    span(c, cr, cc, ldc, clo, chi);
    return clo < ahi && alo < chi;
}

hipError_t validate(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                    const float *C, int ldc)
{
    if (M < 0 || N < 0 || K < 0) return hipErrorInvalidValue;
    if (!sgemm::leading_dims_ok(M, N, K, lda, ldb, ldc)) return hipErrorInvalidValue;
    if (M == 0 || N == 0) return hipSuccess;
    if (K > 0 && (!A || !B || misaligned4(A) || misaligned4(B))) return hipErrorInvalidValue;
    if (!C || misaligned4(C)) return hipErrorInvalidValue;
    if (K > 0 && (overlaps(A, M, K, lda, C, M, N, ldc) || overlaps(B, K, N, ldb, C, M, N, ldc)))
        return hipErrorInvalidValue;
    return hipSuccess;
}

// Direct global -> LDS loads need 16-byte aligned rows, and byte offsets inside
// a slice below 2^31 (the offset given to chunks that must read as zero).
bool direct_loads_ok(const float *A, int lda, const float *B, int ldb)
{
    const bool al = (((uintptr_t)A | (uintptr_t)B) & 15u) == 0 && lda % 4 == 0 && ldb % 4 == 0;
    // (a null pointer stands for an aligned start: used by sgemm_f32_plan)
    return al && lda <= (1 << 20) && ldb <= (1 << 24);
}

hipError_t launch(const Variant &v, const sgemm_cfg &cfg, int M, int N, int K,
                  const float *A, int lda, const float *B, int ldb, float *C, int ldc,
                  hipStream_t stream)
{
    int tiles_m = cfg.tiles_m, tiles_n = cfg.tiles_n;
    int group_m = cfg.group_m, xcd = cfg.xcd_remap;
    int direct = direct_loads_ok(A, lda, B, ldb) ? 1 : 0;
    void *args[] = {&M, &N, &K, (void *)&A, &lda, (void *)&B, &ldb, &C, &ldc,
                    &tiles_m, &tiles_n, &group_m, &xcd, &direct};
    return hipLaunchKernel(v.fn, dim3((unsigned)cfg.grid), dim3((unsigned)v.threads), args, 0, stream);
}

}  // namespace

extern "C" {

int sgemm_f32_num_variants(void) { return kNumVariants; }

int sgemm_f32_variant(int id, sgemm_cfg *out)
{
    if (!out || id < 0 || id >= kNumVariants) return hipErrorInvalidValue;
    sgemm::describe(kVariants[id], id, out);
    return hipSuccess;
}

const char *sgemm_f32_version(void) { return "libsgemm 0.2.0 gfx950 fp32 (mfma_f32_32x32x2 + valu comparison)"; }

namespace {
int plan_for(int M, int N, int K, int lda, int ldb, int ldc, int num_cus, bool direct, sgemm_cfg *out)
{
    if (!out || M < 0 || N < 0 || K < 0) return hipErrorInvalidValue;
    if (!sgemm::leading_dims_ok(M, N, K, lda, ldb, ldc)) return hipErrorInvalidValue;
    const int id = sgemm::select_variant(kVariants, kNumVariants, M, N, K,
                                         num_cus > 0 ? num_cus : 256, direct);
    return sgemm::finish_cfg(kVariants[id], id, M, N, out) ? hipSuccess : hipErrorInvalidValue;
}
}  // namespace

int sgemm_f32_plan(int M, int N, int K, int lda, int ldb, int ldc, int num_cus, sgemm_cfg *out)
{
    // operands are assumed to start 16-byte aligned (as allocations do)
    return plan_for(M, N, K, lda, ldb, ldc, num_cus, direct_loads_ok(nullptr, lda, nullptr, ldb), out);
}

int sgemm_f32_query(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                    float *C, int ldc, sgemm_cfg *out)
{
    if (!out) return hipErrorInvalidValue;
    hipError_t e = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (e != hipSuccess) return e;
    int cus = 0;
    e = device_cus(&cus);
    if (e != hipSuccess) return e;
    return plan_for(M, N, K, lda, ldb, ldc, cus, direct_loads_ok(A, lda, B, ldb), out);
}

int sgemm_f32_ex(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                 float *C, int ldc, hipStream_t stream, const sgemm_cfg *force)
{
    hipError_t e = validate(M, N, K, A, lda, B, ldb, C, ldc);
    if (e != hipSuccess) return e;
    if (M == 0 || N == 0) return hipSuccess;
    sgemm_cfg cfg;
    int id;
    if (force) {
        id = force->id;
        if (id < 0 || id >= kNumVariants || force->group_m < 0) return hipErrorInvalidValue;
        if (!sgemm::finish_cfg(kVariants[id], id, M, N, &cfg)) return hipErrorInvalidValue;
        cfg.group_m = force->group_m;
        cfg.xcd_remap = force->xcd_remap ? 1 : 0;
    } else {
        int cus = 0;
        e = device_cus(&cus);
        if (e != hipSuccess) return e;
        id = sgemm::select_variant(kVariants, kNumVariants, M, N, K, cus,
                                   direct_loads_ok(A, lda, B, ldb));
        if (!sgemm::finish_cfg(kVariants[id], id, M, N, &cfg)) return hipErrorInvalidValue;
    }
    return launch(kVariants[id], cfg, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int sgemm_f32(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
              float *C, int ldc, hipStream_t stream)
{
    return sgemm_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, stream, nullptr);
}

}  // extern "C"
