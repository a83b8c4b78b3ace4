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
#include "sgemm_valu.hpp"
#include "select.hpp"

namespace {

using sgemm::Variant;

template <int BM, int BN, int BK, int WM, int WN, int STAGE_AT>
Variant mfma_variant(int eff_permille)
{
    typedef sgemm::MfmaTraits<BM, BN, BK, WM, WN, STAGE_AT> T;
    return Variant{SGEMM_KERNEL_MFMA, BM, BN, BK, WM, WN, STAGE_AT,
                   T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
                   reinterpret_cast<const void *>(
                       &sgemm::sgemm_mfma_kernel<BM, BN, BK, WM, WN, STAGE_AT>),
                   eff_permille};
}

Variant valu_variant()
{
    typedef sgemm::ValuTraits T;
    return Variant{SGEMM_KERNEL_VALU, T::BM, T::BN, T::BK, 1, 1, -1,
                   T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
                   reinterpret_cast<const void *>(&sgemm::sgemm_valu_kernel), 0};
}

// The compiled variants.  Indices are part of the ABI of sgemm_f32_ex.  The
// last argument is the fraction of the FP32 matrix peak (x1000) the variant
// sustains per round of full tiles on MI355X (measured at 8192^3 and divided
// by that shape's wave quantisation), which the selector's cost model uses;
// 0 keeps a variant out of automatic selection (comparison kernels).
const Variant kVariants[] = {
    mfma_variant<256, 256, 16, 4, 2, 0>(894),   // 0: 8 waves of 64x128
    mfma_variant<128, 128, 16, 2, 2, 0>(879),   // 1: 4 waves of 64x64
    mfma_variant<128, 128, 32, 2, 2, 1>(839),   // 2: 4 waves of 64x64, BK 32
    mfma_variant<128, 256, 16, 2, 2, 0>(0),     // 3: 4 waves of 64x128
    mfma_variant<256, 128, 16, 4, 1, 0>(0),     // 4: 4 waves of 64x128
    mfma_variant<256, 256, 16, 4, 2, -1>(0),    // 5: plain order (comparison)
    mfma_variant<128, 128, 16, 2, 2, -1>(0),    // 6: plain order (comparison)
    valu_variant(),                             // 7: vector-FMA comparison
    mfma_variant<192, 192, 16, 2, 6, 0>(746),   // 8: 12 waves of 96x32
    mfma_variant<192, 192, 32, 2, 6, 1>(782),   // 9: 12 waves of 96x32, BK 32
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

hipError_t launch(const Variant &v, const sgemm_cfg &cfg, int M, int N, int K,
                  const float *A, int lda, const float *B, int ldb, float *C, int ldc,
                  hipStream_t stream)
{
    int tiles_m = cfg.tiles_m, tiles_n = cfg.tiles_n;
    int group_m = cfg.group_m, xcd = cfg.xcd_remap;
    void *args[] = {&M, &N, &K, (void *)&A, &lda, (void *)&B, &ldb, &C, &ldc,
                    &tiles_m, &tiles_n, &group_m, &xcd};
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

int sgemm_f32_plan(int M, int N, int K, int lda, int ldb, int ldc, int num_cus, sgemm_cfg *out)
{
    if (!out || M < 0 || N < 0 || K < 0) return hipErrorInvalidValue;
    if (!sgemm::leading_dims_ok(M, N, K, lda, ldb, ldc)) return hipErrorInvalidValue;
    const int id = sgemm::select_variant(kVariants, kNumVariants, M, N, K, num_cus > 0 ? num_cus : 256);
    return sgemm::finish_cfg(kVariants[id], id, M, N, out) ? hipSuccess : hipErrorInvalidValue;
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
    return sgemm_f32_plan(M, N, K, lda, ldb, ldc, cus, out);
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
        id = sgemm::select_variant(kVariants, kNumVariants, M, N, K, cus);
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
