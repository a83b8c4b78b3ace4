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
#include <string.h>

#include <mutex>

#include "sgemm.h"
#include "sgemm_mfma.hpp"
#include "sgemm_mfma_dl.hpp"
#include "sgemm_mfma_sk.hpp"
#include "sgemm_valu_sk.hpp"
#include "sgemm_reduce.hpp"
#include "sgemm_strip.hpp"
#include "sgemm_valu.hpp"
#include "select.hpp"

namespace {

using sgemm::Choice;
using sgemm::GemmArgs;
using sgemm::Problem;
using sgemm::Variant;

template <int BM, int BN, int BK, int WM, int WN, int STAGE_AT>
Variant mfma_variant(int eff_permille, int eff_one_permille, int eff_unaligned_permille)
{
    typedef sgemm::MfmaTraits<BM, BN, BK, WM, WN, STAGE_AT> T;
    return Variant{SGEMM_KERNEL_MFMA, BM, BN, BK, WM, WN, STAGE_AT, 0, 0,
                   T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
                   {reinterpret_cast<const void *>(
                        &sgemm::sgemm_mfma_kernel<BM, BN, BK, WM, WN, STAGE_AT>),
                    nullptr, nullptr, nullptr},
                   eff_permille, eff_one_permille, eff_unaligned_permille, 0, 0, 0, 0};
}

// OPS: bit (transa + 2*transb) set for each operand layout to compile.  DW:
// 4-byte direct loads (rows need only be 4-byte aligned).
// MB: 32x32 (32) or 16x16 (16) MFMA blocks.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int OPS, bool DW = false,
          int PIPE = 0, int MB = 32>
Variant dl_variant(int eff_permille, int eff_one_permille, int eff_unaligned_permille,
                   int fixed_ns = 0)
{
    typedef sgemm::DlTraits<BM, BN, BK, WM, WN, STAGES, false, false, DW, MB> T;
    Variant v{SGEMM_KERNEL_MFMA, BM, BN, BK, WM, WN, -1, STAGES, DW ? 1 : 0,
              T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
              {nullptr, nullptr, nullptr, nullptr}, eff_permille, eff_one_permille,
              eff_unaligned_permille, fixed_ns, 0, 0, 0};
    v.fn[0] = reinterpret_cast<const void *>(
        &sgemm::sgemm_mfma_dl_kernel<BM, BN, BK, WM, WN, STAGES, false, false, DW, PIPE, MB>);
    if constexpr ((OPS & 2) != 0)
        v.fn[1] = reinterpret_cast<const void *>(
            &sgemm::sgemm_mfma_dl_kernel<BM, BN, BK, WM, WN, STAGES, true, false, DW, PIPE, MB>);
    if constexpr ((OPS & 4) != 0)
        v.fn[2] = reinterpret_cast<const void *>(
            &sgemm::sgemm_mfma_dl_kernel<BM, BN, BK, WM, WN, STAGES, false, true, DW, PIPE, MB>);
    if constexpr ((OPS & 8) != 0)
        v.fn[3] = reinterpret_cast<const void *>(
            &sgemm::sgemm_mfma_dl_kernel<BM, BN, BK, WM, WN, STAGES, true, true, DW, PIPE, MB>);
    return v;
}

// MB x MB tiles (32x32 or 16x16 MFMA blocks) with K split across the W waves
// of the workgroup (every layout).  waves_m = W describes the waves (they
// share the tile and split K); bk is the k of one group of four MFMA steps.
template <int W, int MB = 32>
Variant sk_variant(int eff_permille, int eff_one_permille, int eff_unaligned_permille, int fixed_ns,
                   int spill_permille, int spill_full_permille, int coresident)
{
    typedef sgemm::SkTraits<W, MB> T;
    return Variant{SGEMM_KERNEL_MFMA, T::BM, T::BN, T::GK, W, 1, -1, 0, 0,
                   T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
                   {reinterpret_cast<const void *>(&sgemm::sgemm_mfma_sk_kernel<W, false, false, MB>),
                    reinterpret_cast<const void *>(&sgemm::sgemm_mfma_sk_kernel<W, true, false, MB>),
                    reinterpret_cast<const void *>(&sgemm::sgemm_mfma_sk_kernel<W, false, true, MB>),
                    reinterpret_cast<const void *>(&sgemm::sgemm_mfma_sk_kernel<W, true, true, MB>)},
                   eff_permille, eff_one_permille, eff_unaligned_permille, fixed_ns,
                   spill_permille, spill_full_permille, coresident, 1};
}

// 8x8 tiles with K split over the lane pairs and W waves of the workgroup,
// on vector FMAs (every layout); bk is the k of one group (one per lane pair).
template <int W>
Variant vsk_variant(int eff_permille, int eff_one_permille, int eff_unaligned_permille, int fixed_ns,
                    int spill_permille, int spill_full_permille, int coresident)
{
    typedef sgemm::VskTraits<W> T;
    return Variant{SGEMM_KERNEL_VALU, T::BM, T::BN, T::GK, W, 1, -1, 0, 0,
                   T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
                   {reinterpret_cast<const void *>(&sgemm::sgemm_valu_sk_kernel<W, false, false>),
                    reinterpret_cast<const void *>(&sgemm::sgemm_valu_sk_kernel<W, true, false>),
                    reinterpret_cast<const void *>(&sgemm::sgemm_valu_sk_kernel<W, false, true>),
                    reinterpret_cast<const void *>(&sgemm::sgemm_valu_sk_kernel<W, true, true>)},
                   eff_permille, eff_one_permille, eff_unaligned_permille, fixed_ns,
                   spill_permille, spill_full_permille, coresident, 1};
}

Variant valu_variant()
{
    typedef sgemm::ValuTraits T;
    return Variant{SGEMM_KERNEL_VALU, T::BM, T::BN, T::BK, 1, 1, -1, 0, 0,
                   T::NT, (int)(T::LDS_FLOATS * sizeof(float)),
                   {reinterpret_cast<const void *>(&sgemm::sgemm_valu_kernel),
                    nullptr, nullptr, nullptr},
                   0, 0, 0, 0, 0, 0, 0};
}

constexpr int kAllOps = 0xf;
// Direct-load main loop: cross-slice pipeline (2) with accumulators in AGPRs (4).
constexpr int kCrossSliceAgpr = 6;

// The compiled variants.  Indices are part of the ABI of sgemm_f32_ex.  The
// three last arguments are fractions of the FP32 matrix peak (x1000) the
// variant sustains on MI355X, which the selector's cost model uses.  Each is
// the model inverted on one measured shape, K = 4096 throughout (BM x BN the
// variant's tile): over four rounds of full tiles with 16-byte aligned rows
// (32 BM x 32 BN), over one round, one workgroup per CU (16 BM x 16 BN), and
// with rows that are not 16-byte aligned (32 BM - 5 x 32 BN - 5, K = 4099).
// `python -m fp32_gemm_sgemm_amd.calibrate` measures them; the figures below
// come from such runs on MI355X (each family of related tiles from one run:
// the 64x64 tiles together, the 4-byte-load tiles of 128x128 and up together),
// with the launch floor every launch pays taken off each time.  The K-split tiles carry four more numbers:
// their fixed cost per tile in ns; the factors (x1000) by which a slice slows
// once the operand rows and columns one XCD's tiles read exceed its L2, over
// one round and over several (their rates are measured where those fit); and
// how many of their workgroups share a CU (from their register use: 62, 72
// and 72 per lane for the 32x32 tiles with W = 4, 8, 16 in the NN layout, so
// 8, 3 and 1; 48 for the 16x16 ones, so 4 and 2 for W = 8 and 16 at 8 waves
// per SIMD; 108 for the 8x8 vector-FMA tiles, so 4), whose fixed costs
// overlap.  The selector offers the 16x16 and 8x8 tiles only where K cannot
// be split across workgroups (the 8x8 ones also need K >= 4096 and more than
// 4 rows and columns).  The others use the model's common 2.5 us, no spill
// term and one fixed cost per round.
// The 64x64 tiles carry their own fixed cost (--fit-fixed).  The two-stage
// 32-deep ones are rated over one round at K = 4096, where the operands one
// XCD's tiles read stream from beyond its L2: with fewer K they run faster only
// when the same operands are still in L2 from the call before, so the
// four-stage ones (20, 21), which keep their rate either way, are the one-round
// choice.
// The 32x64 tile (25) puts three workgroups on a CU, so its four-round shape
// (1,024 tiles) runs as unequal waves of 768 and 256 and reads 734; inverted on
// 1536 x 1024 x 4096 (768 tiles, three per CU) the model gives 903.  Its table
// figure, 880, lies between: every plan it changes on a 432-shape grid was
// timed faster than the plan it replaced.
// The 4-byte direct-load variants serve only rows that are not 16-byte
// aligned.  The vector-FMA comparison kernel carries no figures: the selector
// never picks it.
const Variant kVariants[] = {
    mfma_variant<256, 256, 16, 4, 2, 0>(888, 887, 690),    // 0: 8 waves of 64x128
    mfma_variant<128, 128, 16, 2, 2, 0>(848, 754, 587),    // 1: 4 waves of 64x64
    valu_variant(),                                        // 2: vector-FMA comparison
    mfma_variant<192, 192, 32, 2, 6, 1>(886, 871, 710),    // 3: 12 waves of 96x32, BK 32
    dl_variant<256, 256, 32, 4, 2, 2, kAllOps, false, kCrossSliceAgpr>(959, 954, 660),  // 4: direct loads, 2 stages of BK 32
    dl_variant<128, 128, 32, 2, 2, 3, kAllOps>(778, 761, 405),  // 5: direct loads
    dl_variant<192, 192, 32, 2, 6, 2, kAllOps, false, kCrossSliceAgpr>(951, 936, 609),  // 6: direct loads
    dl_variant<128, 128, 32, 4, 2, 2, kAllOps, false, kCrossSliceAgpr>(925, 928, 661),  // 7: direct loads, 8 waves of 32x64
    mfma_variant<128, 128, 16, 2, 4, 0>(827, 825, 671),    // 8: 8 waves of 64x32
    mfma_variant<128, 128, 32, 2, 4, 1>(817, 790, 743),    // 9: 8 waves of 64x32, BK 32
    dl_variant<192, 192, 32, 2, 6, 2, kAllOps, true, kCrossSliceAgpr>(946, 910, 942),  // 10: 4-byte direct loads
    dl_variant<64, 64, 32, 2, 2, 2, kAllOps, false, kCrossSliceAgpr>(895, 662, 509, 3329),  // 11: direct loads, 4 waves of 32x32
    dl_variant<64, 64, 32, 2, 2, 2, kAllOps, true, kCrossSliceAgpr>(903, 651, 897, 3874),  // 12: 4-byte direct loads
    dl_variant<128, 128, 32, 4, 2, 2, kAllOps, true, kCrossSliceAgpr>(923, 888, 915),  // 13: 4-byte direct loads, 8 waves of 32x64
    sk_variant<4>(500, 576, 424, 3204, 1054, 990, 8),      // 14: 32x32, K split over 4 waves
    sk_variant<16>(681, 572, 581, 3242, 1045, 1179, 1),    // 15: 32x32, K split over 16 waves
    sk_variant<8>(608, 623, 507, 3207, 1053, 1085, 3),     // 16: 32x32, K split over 8 waves
    dl_variant<64, 64, 64, 2, 2, 2, kAllOps, false, kCrossSliceAgpr>(893, 765, 336, 4108),  // 17: direct loads, 64-deep slices
    dl_variant<64, 64, 64, 2, 2, 2, kAllOps, true, kCrossSliceAgpr>(863, 706, 855, 4808),  // 18: 4-byte direct loads, 64-deep slices
    dl_variant<256, 256, 16, 4, 2, 2, kAllOps, true, kCrossSliceAgpr>(932, 955, 927),  // 19: 4-byte direct loads, 16-deep slices
    dl_variant<64, 64, 32, 2, 2, 4, kAllOps, false, kCrossSliceAgpr, 16>(906, 868, 371, 3900),  // 20: direct loads, 4 stages, 16x16 blocks
    dl_variant<64, 64, 32, 2, 2, 4, kAllOps, true, kCrossSliceAgpr, 16>(894, 770, 894, 4455),   // 21: 4-byte direct loads, 4 stages, 16x16 blocks
    sk_variant<16, 16>(293, 365, 256, 3048, 1195, 866, 2),    // 22: 16x16, K split over 16 waves
    sk_variant<8, 16>(309, 455, 251, 3056, 1410, 909, 4),     // 23: 16x16, K split over 8 waves
    vsk_variant<4>(108, 121, 76, 3032, 1022, 859, 4),         // 24: 8x8 vector FMA, K split over lane pairs and 4 waves
    dl_variant<32, 64, 32, 2, 2, 4, kAllOps, false, kCrossSliceAgpr, 16>(880, 752, 157, 3273),  // 25: direct loads, 4 stages, 4 waves of 16x32 on 16x16 blocks
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

// ---- static scratch (sgemm_f32_ex_noalloc) --------------------------------------
// The partials of K splits for callers that cannot allocate: one array in each
// GPU's memory, held from the code object's load until the process ends.  In
// host code `scratch` names a host-side stand-in, not a device address: kernels
// and copies use the address looked up per device below, never the name.
static __device__ __align__(256) unsigned char scratch[SGEMM_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not yet)

// The current device's address of `scratch`, looked up once per device with
// that device current.
hipError_t device_scratch(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// ---- validation ---------------------------------------------------------------
bool misaligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

// Address range [lo, hi) spanned by `count` row-major rows x cols matrices
// with row stride ld, `stride` elements apart.
struct Span {
    uintptr_t lo, hi;
};

Span span(const void *p, int rows, int cols, int ld, long long stride, int count)
{
    const uint64_t one = (uint64_t)(rows - 1) * (uint64_t)ld + (uint64_t)cols;
    Span s;
    s.lo = (uintptr_t)p;
    s.hi = s.lo + ((uint64_t)(count - 1) * (uint64_t)stride + one) * sizeof(float);
    return s;
}

bool overlap(const Span &a, const Span &b) { return a.lo < b.hi && b.lo < a.hi; }

// A call after the sizes are known valid: the pointers, strides and workspace.
struct Call {
    Problem p;
    float alpha, beta;
    const float *A;
    const float *B;
    float *C;
    long long sa, sb, sc;
    void *ws;
    size_t ws_bytes;
};

// Whether A and B are read at all.
bool reads_operands(const Call &c) { return c.p.K > 0 && c.alpha != 0.0f; }

hipError_t validate(const Call &c)
{
    const Problem &p = c.p;
    if (!sgemm::sizes_ok(p)) return hipErrorInvalidValue;
    if (c.sa < 0 || c.sb < 0 || c.sc < 0) return hipErrorInvalidValue;
    if (p.M == 0 || p.N == 0 || p.batch == 0) return hipSuccess;
    if (!c.C || misaligned(c.C, 4)) return hipErrorInvalidValue;
    if (p.batch > 1 && c.sc < (long long)(p.M - 1) * p.ldc + p.N) return hipErrorInvalidValue;
    const Span cs = span(c.C, p.M, p.N, p.ldc, c.sc, p.batch);
    if (c.ws_bytes > 0) {
        if (!c.ws || misaligned(c.ws, 16)) return hipErrorInvalidValue;
        const Span w{(uintptr_t)c.ws, (uintptr_t)c.ws + c.ws_bytes};
        if (overlap(w, cs)) return hipErrorInvalidValue;
    }
    if (p.K == 0) return hipSuccess;
    if (!c.A || !c.B || misaligned(c.A, 4) || misaligned(c.B, 4)) return hipErrorInvalidValue;
    const Span as = p.transa ? span(c.A, p.K, p.M, p.lda, c.sa, p.batch)
                             : span(c.A, p.M, p.K, p.lda, c.sa, p.batch);
    const Span bs = p.transb ? span(c.B, p.N, p.K, p.ldb, c.sb, p.batch)
                             : span(c.B, p.K, p.N, p.ldb, c.sb, p.batch);
    if (overlap(as, cs) || overlap(bs, cs)) return hipErrorInvalidValue;
    if (c.ws_bytes > 0) {
        const Span w{(uintptr_t)c.ws, (uintptr_t)c.ws + c.ws_bytes};
        if (overlap(w, as) || overlap(w, bs)) return hipErrorInvalidValue;
    }
    return hipSuccess;
}

// Rows start 16-byte aligned in every batch entry (a null pointer stands for
// an aligned start: used by plan).  16-byte direct global -> LDS loads need
// this and the leading-dimension limits of sgemm::direct_lds_ok; 4-byte ones
// need only the limits.
bool rows_aligned16(const Call &c)
{
    const uintptr_t a = (uintptr_t)c.A, b = (uintptr_t)c.B;
    return ((a | b) & 15u) == 0 && c.p.lda % 4 == 0 && c.p.ldb % 4 == 0 &&
           (c.p.batch <= 1 || (c.sa % 4 == 0 && c.sb % 4 == 0));
}

bool direct_loads_ok(const Variant &v, const Call &c)
{
    return sgemm::direct_lds_ok(c.p) && (v.dword || rows_aligned16(c));
}

// Workgroups per launch: the dispatch packet counts work-items in 32 bits.
long long max_wgs_per_launch(int threads) { return (long long)(UINT32_MAX / (uint32_t)threads) & ~7ll; }

hipError_t launch_gemm(const Variant &v, const sgemm_cfg &cfg, const Call &c, hipStream_t stream)
{
    const Problem &p = c.p;
    const void *fn = v.fn[sgemm::op_index(p)];
    GemmArgs g;
    g.A = c.A;
    g.B = c.B;
    g.batch_a = c.sa;
    g.batch_b = c.sb;
    g.M = p.M;
    g.N = p.N;
    g.K = p.K;
    g.lda = p.lda;
    g.ldb = p.ldb;
    g.k_chunk = cfg.k_chunk;
    g.splits = cfg.splits;
    g.tiles_m = cfg.tiles_m;
    g.tiles_n = cfg.tiles_n;
    g.group_m = cfg.group_m;
    g.xcd_remap = cfg.xcd_remap;
    g.direct = direct_loads_ok(v, c) ? 1 : 0;
    const long long ldp = sgemm::partial_ld(p.N);
    if (cfg.splits > 1) {
        // partials: [batch][split][M][ldp] in the workspace
        g.C = static_cast<float *>(c.ws);
        g.ldc = (int)ldp;
        g.split_c = (long long)p.M * ldp;
        g.batch_c = g.split_c * cfg.splits;
        g.alpha = 1.0f;
        g.beta = 0.0f;
    } else {
        g.C = c.C;
        g.ldc = p.ldc;
        g.split_c = 0;
        g.batch_c = c.sc;
        g.alpha = c.alpha;
        g.beta = c.beta;
    }
    const long long per = max_wgs_per_launch(v.threads);
    for (long long base = 0; base < cfg.grid; base += per) {
        const long long n = cfg.grid - base < per ? cfg.grid - base : per;
        g.wg_base = (int)base;
        void *args[] = {&g};
        hipError_t e = hipLaunchKernel(fn, dim3((unsigned)n), dim3((unsigned)v.threads), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// C = alpha * (sum of `splits` partials) + beta * C; splits == 0: C = beta * C.
hipError_t launch_reduce(const Call &c, int splits, float alpha, hipStream_t stream)
{
    const Problem &p = c.p;
    sgemm::ReduceArgs r;
    r.ldp = (int)sgemm::partial_ld(p.N);
    r.P = static_cast<const float *>(c.ws);
    r.split_p = (long long)p.M * r.ldp;
    r.batch_p = r.split_p * splits;
    r.quads = r.split_p / 4;
    r.M = p.M;
    r.N = p.N;
    r.ldc = p.ldc;
    r.splits = splits;
    r.alpha = alpha;
    r.beta = c.beta;
    const long long blocks = (r.quads + 255) / 256;
    if (blocks > INT_MAX) return hipErrorInvalidValue;
    constexpr int kMaxY = 65535;
    for (int z0 = 0; z0 < p.batch; z0 += kMaxY) {
        const int nz = p.batch - z0 < kMaxY ? p.batch - z0 : kMaxY;
        sgemm::ReduceArgs rz = r;
        rz.P = r.P ? r.P + (long long)z0 * r.batch_p : nullptr;
        rz.C = c.C + (long long)z0 * c.sc;
        rz.batch_c = c.sc;
        void *args[] = {&rz};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&sgemm::splitk_reduce_kernel),
                                       dim3((unsigned)blocks, (unsigned)nz), dim3(256), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The edge strips of a plan (sgemm_strip.hpp): the last sm rows of C (all N
// columns), and the last sn columns of the M - sm rows above them.  The row
// strip streams op(B), which is k-contiguous when B is transposed; the column
// strip streams op(A), k-contiguous when A is not.
const void *strip_kernel(const Problem &p)
{
    static const void *const fns[4] = {
        reinterpret_cast<const void *>(&sgemm::sgemm_strip_kernel<false, true>),   // NN
        reinterpret_cast<const void *>(&sgemm::sgemm_strip_kernel<false, false>),  // TN
        reinterpret_cast<const void *>(&sgemm::sgemm_strip_kernel<true, true>),    // NT
        reinterpret_cast<const void *>(&sgemm::sgemm_strip_kernel<true, false>),   // TT
    };
    return fns[sgemm::op_index(p)];
}

hipError_t launch_strips(const Call &c, int sm, int sn, int cus, hipStream_t stream)
{
    const Problem &p = c.p;
    const int m_main = p.M - sm, n_main = p.N - sn;
    // workgroups, order and width of each strip (shared with the cost model)
    const sgemm::StripPlan g = sgemm::strip_plan(p, sm, sn, cus);
    sgemm::StripArgs a = {};
    a.K = p.K;
    a.alpha = c.alpha;
    a.beta = c.beta;
    sgemm::Strip &rs = a.s[0], &cs = a.s[1];
    if (g.row.wgs > 0) {
        // out(x, y) = C[m_main + y][x] = sum_k op(B)[k][x] * op(A)[m_main + y][k]
        rs.big = c.B;
        rs.ld_big = p.ldb;
        rs.batch_big = c.sb;
        if (p.transa) {
            rs.small = c.A + m_main;
            rs.s_y = 1;
            rs.s_k = p.lda;
        } else {
            rs.small = c.A + (long long)m_main * p.lda;
            rs.s_y = p.lda;
            rs.s_k = 1;
        }
        rs.batch_small = c.sa;
        rs.out = c.C + (long long)m_main * p.ldc;
        rs.o_x = 1;
        rs.o_y = p.ldc;
        rs.batch_out = c.sc;
        rs.X = p.N;
        rs.r = sm;
        rs.wgs = g.row.wgs;
        rs.narrow = g.row.narrow ? 1 : 0;
    }
    if (g.col.wgs > 0) {
        // out(x, y) = C[x][n_main + y] = sum_k op(A)[x][k] * op(B)[k][n_main + y]
        cs.big = c.A;
        cs.ld_big = p.lda;
        cs.batch_big = c.sa;
        if (p.transb) {
            cs.small = c.B + (long long)n_main * p.ldb;
            cs.s_y = p.ldb;
            cs.s_k = 1;
        } else {
            cs.small = c.B + n_main;
            cs.s_y = 1;
            cs.s_k = p.ldb;
        }
        cs.batch_small = c.sb;
        cs.out = c.C + n_main;
        cs.o_x = p.ldc;
        cs.o_y = 1;
        cs.batch_out = c.sc;
        cs.X = m_main;
        cs.r = sn;
        cs.wgs = g.col.wgs;
        cs.narrow = g.col.narrow ? 1 : 0;
    }
    // An x-contiguous stream reads non-temporally when the other strip shares
    // the launch (it keeps L2 for that strip's staged operand).
    rs.nt = cs.wgs > 0 ? 1 : 0;
    cs.nt = rs.wgs > 0 ? 1 : 0;
    const long long wgs = (long long)rs.wgs + cs.wgs;
    if (wgs == 0) return hipSuccess;
    if (wgs > INT_MAX) return hipErrorInvalidValue;
    constexpr int kMaxY = 65535;
    for (int z0 = 0; z0 < p.batch; z0 += kMaxY) {
        const int nz = p.batch - z0 < kMaxY ? p.batch - z0 : kMaxY;
        a.z0 = z0;
        void *args[] = {&a};
        hipError_t e = hipLaunchKernel(strip_kernel(p), dim3((unsigned)wgs, (unsigned)nz),
                                       dim3(sgemm::kStripThreads), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The part of a call the tiles compute: its first M - sm rows and N - sn
// columns (same operands, strides and workspace).
Call main_part(const Call &c, int sm, int sn)
{
    Call m = c;
    m.p = sgemm::main_block(c.p, sm, sn);
    return m;
}

// The selector's inputs and its choice, remembered per thread for the last
// few distinct calls: the search over variants, splits and strips costs about
// 2 us of host time, which a stream of small products would pay on every call.
struct PlanKey {
    Problem p;
    int cus, aligned16, lds_ok;
    long long ws;
};
struct PlanEntry {
    PlanKey key;
    Choice choice;
    int valid;
};
constexpr int kPlanCacheEntries = 8;
thread_local PlanEntry t_plan_cache[kPlanCacheEntries];
thread_local int t_plan_next;

Choice cached_plan(const Problem &p, int cus, bool aligned16, bool lds_ok, long long ws)
{
    PlanKey key;
    memset(&key, 0, sizeof(key));  // padding too: keys compare bytewise
    key.p = p;
    key.cus = cus;
    key.aligned16 = aligned16 ? 1 : 0;
    key.lds_ok = lds_ok ? 1 : 0;
    key.ws = ws;
    for (int i = 0; i < kPlanCacheEntries; ++i)
        if (t_plan_cache[i].valid && memcmp(&t_plan_cache[i].key, &key, sizeof(key)) == 0)
            return t_plan_cache[i].choice;
    const Choice ch = sgemm::select_plan(kVariants, kNumVariants, p, cus, aligned16, lds_ok, ws);
    PlanEntry &e = t_plan_cache[t_plan_next];
    t_plan_next = (t_plan_next + 1) % kPlanCacheEntries;
    e.key = key;
    e.choice = ch;
    e.valid = 1;
    return ch;
}

int plan_for(const Call &c, int cus, sgemm_cfg *out)
{
    if (!out || !sgemm::sizes_ok(c.p)) return hipErrorInvalidValue;
    const long long ws = c.ws_bytes > (size_t)LLONG_MAX ? LLONG_MAX : (long long)c.ws_bytes;
    const Choice ch = cached_plan(c.p, cus > 0 ? cus : 256, rows_aligned16(c),
                                  sgemm::direct_lds_ok(c.p), ws);
    if (ch.id < 0) return hipErrorInvalidValue;
    return sgemm::finish_cfg(kVariants[ch.id], ch.id, c.p, ch.splits, ch.strip_m, ch.strip_n, out)
               ? hipSuccess
               : hipErrorInvalidValue;
}

// A forced configuration completed for this call (see sgemm_f32_cfg_geometry).
int forced_cfg(const Problem &p, const sgemm_cfg *force, sgemm_cfg *cfg)
{
    if (!sgemm::sizes_ok(p)) return hipErrorInvalidValue;
    if (force->id < 0 || force->id >= kNumVariants || force->group_m < 0) return hipErrorInvalidValue;
    const int id = force->id;
    if (!kVariants[id].fn[sgemm::op_index(p)] || !sgemm::variant_fits(kVariants[id], p))
        return hipErrorInvalidValue;
    const int group_m = force->group_m, xcd = force->xcd_remap ? 1 : 0;
    if (!sgemm::finish_cfg(kVariants[id], id, p, force->splits, force->strip_m, force->strip_n, cfg))
        return hipErrorInvalidValue;
    cfg->group_m = group_m;
    cfg->xcd_remap = xcd;
    return hipSuccess;
}

int run(const Call &c, hipStream_t stream, const sgemm_cfg *force)
{
    hipError_t e = validate(c);
    if (e != hipSuccess) return e;
    const Problem &p = c.p;
    sgemm_cfg cfg;
    if (force) {
        const int r = forced_cfg(p, force, &cfg);
        if (r != hipSuccess) return r;
    }
    if (p.M == 0 || p.N == 0 || p.batch == 0) return hipSuccess;
    if (!reads_operands(c)) {
        // alpha * (empty or ignored product) + beta * C
        if (c.beta == 1.0f) return hipSuccess;
        return launch_reduce(c, 0, 0.0f, stream);
    }
    int id = 0;
    // (arguments are checked before the first HIP call)
    if (force && (unsigned long long)cfg.workspace_bytes > c.ws_bytes) return hipErrorInvalidValue;
    int cus = 0;
    e = device_cus(&cus);
    if (e != hipSuccess) return e;
    if (force) {
        id = cfg.id;
    } else {
        const int r = plan_for(c, cus, &cfg);
        if (r != hipSuccess) return r;
        id = cfg.id;
    }
    const Call m = main_part(c, cfg.strip_m, cfg.strip_n);
    if (m.p.M > 0 && m.p.N > 0) {
        e = launch_gemm(kVariants[id], cfg, m, stream);
        if (e == hipSuccess && cfg.splits > 1) e = launch_reduce(m, cfg.splits, c.alpha, stream);
        if (e != hipSuccess) return e;
    }
    return launch_strips(c, cfg.strip_m, cfg.strip_n, cus, stream);
}

Call make_call(int transa, int transb, int M, int N, int K, float alpha,
               const float *A, int lda, long long sa, const float *B, int ldb, long long sb,
               float beta, float *C, int ldc, long long sc, int batch, void *ws, size_t ws_bytes)
{
    Call c;
    c.p = Problem{transa, transb, M, N, K, lda, ldb, ldc, batch};
    c.alpha = alpha;
    c.beta = beta;
    c.A = A;
    c.B = B;
    c.C = C;
    c.sa = sa;
    c.sb = sb;
    c.sc = sc;
    c.ws = ws;
    c.ws_bytes = ws ? ws_bytes : 0;
    return c;
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

int sgemm_f32_variant_ops(int id)
{
    if (id < 0 || id >= kNumVariants) return -1;
    int m = 0;
    for (int o = 0; o < 4; ++o)
        if (kVariants[id].fn[o]) m |= 1 << o;
    return m;
}

const char *sgemm_f32_version(void)
{
    return "libsgemm 0.5.0 gfx950 fp32 (mfma_f32_32x32x2; NN/NT/TN/TT, alpha/beta, split-K, strided batch, "
           "edge strips; valu comparison)";
}

int sgemm_f32_plan(int transa, int transb, int M, int N, int K, int lda, int ldb, int ldc, int batch,
                   int num_cus, long long workspace_bytes, sgemm_cfg *out)
{
    // operands are assumed to start 16-byte aligned (as allocations do)
    Call c = make_call(transa, transb, M, N, K, 1.0f, nullptr, lda, 0, nullptr, ldb, 0, 0.0f,
                       nullptr, ldc, 0, batch, nullptr, 0);
    c.ws_bytes = workspace_bytes > 0 ? (size_t)workspace_bytes : 0;
    return plan_for(c, num_cus, out);
}

int sgemm_f32_cfg_geometry(int transa, int transb, int M, int N, int K, int lda, int ldb, int ldc,
                           int batch, sgemm_cfg *cfg)
{
    if (!cfg) return hipErrorInvalidValue;
    const Problem p{transa, transb, M, N, K, lda, ldb, ldc, batch};
    sgemm_cfg out;
    const int r = forced_cfg(p, cfg, &out);
    if (r == hipSuccess) *cfg = out;
    return r;
}

int sgemm_f32_workspace_size(int transa, int transb, int M, int N, int K, int lda, int ldb, int ldc,
                             int batch, size_t *bytes)
{
    if (!bytes) return hipErrorInvalidValue;
    int cus = 0;
    hipError_t e = device_cus(&cus);
    if (e != hipSuccess) return e;
    sgemm_cfg cfg;
    const int r = sgemm_f32_plan(transa, transb, M, N, K, lda, ldb, ldc, batch, cus, LLONG_MAX, &cfg);
    if (r != hipSuccess) return r;
    *bytes = (size_t)cfg.workspace_bytes;
    return hipSuccess;
}

int sgemm_f32_query(int transa, int transb, int M, int N, int K,
                    const float *A, int lda, long long stride_a,
                    const float *B, int ldb, long long stride_b,
                    float *C, int ldc, long long stride_c,
                    int batch, void *workspace, size_t workspace_bytes, sgemm_cfg *out)
{
    if (!out) return hipErrorInvalidValue;
    const Call c = make_call(transa, transb, M, N, K, 1.0f, A, lda, stride_a, B, ldb, stride_b, 0.0f,
                             C, ldc, stride_c, batch, workspace, workspace_bytes);
    hipError_t e = validate(c);
    if (e != hipSuccess) return e;
    int cus = 0;
    e = device_cus(&cus);
    if (e != hipSuccess) return e;
    return plan_for(c, cus, out);
}

int sgemm_f32_ex(int transa, int transb, int M, int N, int K, float alpha,
                 const float *A, int lda, long long stride_a,
                 const float *B, int ldb, long long stride_b,
                 float beta, float *C, int ldc, long long stride_c, int batch,
                 void *workspace, size_t workspace_bytes, hipStream_t stream, const sgemm_cfg *cfg)
{
    const Call c = make_call(transa, transb, M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b, beta,
                             C, ldc, stride_c, batch, workspace, workspace_bytes);
    return run(c, stream, cfg);
}

int sgemm_f32_ex_noalloc(int transa, int transb, int M, int N, int K, float alpha,
                         const float *A, int lda, long long stride_a,
                         const float *B, int ldb, long long stride_b,
                         float beta, float *C, int ldc, long long stride_c, int batch,
                         hipStream_t stream, const sgemm_cfg *cfg)
{
    Call c = make_call(transa, transb, M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b, beta,
                       C, ldc, stride_c, batch, nullptr, 0);
    // arguments are checked before the first HIP call (the scratch lookup)
    const hipError_t v = validate(c);
    if (v != hipSuccess) return v;
    if (cfg) {
        // a forced split must fit in the scratch (checked before any HIP call)
        sgemm_cfg geo;
        const int r = forced_cfg(c.p, cfg, &geo);
        if (r != hipSuccess) return r;
        if ((unsigned long long)geo.workspace_bytes > (unsigned long long)SGEMM_SCRATCH_BYTES)
            return hipErrorOutOfMemory;
    }
    void *ws = nullptr;
    const hipError_t e = device_scratch(&ws);
    if (e != hipSuccess) return e;
    c.ws = ws;
    c.ws_bytes = SGEMM_SCRATCH_BYTES;
    return run(c, stream, cfg);
}

int sgemm_f32_strided_batched(int transa, int transb, int M, int N, int K, float alpha,
                              const float *A, int lda, long long stride_a,
                              const float *B, int ldb, long long stride_b,
                              float beta, float *C, int ldc, long long stride_c, int batch,
                              void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return sgemm_f32_ex(transa, transb, M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b, beta,
                        C, ldc, stride_c, batch, workspace, workspace_bytes, stream, nullptr);
}

int sgemm_f32_gemm(int transa, int transb, int M, int N, int K, float alpha,
                   const float *A, int lda, const float *B, int ldb,
                   float beta, float *C, int ldc,
                   void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return sgemm_f32_ex(transa, transb, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1,
                        workspace, workspace_bytes, stream, nullptr);
}

int sgemm_f32(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
              float *C, int ldc, hipStream_t stream)
{
    return sgemm_f32_ex(SGEMM_OP_N, SGEMM_OP_N, M, N, K, 1.0f, A, lda, 0, B, ldb, 0, 0.0f, C, ldc, 0, 1,
                        nullptr, 0, stream, nullptr);
}

}  // extern "C"

#if SGEMM_TIMELINE
// Timeline build only: the clock readings of the direct-load kernel (the
// layout is documented in sgemm_timeline.h).
extern "C" {

int sgemm_f32_timeline_layout(int *phase_wgs, int *slice_wgs, int *waves, int *slices)
{
    if (!phase_wgs || !slice_wgs || !waves || !slices) return (int)hipErrorInvalidValue;
    static_assert(sgemm::kTlPhaseValues == 6, "phase readings per workgroup");
    *phase_wgs = sgemm::kTlPhaseWgs;
    *slice_wgs = sgemm::kTlSliceWgs;
    *waves = sgemm::kTlWaves;
    *slices = sgemm::kTlSlices;
    return (int)hipSuccess;
}

int sgemm_f32_timeline_read(unsigned long long *phase, size_t phase_bytes, unsigned int *slice,
                            size_t slice_bytes)
{
    if (phase_bytes > sizeof(sgemm::g_tl_phase) || slice_bytes > sizeof(sgemm::g_tl_slice) ||
        (phase_bytes && !phase) || (slice_bytes && !slice))
        return (int)hipErrorInvalidValue;
    hipError_t e = hipSuccess;
    if (phase_bytes)
        e = hipMemcpyFromSymbol(phase, HIP_SYMBOL(sgemm::g_tl_phase), phase_bytes, 0,
                                hipMemcpyDeviceToHost);
    if (e == hipSuccess && slice_bytes)
        e = hipMemcpyFromSymbol(slice, HIP_SYMBOL(sgemm::g_tl_slice), slice_bytes, 0,
                                hipMemcpyDeviceToHost);
    return (int)e;
}

int sgemm_f32_timeline_clock_khz(int *khz)
{
    if (!khz) return (int)hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
    return (int)e;
}

int sgemm_f32_timeline_clear(void)
{
    constexpr size_t kBytes = sizeof(sgemm::g_tl_slice) > sizeof(sgemm::g_tl_phase)
                                  ? sizeof(sgemm::g_tl_slice) : sizeof(sgemm::g_tl_phase);
    static const unsigned char zeros[kBytes] = {};
    hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(sgemm::g_tl_phase), zeros, sizeof(sgemm::g_tl_phase), 0,
                                     hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpyToSymbol(HIP_SYMBOL(sgemm::g_tl_slice), zeros, sizeof(sgemm::g_tl_slice), 0,
                              hipMemcpyHostToDevice);
    return (int)e;
}

}  // extern "C"
#endif
