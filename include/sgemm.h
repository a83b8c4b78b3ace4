/*
 * libsgemm: single-precision GEMM for AMD Instinct MI355X (gfx950).
 *
 *   C = A x B,  A is M x K, B is K x N, C is M x N, all row-major float32.
 *
 * The operation is the one defined in "4.1 CUDA GEMM operator performance
 * optimization" (section 1.1 "What GEMM computes": C = A x B with 2*M*N*K
 * floating-point operations) with the row-major indexing of its naive kernel
 * (section 3.1) generalised to leading dimensions:
 *
 *   C[i*ldc + j] = sum_{k<K} A[i*lda + k] * B[k*ldb + j]   for i < M, j < N.
 *
 * The host workflow (device memory owned by the caller, asynchronous launch on
 * a stream, errors returned from the API call and execution faults surfacing
 * at the next synchronisation) follows the DD2360 workbook "Applied GPU
 * Programming", Module 5 (sections 5.4-5.6) and Module 16 (streams).
 *
 * Every entry point returns a hipError_t value as int: 0 (hipSuccess) on
 * success.
 */
#ifndef SGEMM_H
#define SGEMM_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel families. */
#define SGEMM_KERNEL_MFMA 0 /* matrix cores: v_mfma_f32_32x32x2_f32 */
#define SGEMM_KERNEL_VALU 1 /* vector FMA, kept only as a measured comparison */

/* A launch configuration: what a variant is and how it is launched. */
typedef struct sgemm_cfg {
    int id;        /* variant index, 0 .. sgemm_f32_num_variants()-1 */
    int kernel;    /* SGEMM_KERNEL_MFMA or SGEMM_KERNEL_VALU */
    int bm, bn, bk;       /* workgroup tile: BM x BN outputs, BK-deep K slices */
    int waves_m, waves_n; /* wavefront grid inside a workgroup */
    int group_m;   /* raster: tile rows per group, walked column by column
                      (0 = plain row-major order over tiles) */
    int xcd_remap; /* 1: give each XCD a contiguous run of logical tiles */
    /* filled in by plan/query: */
    int grid;      /* workgroups launched */
    int threads;   /* threads per workgroup */
    int lds_bytes; /* LDS per workgroup */
    int tiles_m, tiles_n;
} sgemm_cfg;

/*
 * sgemm_f32: C = A x B on `stream` (0 = the null stream).
 *
 * Arguments
 *   M, N, K   sizes, >= 0.
 *   A, lda    device pointer to A, row-major M x K, row stride lda >= max(1,K).
 *   B, ldb    device pointer to B, row-major K x N, row stride ldb >= max(1,N).
 *   C, ldc    device pointer to C, row-major M x N, row stride ldc >= max(1,N).
 *             C is overwritten and never read; elements j >= N of each row
 *             (the padding up to ldc) are left untouched.
 *   stream    a HIP stream of the current device.
 * Pointers must be 4-byte aligned; any dword-aligned start and stride runs on
 * the same kernels (16-byte loads and stores need only dword alignment on
 * gfx950).  Limits: M, N, K <= INT_MAX - 1024, lda <= 2^22 - 64,
 * ldb <= 2^25 - 512 (byte offsets inside one K slice are 32-bit).
 *
 * Semantics of degenerate sizes: M == 0 or N == 0 does nothing; K == 0 sets
 * the M x N block of C to zero (an empty sum).
 *
 * Ownership: A, B and C belong to the caller and must stay valid until the
 * work on `stream` completes.  The library allocates no device memory, keeps
 * no pointer after returning and never synchronises; it is re-entrant.
 *
 * Errors (returned before anything is launched):
 *   hipErrorInvalidValue  negative size; a leading dimension below its
 *                         minimum; a null or misaligned pointer for an operand
 *                         with a non-zero extent; C overlapping A or B; a grid
 *                         too large to launch.
 *   otherwise             the error of the device query or of the launch.
 * Faults during execution surface at the caller's next synchronisation.
 */
int sgemm_f32(int M, int N, int K,
              const float *A, int lda,
              const float *B, int ldb,
              float *C, int ldc,
              hipStream_t stream);

/*
 * sgemm_f32_ex: sgemm_f32 with a forced configuration, for sweeps and for the
 * measured comparison kernels.  cfg == NULL behaves as sgemm_f32.  Otherwise
 * cfg->id selects the variant (see sgemm_f32_variant; an id out of range, or
 * cfg->group_m < 0, returns hipErrorInvalidValue) and cfg->group_m and
 * cfg->xcd_remap set the tile order; the other fields are ignored.  Same
 * arguments, ownership and errors as sgemm_f32.
 */
int sgemm_f32_ex(int M, int N, int K,
                 const float *A, int lda,
                 const float *B, int ldb,
                 float *C, int ldc,
                 hipStream_t stream, const sgemm_cfg *cfg);

/*
 * sgemm_f32_plan: the configuration sgemm_f32 chooses for these sizes on a
 * device with `num_cus` compute units (<= 0 means 256).  Pure host logic, no
 * HIP call.  Writes *out; returns hipErrorInvalidValue for invalid sizes or
 * leading dimensions, or out == NULL.  The geometry fields follow the
 * round-up-and-guard rule (DD2360 workbook, Module 6, section 6.3):
 * tiles_m = ceil(M/BM), tiles_n = ceil(N/BN), grid = tiles_m * tiles_n.
 */
int sgemm_f32_plan(int M, int N, int K, int lda, int ldb, int ldc,
                   int num_cus, sgemm_cfg *out);

/*
 * sgemm_f32_query: the configuration sgemm_f32 would launch for these
 * arguments on the current device (queries the device once and caches it).
 */
int sgemm_f32_query(int M, int N, int K,
                    const float *A, int lda,
                    const float *B, int ldb,
                    float *C, int ldc, sgemm_cfg *out);

/* Number of compiled variants, and the description of variant `id`. */
int sgemm_f32_num_variants(void);
int sgemm_f32_variant(int id, sgemm_cfg *out);

/* Library version string (static storage). */
const char *sgemm_f32_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_H */
