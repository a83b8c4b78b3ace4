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

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel families. */
#define SGEMM_KERNEL_MFMA 0 /* matrix cores: v_mfma_f32_32x32x2_f32 (v_mfma_f32_16x16x4_f32
                               for the four-stage 64 x 64 tiles and the 16 x 16 tiles) */
#define SGEMM_KERNEL_VALU 1 /* vector FMA: the 8 x 8 tiles that split K over lane
                               pairs and waves, and the 128 x 128 register-blocked
                               tile kept only as a measured comparison */

/* Operand layouts (transa, transb). */
#define SGEMM_OP_N 0 /* the operand as stored, row-major */
#define SGEMM_OP_T 1 /* its transpose */

/* A launch configuration: what a variant is and how it is launched. */
typedef struct sgemm_cfg {
    int id;        /* variant index, 0 .. sgemm_f32_num_variants()-1 */
    int kernel;    /* SGEMM_KERNEL_MFMA or SGEMM_KERNEL_VALU */
    int bm, bn, bk;       /* workgroup tile: BM x BN outputs, BK-deep K slices */
    int waves_m, waves_n; /* wavefront grid inside a workgroup (the 32 x 32,
                             16 x 16 and 8 x 8 variants that split K inside the
                             workgroup report waves_m = their wave count,
                             waves_n = 1, and bk = the k of one group: four
                             MFMA steps, or one k per lane pair) */
    int group_m;   /* raster: tile rows per group, walked column by column
                      (0 = plain row-major order over tiles) */
    int xcd_remap; /* 1: give each XCD a contiguous run of logical tiles */
    int splits;    /* K split across workgroups (1 = none) */
    /* filled in by plan/query: */
    int k_chunk;   /* K range of one split */
    int grid;      /* workgroups launched: tiles_m * tiles_n * splits * batch */
    int threads;   /* threads per workgroup */
    int lds_bytes; /* LDS per workgroup */
    int tiles_m, tiles_n;
    long long workspace_bytes; /* workspace the configuration needs */
    /* Edge strips (0 = none): the last strip_m rows of C, and the last
       strip_n columns of the rows above them, are computed by a
       bandwidth-bound strip kernel instead of by tiles, and the tile
       geometry above (tiles_m, tiles_n, grid, splits, workspace_bytes)
       describes the (M - strip_m) x (N - strip_n) block that remains.  At
       most 4 each.  Chosen by plan/query; an input of sgemm_f32_ex.  A strip
       whose streamed operand runs along k takes 16-row workgroups instead of
       32 when the launch's strips have fewer workgroups (times the batch
       count) than the device has compute units; the two forms add K in
       different fixed orders, so a strip's bits depend on the batch count
       and the device's CU count (and are reproducible for both fixed). */
    int strip_m, strip_n;
    /* The cost model's figures for this variant (reported, never read): */
    int fixed_ns;       /* fixed cost of one tile (ns) */
    int spill_permille; /* slice cost, x1000 of the L2-resident one, once the
                           operand rows and columns one XCD's tiles read exceed
                           its L2, over one round (0 = not modelled) */
    int spill_full_permille; /* the same over several rounds */
    int coresident;     /* workgroups per CU whose fixed costs the model overlaps */
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
 * Pointers must be 4-byte aligned; any dword-aligned start and stride runs
 * (16-byte loads and stores need only dword alignment on gfx950; rows that
 * start 16-byte aligned also allow direct global-to-LDS loads).  Limits:
 * M, N, K, lda, ldb, ldc <= INT_MAX - 1024.  The LDS-tiled kernels use
 * 32-bit byte offsets inside one K slice and serve lda <= 2^22 - 64 and
 * ldb <= 2^25 - 512; larger leading dimensions run on the kernels that
 * address in 64 bits (the 32 x 32, 16 x 16 and 8 x 8 tiles that split K
 * inside the workgroup, and the edge-strip kernel), more slowly.
 *
 * Semantics of degenerate sizes: M == 0 or N == 0 does nothing; K == 0 sets
 * the M x N block of C to zero (an empty sum).
 *
 * Ownership: A, B and C belong to the caller and must stay valid until the
 * work on `stream` completes.  The library allocates no device memory, keeps
 * no pointer after returning and never synchronises; it is re-entrant.  This
 * entry point has no workspace, so it never splits K.
 *
 * Errors (returned before anything is launched):
 *   hipErrorInvalidValue  negative size; a leading dimension below its
 *                         minimum or above its limit; a null or misaligned
 *                         pointer for an operand with a non-zero extent; C
 *                         overlapping A or B; a grid too large to launch.
 *   otherwise             the error of the device query or of the launch.
 * Faults during execution surface at the caller's next synchronisation.
 */
int sgemm_f32(int M, int N, int K,
              const float *A, int lda,
              const float *B, int ldb,
              float *C, int ldc,
              hipStream_t stream);

/*
 * sgemm_f32_gemm: the BLAS-style product
 *
 *   C = alpha * op(A) x op(B) + beta * C,   op(A) M x K, op(B) K x N,
 *
 * where op(X) = X for SGEMM_OP_N and the transpose of X for SGEMM_OP_T.  All
 * matrices are row-major; a transposed operand is the one stored the other
 * way round, which is how a row-major matrix looks to a column-major library
 * (DD2360 workbook, Module 15, section 15.2: passing a transpose flag instead
 * of moving data), and how the products with a transposed operand in
 * attention arise ("4.1 CUDA GEMM operator performance optimization",
 * section 1.2).  No operand is copied: transposed operands are loaded as
 * they are stored.
 *
 *   transa    SGEMM_OP_N: A is M x K (lda >= max(1,K));
 *             SGEMM_OP_T: A is stored K x M (lda >= max(1,M)).
 *   transb    SGEMM_OP_N: B is K x N (ldb >= max(1,N));
 *             SGEMM_OP_T: B is stored N x K (ldb >= max(1,K)).
 *   alpha, beta  scalars.  C is read only when beta != 0; with beta == 0 its
 *             previous contents (NaN included) are ignored.  alpha == 0 or
 *             K == 0 gives C = beta * C without reading A or B (beta == 1
 *             then launches nothing).
 *   workspace, workspace_bytes
 *             optional device memory (16-byte aligned, not overlapping A, B
 *             or C; NULL with 0 bytes for none) that lets the selector split K
 *             across workgroups when the output has too few tiles to fill the
 *             chip.  Each split writes its partial product to the workspace
 *             and a second kernel adds the partials in a fixed order, so the
 *             result is reproducible bit for bit.  The library uses at most
 *             workspace_bytes; sgemm_f32_workspace_size gives what the
 *             selector would like.  The workspace is scratch: its contents
 *             on entry do not matter, and the caller must not touch it until
 *             the work on `stream` completes.
 * Limits: as sgemm_f32; the LDS-tiled kernels serve a leading dimension up
 * to 2^22 - 64 for a k-contiguous operand (A, or a transposed B) and up to
 * 2^25 - 512 for the other (B, or a transposed A), larger ones run on the
 * 64-bit kernels.  Otherwise as sgemm_f32 (the two are the same for
 * transa = transb = SGEMM_OP_N, alpha = 1, beta = 0 and no workspace).
 */
int sgemm_f32_gemm(int transa, int transb, int M, int N, int K,
                   float alpha,
                   const float *A, int lda,
                   const float *B, int ldb,
                   float beta,
                   float *C, int ldc,
                   void *workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * sgemm_f32_strided_batched: `batch` independent products
 *
 *   C_z = alpha * op(A_z) x op(B_z) + beta * C_z,   z = 0 .. batch-1,
 *
 * with X_z = X + z * stride_x (elements), as in the batched matrix products
 * of multi-head attention ("4.1 CUDA GEMM operator performance
 * optimization", section 1.2), in one launch.  Strides are >= 0 (0 reuses one
 * operand for every entry); stride_c must keep the C_z apart
 * (stride_c >= (M-1)*ldc + N when batch > 1).  batch == 0 does nothing.  The
 * memory spanned by all C_z must not overlap that of all A_z or all B_z.
 * Workspace as for sgemm_f32_gemm (a split needs room for every entry's
 * partials).  Other arguments as sgemm_f32_gemm.
 */
int sgemm_f32_strided_batched(int transa, int transb, int M, int N, int K,
                              float alpha,
                              const float *A, int lda, long long stride_a,
                              const float *B, int ldb, long long stride_b,
                              float beta,
                              float *C, int ldc, long long stride_c,
                              int batch,
                              void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * sgemm_f32_workspace_size: *bytes = the workspace the selector's preferred
 * configuration uses for these sizes on the current device, assuming
 * 16-byte aligned operands (0 when it does not split K).  Passing that much
 * to sgemm_f32_gemm / sgemm_f32_strided_batched lets them run it.
 */
int sgemm_f32_workspace_size(int transa, int transb, int M, int N, int K,
                             int lda, int ldb, int ldc, int batch, size_t *bytes);

/*
 * sgemm_f32_ex: sgemm_f32_strided_batched with a forced configuration, for
 * sweeps and for the measured comparison kernels.  cfg == NULL behaves as
 * sgemm_f32_strided_batched.  Otherwise cfg->id selects the variant (see
 * sgemm_f32_variant), cfg->splits the requested K split (<= 1: none; the
 * split actually used is reported by sgemm_f32_plan), cfg->group_m and
 * cfg->xcd_remap the tile order, and cfg->strip_m, cfg->strip_n the edge
 * strips (0 .. min(4, M) rows and 0 .. min(4, N) columns; 0 for none); the
 * other fields are ignored.  Returns hipErrorInvalidValue for an id out of
 * range, a variant not compiled for the operand layout, an LDS-tiled
 * variant for leading dimensions past its limits (2^22 - 64 for a
 * k-contiguous operand, 2^25 - 512 for the other, 2^23 for an
 * index-contiguous operand of a variant with 64-deep slices, bk = 64),
 * cfg->group_m < 0,
 * strips out of range, or a workspace too small for the split.  Same
 * arguments, ownership and errors as sgemm_f32_strided_batched.
 */
int sgemm_f32_ex(int transa, int transb, int M, int N, int K,
                 float alpha,
                 const float *A, int lda, long long stride_a,
                 const float *B, int ldb, long long stride_b,
                 float beta,
                 float *C, int ldc, long long stride_c,
                 int batch,
                 void *workspace, size_t workspace_bytes,
                 hipStream_t stream, const sgemm_cfg *cfg);

/* Bytes of device scratch the library holds per GPU for sgemm_f32_ex_noalloc. */
#define SGEMM_SCRATCH_BYTES (32u << 20)

/*
 * sgemm_f32_ex_noalloc: sgemm_f32_ex without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Nothing is
 * allocated on any call: a K split keeps its partial products in a scratch
 * array of SGEMM_SCRATCH_BYTES that the library holds in the device memory of
 * each GPU it runs on, from the first call on that GPU (which looks up the
 * array's address there) until the process ends.  The caller still passes
 * the operands and C as for sgemm_f32_ex.
 *
 *   cfg == NULL  the selector's choice among the plans whose partials fit in
 *                the scratch (larger products run without a K split, as
 *                sgemm_f32_strided_batched does with no workspace).
 *   cfg != NULL  the forced configuration, as sgemm_f32_ex; a K split whose
 *                partials need more than SGEMM_SCRATCH_BYTES is refused with
 *                hipErrorOutOfMemory before anything is launched.
 *
 * The result is the one sgemm_f32_ex gives for the same plan with a
 * workspace of SGEMM_SCRATCH_BYTES (bit for bit).  The scratch keeps the
 * last call's partials; every split writes its partials before they are
 * read, so nothing in it has to start at zero.  Every call on one GPU shares
 * that GPU's scratch: calls that may overlap on one GPU (several streams or
 * host threads) race on it and must be serialised by the caller.  Other
 * arguments, ownership and errors as sgemm_f32_ex; the stream's device must
 * be the current device.
 */
int sgemm_f32_ex_noalloc(int transa, int transb, int M, int N, int K,
                         float alpha,
                         const float *A, int lda, long long stride_a,
                         const float *B, int ldb, long long stride_b,
                         float beta,
                         float *C, int ldc, long long stride_c,
                         int batch,
                         hipStream_t stream, const sgemm_cfg *cfg);

/*
 * sgemm_f32_plan: the configuration the library chooses for these sizes on
 * a device with `num_cus` compute units (<= 0 means 256), given
 * `workspace_bytes` of workspace and 16-byte aligned operands.  Pure host
 * logic, no HIP call.  Writes *out; returns hipErrorInvalidValue for invalid
 * sizes, layouts or leading dimensions, or out == NULL.  The geometry follows
 * the round-up-and-guard rule (DD2360 workbook, Module 6, section 6.3):
 * tiles_m = ceil(M'/BM), tiles_n = ceil(N'/BN), grid = tiles_m * tiles_n *
 * splits * batch, where M' = M - strip_m and N' = N - strip_n are the sizes
 * left to the tiles when the selector hands a few edge rows or columns to the
 * strip kernel (strip_m = M mod BM or strip_n = N mod BN when that is at most
 * 4 and the cost model prefers it; all of M or N when it is that small).
 */
int sgemm_f32_plan(int transa, int transb, int M, int N, int K,
                   int lda, int ldb, int ldc, int batch,
                   int num_cus, long long workspace_bytes, sgemm_cfg *out);

/*
 * sgemm_f32_cfg_geometry: completes a forced configuration.  Reads cfg->id,
 * cfg->splits, cfg->group_m, cfg->xcd_remap, cfg->strip_m and cfg->strip_n
 * (as sgemm_f32_ex does) and fills in the rest as sgemm_f32_plan would for
 * that variant, requested split and strips: the split actually used,
 * k_chunk, the grid and the workspace bytes it needs.  Pure host logic.
 * Returns hipErrorInvalidValue for invalid sizes, an id out of range, a
 * variant not compiled for the operand layout, cfg->group_m < 0 or strips
 * out of range.
 */
int sgemm_f32_cfg_geometry(int transa, int transb, int M, int N, int K,
                           int lda, int ldb, int ldc, int batch, sgemm_cfg *cfg);

/*
 * sgemm_f32_query: the configuration sgemm_f32_ex(..., cfg = NULL) would
 * launch for these arguments on the current device (queries the device once
 * and caches it).  Same validation as the launch.
 */
int sgemm_f32_query(int transa, int transb, int M, int N, int K,
                    const float *A, int lda, long long stride_a,
                    const float *B, int ldb, long long stride_b,
                    float *C, int ldc, long long stride_c,
                    int batch, void *workspace, size_t workspace_bytes,
                    sgemm_cfg *out);

/* Number of compiled variants, and the description of variant `id`. */
int sgemm_f32_num_variants(void);
int sgemm_f32_variant(int id, sgemm_cfg *out);

/*
 * sgemm_f32_variant_ops: bit (transa + 2*transb) is set when variant `id` is
 * compiled for that operand layout; -1 for an id out of range.
 */
int sgemm_f32_variant_ops(int id);

/* Library version string (static storage). */
const char *sgemm_f32_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_H */
