// Single-precision GEMM on CDNA4 matrix cores (gfx950): C = A x B, row-major.
//
// Hierarchy (the global -> shared -> register tiling of "4.1 CUDA GEMM
// operator performance optimization", sections 4-6, re-derived for 64-wide
// wavefronts and the FP32 MFMA instruction instead of per-thread FMAs):
//
//   workgroup  BM x BN tile of C, walks K in BK-deep slices staged in LDS,
//              double buffered: the next slice is fetched from global memory
//              into registers while the current one is multiplied, then
//              written to the other LDS buffer; one barrier per slice (the
//              register + shared double buffering of section 9).
//   wavefront  (BM/WAVES_M) x (BN/WAVES_N) sub-tile = RM x NB blocks of 32x32,
//              accumulated by v_mfma_f32_32x32x2_f32 (4096 FLOP each).
//
// MFMA operand layout (32x32x2, fp32): lane l supplies A[l%32][l/32] and
// B[l/32][l%32]; the 16 accumulators of lane l hold D[i][l%32] for
// i = 8*(r/4) + 4*(l/32) + r%4, r = 0..15.
//
// Two re-indexings make every LDS read a 16-byte ds_read_b128 and every
// interior store a 16-byte global store, without changing what is summed:
//  * k permutation: within an 8-deep k group, MFMA step t (0..3) takes k = t
//    from lanes 0-31 and k = 4 + t from lanes 32-63.  A lane therefore reads
//    A[row][kb + 4*(l/32) .. +3] as one float4 (A stays row-major in LDS).
//    Each k still meets its own row of B, so the sum is the same set of
//    products, only in another order.
//  * column interleave: the NB column blocks of a wave own columns
//    c0 + NB*j + cb (j = 0..31, cb < NB).  One NB-wide LDS read of B row k at
//    c0 + NB*(l%32) gives lane l its operand for all NB blocks, and in the
//    epilogue a lane holds NB adjacent columns of each of its rows.
//
// Edges: elements outside M x K or K x N are loaded as zeros (a zero adds
// nothing), so every wave runs every barrier; stores are masked to i < M,
// j < N (the zero-padding and guard of the DD2360 workbook, section 14.3).
// Tiles entirely inside the matrices take an unchecked path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Linear workgroup id -> (tile row, tile column).
//
// The dispatcher hands workgroups to the 8 XCDs round-robin by linear id, and
// each XCD has its own L2.  With xcd_remap, the workgroups that land on one
// XCD get a contiguous run of logical ids, so tiles that share A rows and B
// columns share an L2.  group_m > 0 then walks the logical ids down groups of
// group_m tile rows, column by column, so a run of consecutive ids covers a
// compact block of tiles instead of one long tile row.
__device__ __forceinline__ void map_tile(int wg, int nwg, int tiles_m, int tiles_n,
                                         int group_m, int xcd_remap, int &tm, int &tn)
{
    if (xcd_remap) {
        constexpr int NX = 8;
        const int x = wg % NX, idx = wg / NX;
        const int q = nwg / NX, r = nwg % NX;
        wg = x * q + (x < r ? x : r) + idx;
    }
    if (group_m > 0) {
        const int per_group = group_m * tiles_n;
        const int g = wg / per_group;
        const int first = g * group_m;
        const int rows = min(tiles_m - first, group_m);
        const int in = wg - g * per_group;
        tm = first + in % rows;
        tn = in / rows;
    } else {
        tm = wg / tiles_n;
        tn = wg - tm * tiles_n;
    }
}

template <int NB> struct FragB;
template <> struct FragB<1> { typedef float T; };
template <> struct FragB<2> { typedef f32x2 T; };
template <> struct FragB<4> { typedef f32x4 T; };

template <int NB>
__device__ __forceinline__ float frag_elem(const typename FragB<NB>::T &v, int cb)
{
    if constexpr (NB == 1) return v;
    else return v[cb];
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool VEC>
struct MfmaTraits {
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int RM = WTM / 32;
    static constexpr int NB = WTN / 32;
    static constexpr int LDA_S = BK + 4;      // LDS row stride of the A tile (floats)
    static constexpr int LDB_S = BN;          // LDS row stride of the B tile (floats)
    static constexpr int A_VECS = BM * BK / 4 / NT;
    static constexpr int B_VECS = BK * BN / 4 / NT;
    static constexpr int LDS_FLOATS = 2 * (BM * LDA_S + BK * LDB_S);
    static_assert(WTM % 32 == 0 && RM >= 1, "wave tile rows must be a multiple of 32");
    static_assert(NB == 1 || NB == 2 || NB == 4, "wave tile columns must be 32, 64 or 128");
    static_assert(BK % 8 == 0, "BK must be a multiple of 8");
    static_assert(A_VECS * NT * 4 == BM * BK, "A tile must split evenly into float4 per thread");
    static_assert(B_VECS * NT * 4 == BK * BN, "B tile must split evenly into float4 per thread");
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool VEC>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
sgemm_mfma_kernel(int M, int N, int K,
                  const float *__restrict__ A, int lda,
                  const float *__restrict__ B, int ldb,
                  float *__restrict__ C, int ldc,
                  int tiles_m, int tiles_n, int group_m, int xcd_remap)
{
    typedef MfmaTraits<BM, BN, BK, WAVES_M, WAVES_N, VEC> T;
    constexpr int NT = T::NT, WTM = T::WTM, WTN = T::WTN, RM = T::RM, NB = T::NB;
    constexpr int LDA_S = T::LDA_S, LDB_S = T::LDB_S;
    constexpr int A_VECS = T::A_VECS, B_VECS = T::B_VECS;
    constexpr int A_ROW_VECS = BK / 4;  // float4 per A-tile row
    constexpr int B_ROW_VECS = BN / 4;  // float4 per B-tile row
    typedef typename FragB<NB>::T fragb_t;

    __shared__ __attribute__((aligned(16))) float As[2][BM * LDA_S];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB_S];

    int tm, tn;
    map_tile(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, xcd_remap, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const bool tile_inside = (m0 + BM <= M) && (n0 + BN <= N);

    const float *Ablk = A + (int64_t)m0 * lda;
    const float *Bblk = B + n0;

    f32x16 acc[RM][NB];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    f32x4 ra[A_VECS], rb[B_VECS];

    // global -> registers, zero outside the matrices
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
        const bool inside = tile_inside && (k0 + BK <= K);
#pragma unroll
        for (int v = 0; v < A_VECS; ++v) {
            const int idx = tid + v * NT;
            const int row = idx / A_ROW_VECS, c = 4 * (idx % A_ROW_VECS);
            const float *p = Ablk + (int64_t)row * lda + (k0 + c);
            if (VEC && inside) {
                ra[v] = *reinterpret_cast<const f32x4 *>(p);
            } else if (!VEC && inside) {
#pragma unroll
                for (int e = 0; e < 4; ++e) ra[v][e] = p[e];
            } else if (VEC && m0 + row < M && k0 + c + 3 < K) {
                ra[v] = *reinterpret_cast<const f32x4 *>(p);
            } else {
                const bool rv = m0 + row < M;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ra[v][e] = (rv && k0 + c + e < K) ? p[e] : 0.0f;
            }
        }
#pragma unroll
        for (int v = 0; v < B_VECS; ++v) {
            const int idx = tid + v * NT;
            const int kr = idx / B_ROW_VECS, c = 4 * (idx % B_ROW_VECS);
            const float *p = Bblk + (int64_t)(k0 + kr) * ldb + c;
            if (VEC && inside) {
                rb[v] = *reinterpret_cast<const f32x4 *>(p);
            } else if (!VEC && inside) {
#pragma unroll
                for (int e = 0; e < 4; ++e) rb[v][e] = p[e];
            } else if (VEC && k0 + kr < K && n0 + c + 3 < N) {
                rb[v] = *reinterpret_cast<const f32x4 *>(p);
            } else {
                const bool kv = k0 + kr < K;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rb[v][e] = (kv && n0 + c + e < N) ? p[e] : 0.0f;
            }
        }
    };

    // registers -> LDS buffer `buf`
    auto sstore = [&](int buf) {
#pragma unroll
        for (int v = 0; v < A_VECS; ++v) {
            const int idx = tid + v * NT;
            const int row = idx / A_ROW_VECS, c = 4 * (idx % A_ROW_VECS);
            *reinterpret_cast<f32x4 *>(&As[buf][row * LDA_S + c]) = ra[v];
        }
#pragma unroll
        for (int v = 0; v < B_VECS; ++v) {
            const int idx = tid + v * NT;
            const int kr = idx / B_ROW_VECS, c = 4 * (idx % B_ROW_VECS);
            *reinterpret_cast<f32x4 *>(&Bs[buf][kr * LDB_S + c]) = rb[v];
        }
    };

    // one BK slice from LDS buffer `buf` into the accumulators
    auto compute = [&](int buf) {
        const float *as = &As[buf][(wm * WTM + (lane & 31)) * LDA_S + 4 * (lane >> 5)];
        const float *bs = &Bs[buf][(4 * (lane >> 5)) * LDB_S + wn * WTN + NB * (lane & 31)];
#pragma unroll
        for (int kb = 0; kb < BK; kb += 8) {
            f32x4 a[RM];
            fragb_t b[4];
#pragma unroll
            for (int i = 0; i < RM; ++i)
                a[i] = *reinterpret_cast<const f32x4 *>(as + i * 32 * LDA_S + kb);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                b[t] = *reinterpret_cast<const fragb_t *>(bs + (kb + t) * LDB_S);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < RM; ++i)
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            a[i][t], frag_elem<NB>(b[t], j), acc[i][j], 0, 0, 0);
        }
    };

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) gload(kt + 1);
            compute(cur);
            if (kt + 1 < nk) sstore(cur ^ 1);
            __syncthreads();
        }
    }

    // epilogue: lane holds rows 8*(r/4) + 4*(l/32) + r%4 of each 32-row block,
    // and NB adjacent columns c0 + NB*(l%32) .. +NB-1
    const int col = n0 + wn * WTN + NB * (lane & 31);
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row >= M) continue;
            float *p = C + (int64_t)row * ldc + col;
            if (VEC && NB == 4 && col + 3 < N) {
                f32x4 v = {acc[i][0][r], acc[i][NB > 1 ? 1 : 0][r],
                           acc[i][NB > 2 ? 2 : 0][r], acc[i][NB > 3 ? 3 : 0][r]};
                *reinterpret_cast<f32x4 *>(p) = v;
            } else if (VEC && NB == 2 && col + 1 < N) {
                f32x2 v = {acc[i][0][r], acc[i][NB > 1 ? 1 : 0][r]};
                *reinterpret_cast<f32x2 *>(p) = v;
            } else {
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    if (col + j < N) p[j] = acc[i][j][r];
            }
        }
    }
}

}  // namespace sgemm
