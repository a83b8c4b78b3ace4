// Single-precision GEMM on CDNA4 matrix cores (gfx950): C = A x B, row-major.
//
// Hierarchy (the global -> shared -> register tiling of "4.1 CUDA GEMM
// operator performance optimization", sections 4-6, re-derived for 64-wide
// wavefronts and the FP32 MFMA instruction instead of per-thread FMAs):
//
//   workgroup  BM x BN tile of C; walks K in BK-deep slices staged in LDS,
//              two LDS buffers, one barrier per slice (the register + shared
//              double buffering of section 9, made one slice deeper, below).
//   wavefront  (BM/WAVES_M) x (BN/WAVES_N) sub-tile = RM x NB blocks of 32x32,
//              accumulated by v_mfma_f32_32x32x2_f32 (4096 FLOP each) in AGPRs.
//
// MFMA operand layout (32x32x2, fp32): lane l supplies A[l%32][l/32] and
// B[l/32][l%32]; the 16 accumulators of lane l hold D[i][l%32] for
// i = 8*(r/4) + 4*(l/32) + r%4, r = 0..15.
//
// Two re-indexings make every LDS fragment read a 16-byte ds_read_b128 and
// every interior store a 16-byte global store, without changing what is
// summed:
//  * k permutation: within an 8-deep k group, MFMA step t (0..3) takes k = t
//    from lanes 0-31 and k = 4 + t from lanes 32-63.  A lane therefore reads
//    A[row][kb + 4*(l/32) .. +3] as one float4 (A stays row-major in LDS, with
//    4 floats of padding per row so the 32 rows of a read fall in distinct
//    banks).  Each k still meets its own row of B: the sum is the same set of
//    products in another order.
//  * column interleave: the NB column blocks of a wave own columns
//    c0 + NB*j + cb (j = 0..31, cb < NB).  One NB-wide LDS read of B row k at
//    c0 + NB*(l%32) gives lane l its operand for all NB blocks, and in the
//    epilogue a lane holds NB adjacent columns of each of its rows.
//
// Edges: elements outside M x K or K x N are loaded as zeros (a zero adds
// nothing), so every wave runs every barrier; stores are masked to i < M,
// j < N (the zero-padding and guard of the DD2360 workbook, section 14.3).
#pragma once

#include "common.hpp"

namespace sgemm {

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

// STAGE_AT: the k group of a slice after which the next slice is written to
// LDS (the pipelined order described at the main loop).
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGE_AT>
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
    static_assert(STAGE_AT >= 0 && STAGE_AT < BK / 8,
                  "the LDS write must follow one of the slice's k groups");
    static_assert(A_VECS * NT * 4 == BM * BK, "A tile must split evenly into float4 per thread");
    static_assert(B_VECS * NT * 4 == BK * BN, "B tile must split evenly into float4 per thread");
    static_assert(NT % (BK / 4) == 0 && NT % (BN / 4) == 0, "load columns must not depend on v");
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGE_AT>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
sgemm_mfma_kernel(GemmArgs g)
{
    typedef MfmaTraits<BM, BN, BK, WAVES_M, WAVES_N, STAGE_AT> T;
    constexpr int NT = T::NT, WTM = T::WTM, WTN = T::WTN, RM = T::RM, NB = T::NB;
    constexpr int LDA_S = T::LDA_S, LDB_S = T::LDB_S;
    constexpr int A_VECS = T::A_VECS, B_VECS = T::B_VECS;
    constexpr int A_ROW_VECS = BK / 4;  // float4 per A-tile row
    constexpr int B_ROW_VECS = BN / 4;  // float4 per B-tile row
    constexpr int G = BK / 8;           // 8-deep k groups per slice
    typedef typename FragB<NB>::T fragb_t;

    __shared__ __attribute__((aligned(16))) float As[2][BM * LDA_S];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB_S];

    // An (empty) AGPR clobber tells the register allocator this kernel uses
    // AGPRs, so MFMAs keep their accumulators there instead of in ArchVGPRs
    // shared with the LDS fragments, staging registers and addresses.
    asm volatile("" ::: "a0");

    const Work w = map_work(g);
    locate<false, false>(g, w);
    const float *__restrict__ A = g.A;
    const float *__restrict__ B = g.B;
    const int M = g.M, N = g.N, K = g.K, lda = g.lda, ldb = g.ldb;
    const int m0 = w.tm * BM, n0 = w.tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const bool tile_inside = (m0 + BM <= M) && (n0 + BN <= N);

    f32x16 acc[RM][NB];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---- global -> registers ------------------------------------------------
    // A thread loads A_VECS float4 of the A slice (rows idx / A_ROW_VECS,
    // columns 4 * (idx % A_ROW_VECS)) and B_VECS float4 of the B slice; its
    // byte offsets inside a slice are fixed for the whole loop, and each slice
    // only moves the (wave-uniform) base.  Interior slices (tile inside M x N,
    // all BK columns below K) use 16-byte loads without checks.  Edge slices
    // go through buffer resources whose extent ends at the matrix's last
    // element (A[M-1][K-1], B[K-1][N-1]): dword loads past the end return
    // zero, which zero-fills the rows of A at or past M and the rows of B at
    // or past K, and a select zeroes the columns at or past K (A) or N (B)
    // that lie inside the extent (leading-dimension padding or the next row).
    uint32_t a_off[A_VECS], b_off[B_VECS];
#pragma unroll
    for (int v = 0; v < A_VECS; ++v) {
        const int idx = tid + v * NT;
        a_off[v] = 4u * ((uint32_t)(idx / A_ROW_VECS) * (uint32_t)lda + 4u * (uint32_t)(idx % A_ROW_VECS));
    }
#pragma unroll
    for (int v = 0; v < B_VECS; ++v) {
        const int idx = tid + v * NT;
        b_off[v] = 4u * ((uint32_t)(idx / B_ROW_VECS) * (uint32_t)ldb + 4u * (uint32_t)(idx % B_ROW_VECS));
    }
    const int a_col = 4 * (tid % A_ROW_VECS);  // first column of a thread's A float4 in the slice
    const int b_col = 4 * (tid % B_ROW_VECS);  // first column of a thread's B float4 in the tile

    auto gload = [&](int kt, f32x4(&ra)[A_VECS], f32x4(&rb)[B_VECS]) {
        const int k0 = kt * BK;
        const float *abase = A + (int64_t)m0 * lda + k0;
        const float *bbase = B + (int64_t)k0 * ldb + n0;
        if (tile_inside && k0 + BK <= K) {
#pragma unroll
            for (int v = 0; v < A_VECS; ++v)
                ra[v] = *reinterpret_cast<const f32x4u *>(
                    reinterpret_cast<const char *>(abase) + a_off[v]);
#pragma unroll
            for (int v = 0; v < B_VECS; ++v)
                rb[v] = *reinterpret_cast<const f32x4u *>(
                    reinterpret_cast<const char *>(bbase) + b_off[v]);
        } else {
            const auto ar = make_rsrc(abase, 4 * ((int64_t)(M - 1 - m0) * lda + (K - k0)));
            const auto br = make_rsrc(bbase, 4 * ((int64_t)(K - 1 - k0) * ldb + (N - n0)));
#pragma unroll
            for (int v = 0; v < A_VECS; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = buffer_load_f32(ar, a_off[v] + 4u * e);
                    ra[v][e] = (k0 + a_col + e < K) ? x : 0.0f;
                }
#pragma unroll
            for (int v = 0; v < B_VECS; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = buffer_load_f32(br, b_off[v] + 4u * e);
                    rb[v][e] = (n0 + b_col + e < N) ? x : 0.0f;
                }
        }
    };

    // ---- registers -> LDS buffer `buf` ---------------------------------------
    auto sstore = [&](int buf, const f32x4(&ra)[A_VECS], const f32x4(&rb)[B_VECS]) {
#pragma unroll
        for (int v = 0; v < A_VECS; ++v) {
            const int idx = tid + v * NT;
            *reinterpret_cast<f32x4 *>(&As[buf][(idx / A_ROW_VECS) * LDA_S + 4 * (idx % A_ROW_VECS)]) = ra[v];
        }
#pragma unroll
        for (int v = 0; v < B_VECS; ++v) {
            const int idx = tid + v * NT;
            *reinterpret_cast<f32x4 *>(&Bs[buf][(idx / B_ROW_VECS) * LDB_S + 4 * (idx % B_ROW_VECS)]) = rb[v];
        }
    };

    // LDS race check build: this thread's words of buffer `buf` (those sstore
    // writes) set to NaN once the buffer is free.
    auto poison = [&](int buf) {
        if constexpr (kLdsPoison) {
#pragma unroll
            for (int v = 0; v < A_VECS; ++v) {
                const int idx = tid + v * NT;
                lds_poison(&As[buf][(idx / A_ROW_VECS) * LDA_S + 4 * (idx % A_ROW_VECS)], 4);
            }
#pragma unroll
            for (int v = 0; v < B_VECS; ++v) {
                const int idx = tid + v * NT;
                lds_poison(&Bs[buf][(idx / B_ROW_VECS) * LDB_S + 4 * (idx % B_ROW_VECS)], 4);
            }
            lds_poison_done();
        }
    };

    // ---- LDS -> fragments -> MFMA ---------------------------------------------
    // Fragments of one 8-deep k group: RM float4 of A (4 k values of one row
    // per lane) and 4 NB-wide reads of B (one k row each).
    struct Frag {
        f32x4 a[RM];
        fragb_t b[4];
    };
    const float *as0 = &As[0][(wm * WTM + (lane & 31)) * LDA_S + 4 * (lane >> 5)];
    const float *bs0 = &Bs[0][(4 * (lane >> 5)) * LDB_S + wn * WTN + NB * (lane & 31)];
    auto read_frag = [&](int buf, int g, Frag &f) {
        const float *as = as0 + buf * (BM * LDA_S) + 8 * g;
        const float *bs = bs0 + buf * (BK * LDB_S) + 8 * g * LDB_S;
#pragma unroll
        for (int i = 0; i < RM; ++i)
            f.a[i] = *reinterpret_cast<const f32x4 *>(as + i * 32 * LDA_S);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            f.b[t] = *reinterpret_cast<const fragb_t *>(bs + t * LDB_S);
    };
    auto mfma_frag = [&](const Frag &f) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        f.a[i][t], frag_elem<NB>(f.b[t], j), acc[i][j], 0, 0, 0);
    };

    // ---- main loop ---------------------------------------------------------------
    const int nk_real = (K + BK - 1) / BK;
    f32x4 ra0[A_VECS], rb0[B_VECS];
    // Pipelined order.  Two register staging sets: the global loads of
    // slice kt+2 are issued at the start of slice kt, and slice kt+1
    // (fetched one slice earlier) is written to the other LDS buffer after
    // k group STAGE_AT, in the shadow of the remaining MFMAs.  A fetch has
    // about one and a half slices of MFMA time to arrive, and the end of a
    // slice holds only the barrier.  The LDS buffer written during slice
    // kt was last read in slice kt-1, which every wave has left (the
    // barrier closing it).  Fragments ping-pong between two register sets:
    // the reads of group g+1 are issued before the MFMAs of group g.
    f32x4 ra1[A_VECS], rb1[B_VECS];
    // Slices are taken in pairs so the staging set of each is known at
    // compile time; an odd count gets one more slice lying wholly past K,
    // whose loads all read as zero, so the MFMA chain of the loop body is
    // unconditional and its zero products leave the sums unchanged.
    const int nk = (nk_real + 1) & ~1;
    auto slice = [&](int kt, auto &ra_next, auto &rb_next, auto &ra_free, auto &rb_free) {
        const int cur = kt & 1;
        // (buffer cur ^ 1 was last read in slice kt-1, which every wave has left)
        if (kt + 1 < nk) poison(cur ^ 1);
        if (kt + 2 < nk) gload(kt + 2, ra_free, rb_free);
        Frag f[2];
        read_frag(cur, 0, f[0]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g + 1 < G) read_frag(cur, g + 1, f[(g + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frag(f[g & 1]);
            __builtin_amdgcn_sched_barrier(0);
            if (g == STAGE_AT && kt + 1 < nk) sstore(cur ^ 1, ra_next, rb_next);
        }
        __syncthreads();
    };
    if (nk > 0) {
        gload(0, ra0, rb0);
        sstore(0, ra0, rb0);
        gload(1, ra1, rb1);
        __syncthreads();
        for (int kt = 0; kt < nk; kt += 2) {
            slice(kt, ra1, rb1, ra0, rb0);
            slice(kt + 1, ra0, rb0, ra1, rb1);
        }
    }

    // ---- epilogue -----------------------------------------------------------------
    // Lane l holds rows 8*(r/4) + 4*(l/32) + r%4 of each 32-row block and NB
    // adjacent columns c0 + NB*(l%32) .. +NB-1.
    float *__restrict__ C = g.C;
    const int ldc = g.ldc;
    const int col = n0 + wn * WTN + NB * (lane & 31);
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row >= M) continue;
            float v[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) v[j] = acc[i][j][r];
            store_row<NB>(C + (int64_t)row * ldc + col, col, N, v, g.alpha, g.beta);
        }
    }
}

}  // namespace sgemm
