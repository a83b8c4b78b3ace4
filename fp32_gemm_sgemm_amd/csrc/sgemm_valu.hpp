// Vector-FMA single-precision GEMM, kept only as a measured comparison for the
// matrix-core kernel.  It is the classic register-blocked design of
// "4.1 CUDA GEMM operator performance optimization" carried to 64-wide
// wavefronts: a 128x128 workgroup tile (section 4), an 8x8 register tile per
// thread split into four 4x4 quadrants so that each LDS read is a 16-byte
// vector and a 16-lane row of threads reads 256 contiguous bytes (sections
// 5-8), A stored transposed in LDS (section 7.3) and register + LDS double
// buffering with one barrier per K slice (section 9).
#pragma once

#include "common.hpp"

namespace sgemm {

struct ValuTraits {
    static constexpr int BM = 128, BN = 128, BK = 8;
    static constexpr int NT = 256;             // 16 x 16 threads, 4 waves
    static constexpr int LDA_S = BM + 4;       // transposed A tile: [BK][BM + 4]
    static constexpr int LDB_S = BN;           // B tile: [BK][BN]
    static constexpr int LDS_FLOATS = 2 * (BK * LDA_S + BK * LDB_S);
};

__global__ void __launch_bounds__(256)
sgemm_valu_kernel(GemmArgs g)
{
    typedef ValuTraits T;
    constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
    constexpr int LDA_S = T::LDA_S, LDB_S = T::LDB_S;
    typedef f32x4 f4;

    __shared__ __attribute__((aligned(16))) float As[2][BK * LDA_S];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB_S];

    const Work w = map_work(g);
    locate<false, false>(g, w);
    const float *__restrict__ A = g.A;
    const float *__restrict__ B = g.B;
    const int M = g.M, N = g.N, K = g.K, lda = g.lda, ldb = g.ldb;
    const int m0 = w.tm * BM, n0 = w.tn * BN;
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const bool tile_inside = (m0 + BM <= M) && (n0 + BN <= N);

    // cooperative load mapping: one float4 of A and one of B per thread
    const int a_row = tid >> 1, a_col = 4 * (tid & 1);     // A tile 128 x 8
    const int b_row = tid >> 5, b_col = 4 * (tid & 31);    // B tile 8 x 128

    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    f4 ra, rb;
    // Interior slices: 16-byte loads (dword-aligned suffices).  Edge slices:
    // dword loads through buffer resources ending at the matrices' last
    // elements (rows past M or K read as zero) plus a select for columns at
    // or past K (A) or N (B).
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
        const float *pa = A + (int64_t)(m0 + a_row) * lda + (k0 + a_col);
        const float *pb = B + (int64_t)(k0 + b_row) * ldb + (n0 + b_col);
        if (tile_inside && k0 + BK <= K) {
            ra = *reinterpret_cast<const f32x4u *>(pa);
            rb = *reinterpret_cast<const f32x4u *>(pb);
        } else {
            const float *abase = A + (int64_t)m0 * lda + k0;
            const float *bbase = B + (int64_t)k0 * ldb + n0;
            const auto ar = make_rsrc(abase, 4 * ((int64_t)(M - 1 - m0) * lda + (K - k0)));
            const auto br = make_rsrc(bbase, 4 * ((int64_t)(K - 1 - k0) * ldb + (N - n0)));
            const uint32_t ao = 4u * ((uint32_t)a_row * (uint32_t)lda + (uint32_t)a_col);
            const uint32_t bo = 4u * ((uint32_t)b_row * (uint32_t)ldb + (uint32_t)b_col);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xa = buffer_load_f32(ar, ao + 4u * e);
                const float xb = buffer_load_f32(br, bo + 4u * e);
                ra[e] = (k0 + a_col + e < K) ? xa : 0.0f;
                rb[e] = (n0 + b_col + e < N) ? xb : 0.0f;
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int e = 0; e < 4; ++e) As[buf][(a_col + e) * LDA_S + a_row] = ra[e];
        *reinterpret_cast<f4 *>(&Bs[buf][b_row * LDB_S + b_col]) = rb;
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const f4 a0 = *reinterpret_cast<const f4 *>(&As[buf][k * LDA_S + 4 * ty]);
            const f4 a1 = *reinterpret_cast<const f4 *>(&As[buf][k * LDA_S + 64 + 4 * ty]);
            const f4 b0 = *reinterpret_cast<const f4 *>(&Bs[buf][k * LDB_S + 4 * tx]);
            const f4 b1 = *reinterpret_cast<const f4 *>(&Bs[buf][k * LDB_S + 64 + 4 * tx]);
            const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
    };

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if constexpr (kLdsPoison) {
                // LDS race check build: this thread's words of the free buffer
                if (kt + 1 < nk) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) lds_poison(&As[cur ^ 1][(a_col + e) * LDA_S + a_row], 1);
                    lds_poison(&Bs[cur ^ 1][b_row * LDB_S + b_col], 4);
                    lds_poison_done();
                }
            }
            if (kt + 1 < nk) gload(kt + 1);
            compute(cur);
            if (kt + 1 < nk) sstore(cur ^ 1);
            __syncthreads();
        }
    }

    // rows 4*ty + {0..3} and 64 + 4*ty + {0..3}; columns likewise with tx
    float *__restrict__ C = g.C;
    const int ldc = g.ldc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + (i - 4));
        if (row >= M) continue;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int col = n0 + 64 * hh + 4 * tx;
            const float v[4] = {acc[i][4 * hh], acc[i][4 * hh + 1], acc[i][4 * hh + 2], acc[i][4 * hh + 3]};
            store_row<4>(C + (int64_t)row * ldc + col, col, N, v, g.alpha, g.beta);
        }
    }
}

}  // namespace sgemm
