// Small tiles with K split inside the workgroup.
//
// A product whose output has few tiles leaves most compute units idle (the
// wave quantisation of "4.1 CUDA GEMM operator performance optimization",
// section 12.5, and the single-block problem of the "cuda-kernels" README,
// where one 128x128 output with K = 32768 is one block however fast its inner
// loop).  Splitting K across workgroups needs a workspace and a second pass;
// here K is split across the W waves of one workgroup instead, so the partial
// results meet in LDS:
//
//  * a workgroup owns one 32x32 tile of C (one v_mfma_f32_32x32x2_f32 block),
//    four times as many tiles as 64x64 ones;
//  * wave w accumulates the tile over its own K range (a multiple of 8), its
//    fragments loaded straight from global memory into registers: for the MFMA
//    step t of an 8-deep group, lanes 0-31 give k = t and lanes 32-63 k = 4+t,
//    so a lane's four A values (and B values) of a group are 4 successive k of
//    one row or column: one 16-byte load for an operand stored k-contiguous
//    (A, or a transposed B), four 4-byte loads that 32 lanes make into one
//    128-byte row segment for an operand stored index-contiguous (B, or a
//    transposed A);
//  * the W partial tiles are added through LDS in wave order, so a result is
//    the same on every run, and written with alpha/beta like the other
//    kernels' epilogue.
//
// No operand goes through LDS, so the kernel has no barrier in its K loop; the
// loads of the next four groups are in flight while the MFMAs of the current
// ones run.  Rows past M and columns past N are read as row M-1 and column
// N-1 (in bounds, never stored); k past the wave's range reads as zero.
#pragma once

#include "common.hpp"

namespace sgemm {

template <int W> struct SkTraits {
    static constexpr int BM = 32, BN = 32;
    static constexpr int NT = W * 64;
    static constexpr int LDS_FLOATS = W * 16 * 64;
    static constexpr int DEPTH = 4;  // 8-deep k groups in flight per wave
};

template <int W, bool TA, bool TB>
__global__ void __launch_bounds__(W * 64) sgemm_mfma_sk_kernel(GemmArgs g)
{
    typedef SkTraits<W> T;
    constexpr int D = T::DEPTH;
    __shared__ __attribute__((aligned(16))) float red[T::LDS_FLOATS];

    if constexpr (kLdsPoison) {
        // LDS race check build: the partial-tile area starts as NaN everywhere
        const int w0 = threadIdx.x >> 6, l0 = threadIdx.x & 63;
#pragma unroll
        for (int r = 0; r < 16; ++r) lds_poison(&red[(w0 * 16 + r) * 64 + l0], 1);
        lds_poison_done();
        __syncthreads();
    }

    const Work wk = map_work(g);
    locate<TA, TB>(g, wk);
    const float *__restrict__ A = g.A;
    const float *__restrict__ B = g.B;
    const int M = g.M, N = g.N, K = g.K, lda = g.lda, ldb = g.ldb;
    const int m0 = wk.tm * 32, n0 = wk.tn * 32;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l31 = lane & 31, h = lane >> 5;

    // this wave's K range [kb, ke): nfull whole 8-deep groups, then rem < 8
    // more k (only in the last wave, when K is not a multiple of 8)
    const int kc = (((K + W - 1) / W) + 7) & ~7;
    const int kb = wave * kc;
    const int ke = min(K, kb + kc);
    const int len = ke > kb ? ke - kb : 0;
    const int nfull = len >> 3;
    const int rem = len & 7;

    const int ia = min(m0 + l31, M - 1);  // row of op(A) this lane feeds
    const int jb = min(n0 + l31, N - 1);  // column of op(B) this lane feeds
    // op(A)[ia][k] = pa[k * sa]; op(B)[k][jb] = pb[k * sb]
    const float *pa = TA ? A + ia : A + (int64_t)ia * lda;
    const float *pb = TB ? B + (int64_t)jb * ldb : B + jb;
    const int64_t sa = TA ? lda : 1;
    const int64_t sb = TB ? 1 : ldb;

    struct Frag {
        f32x4 a, b;
    };
    // whole group q of this wave: k = kb + 8q + 4h + t, t = 0..3.  The loop
    // below has no branch and no lane-dependent condition, so the compiler
    // waits for each group's loads alone, with the later groups still in
    // flight.
    auto load = [&](int q, Frag &f) {
        const int k = kb + 8 * q + 4 * h;
        if constexpr (!TA) f.a = *reinterpret_cast<const f32x4u *>(pa + k);
        else {
#pragma unroll
            for (int t = 0; t < 4; ++t) f.a[t] = pa[(int64_t)(k + t) * sa];
        }
        if constexpr (TB) f.b = *reinterpret_cast<const f32x4u *>(pb + k);
        else {
#pragma unroll
            for (int t = 0; t < 4; ++t) f.b[t] = pb[(int64_t)(k + t) * sb];
        }
    };
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    auto mma = [&](const Frag &f) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[t], f.b[t], acc, 0, 0, 0);
    };

    if (nfull > 0) {
        // prefetch indices past the last whole group reload it (in bounds,
        // never multiplied in)
        const int last = nfull - 1;
        Frag f[D];
#pragma unroll
        for (int d = 0; d < D; ++d) load(min(d, last), f[d]);
        int q0 = 0;
        for (; q0 + D <= nfull; q0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                mma(f[d]);
                load(min(q0 + D + d, last), f[d]);
            }
        }
        // fewer than D whole groups left, already in f[0..]
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (q0 + d < nfull) mma(f[d]);
    }
    if (rem > 0) {
        // the ragged group: k past ke reads a clamped address and becomes 0
        const int k = kb + 8 * nfull + 4 * h;
        Frag f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int kk = min(k + t, ke - 1);
            const float x = pa[(int64_t)kk * sa], y = pb[(int64_t)kk * sb];
            f.a[t] = k + t < ke ? x : 0.0f;
            f.b[t] = k + t < ke ? y : 0.0f;
        }
        mma(f);
    }

    // partial tiles -> LDS as [wave][register][lane]; then each thread adds
    // the W partials of its outputs in wave order
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    __syncthreads();
    float *__restrict__ C = g.C;
    const int ldc = g.ldc;
    for (int o = tid; o < 16 * 64; o += W * 64) {
        const int r = o >> 6, ln = o & 63;
        float s = red[r * 64 + ln];
#pragma unroll
        for (int w = 1; w < W; ++w) s += red[(w * 16 + r) * 64 + ln];
        // register r of lane ln holds D[8*(r/4) + 4*(ln/32) + r%4][ln%32]
        const int row = m0 + 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3);
        const int col = n0 + (ln & 31);
        if (row < M && col < N) {
            float *p = C + (int64_t)row * ldc + col;
            *p = g.beta != 0.0f ? g.alpha * s + g.beta * *p : g.alpha * s;
        }
    }
}

}  // namespace sgemm
