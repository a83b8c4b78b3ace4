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
//  * a workgroup owns one MB x MB tile of C: one v_mfma_f32_32x32x2_f32 block
//    (MB = 32, four times as many tiles as 64x64 ones) or one
//    v_mfma_f32_16x16x4_f32 block (MB = 16, four times as many again, for
//    outputs too small to give every compute unit a 32x32 tile);
//  * wave w accumulates the tile over its own K range (a multiple of the group
//    depth GK = 8 or 16), its fragments loaded straight from global memory into
//    registers: for the MFMA step t of a group, lane l gives k = 4h + t of the
//    group, h = l / MB (the half or quarter of the wave whose values the MFMA
//    contracts), so a lane's four A values (and B values) of a group are 4
//    successive k of one row or column: one 16-byte load for an operand stored
//    k-contiguous
//    (A, or a transposed B), four 4-byte loads that the MB lanes of a block
//    make into one row segment for an operand stored index-contiguous (B, or a
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

#include <type_traits>

#include "common.hpp"

namespace sgemm {

template <int W, int MB = 32> struct SkTraits {
    static_assert(MB == 32 || MB == 16, "32x32x2 or 16x16x4 blocks");
    static constexpr int BM = MB, BN = MB;
    static constexpr int REGS = MB == 32 ? 16 : 4;  // accumulators per lane
    static constexpr int GK = MB == 32 ? 8 : 16;    // k of one group (4 MFMA steps)
    static constexpr int NT = W * 64;
    static constexpr int LDS_FLOATS = W * REGS * 64;
    static constexpr int DEPTH = 4;  // k groups in flight per wave
};

template <int W, bool TA, bool TB, int MB = 32>
__global__ void __launch_bounds__(W * 64) sgemm_mfma_sk_kernel(GemmArgs g)
{
    typedef SkTraits<W, MB> T;
    constexpr int D = T::DEPTH, REGS = T::REGS, GK = T::GK;
    typedef typename std::conditional<MB == 32, f32x16, f32x4>::type acc_t;
    __shared__ __attribute__((aligned(16))) float red[T::LDS_FLOATS];

    if constexpr (kLdsPoison) {
        // LDS race check build: the partial-tile area starts as NaN everywhere
        const int w0 = threadIdx.x >> 6, l0 = threadIdx.x & 63;
#pragma unroll
        for (int r = 0; r < REGS; ++r) lds_poison(&red[(w0 * REGS + r) * 64 + l0], 1);
        lds_poison_done();
        __syncthreads();
    }

    const Work wk = map_work(g);
    locate<TA, TB>(g, wk);
    const float *__restrict__ A = g.A;
    const float *__restrict__ B = g.B;
    const int M = g.M, N = g.N, K = g.K, lda = g.lda, ldb = g.ldb;
    const int m0 = wk.tm * MB, n0 = wk.tn * MB;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l31 = lane & (MB - 1), h = MB == 32 ? lane >> 5 : lane >> 4;

    // this wave's K range [kb, ke): nfull whole groups, then rem < GK more k
    // (only in the last wave, when K is not a multiple of GK)
    const int kc = (((K + W - 1) / W) + GK - 1) & ~(GK - 1);
    const int kb = wave * kc;
    const int ke = min(K, kb + kc);
    const int len = ke > kb ? ke - kb : 0;
    const int nfull = len / GK;
    const int rem = len % GK;

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
    // whole group q of this wave: k = kb + GK q + 4h + t, t = 0..3.  The loop
    // below has no branch and no lane-dependent condition, so the compiler
    // waits for each group's loads alone, with the later groups still in
    // flight.
    auto load = [&](int q, Frag &f) {
        const int k = kb + GK * q + 4 * h;
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
    acc_t acc;
#pragma unroll
    for (int r = 0; r < REGS; ++r) acc[r] = 0.0f;
    auto mma = [&](const Frag &f) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (MB == 32)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[t], f.b[t], acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.a[t], f.b[t], acc, 0, 0, 0);
        }
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
        const int k = kb + GK * nfull + 4 * h;
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
    for (int r = 0; r < REGS; ++r) red[(wave * REGS + r) * 64 + lane] = acc[r];
    __syncthreads();
    float *__restrict__ C = g.C;
    const int ldc = g.ldc;
    for (int o = tid; o < REGS * 64; o += W * 64) {
        const int r = o >> 6, ln = o & 63;
        float s = red[r * 64 + ln];
#pragma unroll
        for (int w = 1; w < W; ++w) s += red[(w * REGS + r) * 64 + ln];
        // register r of lane ln holds D[8*(r/4) + 4*(ln/32) + r%4][ln%32] of a
        // 32x32 block, D[4*(ln/16) + r][ln%16] of a 16x16 one
        const int row = m0 + (MB == 32 ? 8 * (r >> 2) + 4 * (ln >> 5) + (r & 3) : 4 * (ln >> 4) + r);
        const int col = n0 + (ln & (MB - 1));
        if (row < M && col < N) {
            float *p = C + (int64_t)row * ldc + col;
            *p = g.beta != 0.0f ? g.alpha * s + g.beta * *p : g.alpha * s;
        }
    }
}

}  // namespace sgemm
