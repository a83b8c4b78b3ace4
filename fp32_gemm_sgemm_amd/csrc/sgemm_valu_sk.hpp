// 8x8 tiles with K split over lane pairs and waves, on the vector FMA unit.
//
// An output too small to give every compute unit a 16x16 tile (128x128 is 64
// of them) runs on a few CUs however fast each one is: the wave quantisation
// of "4.1 CUDA GEMM operator performance optimization", section 12.5, and the
// single-block problem of the "cuda-kernels" README.  Without a workspace K
// cannot be split across workgroups, so this kernel makes the tile smaller
// still, 8x8 (128x128 is 256 of them), and splits K inside the workgroup:
//
//  * lane l of a wave takes one k of each 32-deep group, k = 32 q + l / 2 of
//    the wave's K range; the two lanes of a pair share that k, and half
//    h = l % 2 owns rows 4h..4h+3 of the tile;
//  * a lane loads op(A)[4h+t][k] for its four rows and op(B)[k][4h+t] for
//    four of the eight columns, takes the other four from its partner lane
//    (a cross-lane swap), and adds the 4x8 outer product into 32
//    accumulators with vector FMAs;
//  * the per-CU cost of such small tiles is set by the cache lines each wave
//    load instruction touches, not by the arithmetic: a 32-byte row segment of
//    an index-contiguous operand (B as stored, A transposed) is read by the
//    two lanes of a pair in one 16-byte load each, so every k costs one line
//    per such operand, and a k-contiguous operand (A as stored, B transposed)
//    is read along k, 32 successive k of a row per half wave;
//  * the 32 accumulators of a lane are summed over the 32 lane pairs by a
//    transposing butterfly (each step halves the values a lane keeps), then
//    over the W waves through LDS in wave order, so a result is the same on
//    every run, and written with alpha/beta like the other kernels' epilogue;
//  * where both operands are k-contiguous (A as stored, B transposed) a lane
//    instead takes 4 successive k and loads them from all 8 rows of each
//    operand with 16-byte loads, so a wave reads 1 KiB (8 whole lines) of a
//    row per load: half a line per k for the tile (vsk_kk).
//
// No operand goes through LDS and the K loop has no barrier and no branch
// (one copy of it per load form, chosen once per workgroup): the loads of the
// next DEPTH groups are in flight while the FMAs of the current one run.  Rows past M and columns past N read row M-1 and column
// N-1 (in bounds, never stored); k past the wave's range reads as zero.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace sgemm {

template <int W> struct VskTraits {
    static constexpr int BM = 8, BN = 8;
    static constexpr int NT = W * 64;
    static constexpr int GK = 32;  // k of one group: one per lane pair
    static constexpr int LDS_FLOATS = W * 64;
    static constexpr int DEPTH = 4;  // groups of loads in flight per wave
};

// One of the sums of the tile's 64 outputs over this wave's K range, for
// the lane-pair form: lane l returns output (4 (l % 2) + (l / 2) / 8,
// (l / 2) % 8).  g is located (batch entry and K split applied).
template <int W, bool TA, bool TB>
__device__ __forceinline__ float vsk_pairs(const GemmArgs &g, int m0, int n0, int wave, int lane)
{
    typedef VskTraits<W> T;
    constexpr int GK = T::GK, D = T::DEPTH;
    const float *__restrict__ A = g.A;
    const float *__restrict__ B = g.B;
    const int M = g.M, N = g.N, K = g.K, lda = g.lda, ldb = g.ldb;
    const int pair = lane >> 1, h = lane & 1;

    // this wave's K range [kb, ke): nfull whole groups, then rem < GK more k
    // (only in the last wave, when K is not a multiple of GK)
    const int kc = (((K + W - 1) / W) + GK - 1) & ~(GK - 1);
    const int kb = wave * kc;
    const int ke = min(K, kb + kc);
    const int len = ke > kb ? ke - kb : 0;
    const int nfull = len / GK;
    const int rem = len % GK;

    // op(A)[4h+t][k] = pa[t][k * sa]; op(B)[k][4h+t] = pb[t][k * sb]
    const float *pa[4];
    const float *pb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = min(m0 + 4 * h + t, M - 1);
        const int c = min(n0 + 4 * h + t, N - 1);
        pa[t] = TA ? A + r : A + (int64_t)r * lda;
        pb[t] = TB ? B + (int64_t)c * ldb : B + c;
    }
    const int64_t sa = TA ? lda : 1, sb = TB ? 1 : ldb;
    // an index-contiguous operand's four entries load as one 16-byte vector
    // when the whole tile is inside M (or N); at the last tile they load one by
    // one from clamped addresses.  Both flags are the same for the workgroup.
    const bool vec_a = TA && m0 + T::BM <= M, vec_b = !TB && n0 + T::BN <= N;

    struct Frag {
        float a[4], b[4];
    };
    float acc[4][8];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t][j] = 0.0f;
    auto fma = [&](const Frag &f) {
        // columns 0..7 of op(B)[k]: this lane's four and its partner's
        float b[8];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float o = __shfl_xor(f.b[t], 1);
            b[t] = h ? o : f.b[t];
            b[4 + t] = h ? f.b[t] : o;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[t][j] = __builtin_fmaf(f.a[t], b[j], acc[t][j]);
    };

    // the whole groups, with 16-byte loads of A (VA) or B (VB) or not
    auto run = [&](auto va, auto vb) {
        constexpr bool VA = decltype(va)::value, VB = decltype(vb)::value;
        auto load = [&](int q, Frag &f) {
            const int64_t k = kb + GK * q + pair;
            if constexpr (VA) {
                const f32x4 v = *reinterpret_cast<const f32x4u *>(pa[0] + k * sa);
#pragma unroll
                for (int t = 0; t < 4; ++t) f.a[t] = v[t];
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) f.a[t] = pa[t][k * sa];
            }
            if constexpr (VB) {
                const f32x4 v = *reinterpret_cast<const f32x4u *>(pb[0] + k * sb);
#pragma unroll
                for (int t = 0; t < 4; ++t) f.b[t] = v[t];
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) f.b[t] = pb[t][k * sb];
            }
        };
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
                fma(f[d]);
                load(min(q0 + D + d, last), f[d]);
                // keep each group's loads here, DEPTH groups ahead of their
                // use, rather than sunk to the end of the iteration
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // fewer than D whole groups left, already in f[0..]
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (q0 + d < nfull) fma(f[d]);
    };
    typedef std::true_type Y;
    typedef std::false_type X;
    if (nfull > 0) {
        if (vec_a) {
            if (vec_b) run(Y(), Y());
            else run(Y(), X());
        } else {
            if (vec_b) run(X(), Y());
            else run(X(), X());
        }
    }
    if (rem > 0) {
        // the ragged group: k past ke reads a clamped address and becomes 0
        const int k = kb + GK * nfull + pair;
        const int64_t kk = min(k, ke - 1);
        Frag f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float x = pa[t][kk * sa], y = pb[t][kk * sb];
            f.a[t] = k < ke ? x : 0.0f;
            f.b[t] = k < ke ? y : 0.0f;
        }
        fma(f);
    }

    // sum over the 32 lane pairs of each half.  Value x = 8t + j of a lane is
    // acc[t][j]; the step with offset 2s (s = 16, 8, 4, 2, 1) pairs lanes that
    // differ in lane bit 2s, both add their two copies of values x and x + s
    // (the same sums, as addition commutes), and each keeps the one whose bit
    // s matches that lane bit.  Lane l ends with value l / 2 of half l % 2,
    // summed over the wave in a fixed order.  (Selecting between sums, not
    // between array entries, keeps the compiler from indexing the registers
    // by a lane-dependent value.)
    float v[32];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * t + j] = acc[t][j];
#pragma unroll
    for (int s = 16; s >= 1; s >>= 1) {
        const bool hi = (lane & (2 * s)) != 0;
#pragma unroll
        for (int x = 0; x < s; ++x) {
            const float lo = v[x] + __shfl_xor(v[x], 2 * s);
            const float up = v[x + s] + __shfl_xor(v[x + s], 2 * s);
            v[x] = hi ? up : lo;
        }
    }
    return v[0];
}

// The same for the form where both operands are k-contiguous (A as stored,
// B transposed): lane l takes k = 4l..4l+3 of each 256-deep step of its
// wave's range, loads those four k of all eight rows of op(A) and of op(B)^T
// with one 16-byte load per row (a wave reads 1 KiB of each row: 8 whole
// lines), and adds all 64 products of the tile into 64 accumulators.  Lane
// l returns output (l / 8, l % 8).
template <int W>
__device__ __forceinline__ float vsk_kk(const GemmArgs &g, int m0, int n0, int wave, int lane)
{
    constexpr int GS = 256, D = 2;  // k of one step; steps of loads in flight
    const int M = g.M, N = g.N, K = g.K;
    const int kc = (((K + W - 1) / W) + GS - 1) & ~(GS - 1);
    const int kb = wave * kc;
    const int ke = min(K, kb + kc);
    const int len = ke > kb ? ke - kb : 0;
    const int nfull = len / GS;
    const int rem = len % GS;

    // row i of op(A) and of op(B)^T (clamped): the same for every lane
    const float *pa[8];
    const float *pb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        pa[i] = g.A + (int64_t)min(m0 + i, M - 1) * g.lda;
        pb[i] = g.B + (int64_t)min(n0 + i, N - 1) * g.ldb;
    }
    struct Frag {
        f32x4 a[8], b[8];
    };
    auto load = [&](int st, Frag &f) {
        const int k = kb + GS * st + 4 * lane;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f.a[i] = *reinterpret_cast<const f32x4u *>(pa[i] + k);
            f.b[i] = *reinterpret_cast<const f32x4u *>(pb[i] + k);
        }
    };
    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    auto fma = [&](const Frag &f) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(f.a[i][t], f.b[j][t], acc[i][j]);
    };
    if (nfull > 0) {
        // prefetch indices past the last whole step reload it (in bounds,
        // never multiplied in)
        const int last = nfull - 1;
        Frag f[D];
#pragma unroll
        for (int d = 0; d < D; ++d) load(min(d, last), f[d]);
        int s0 = 0;
        for (; s0 + D <= nfull; s0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                fma(f[d]);
                load(min(s0 + D + d, last), f[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int d = 0; d < D - 1; ++d)
            if (s0 + d < nfull) fma(f[d]);
    }
    if (rem > 0) {
        // the ragged step: k past ke reads a clamped address and becomes 0
        const int k = kb + GS * nfull + 4 * lane;
        Frag f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int kk = min(k + t, ke - 1);
            const bool in = k + t < ke;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = pa[i][kk], y = pb[i][kk];
                f.a[i][t] = in ? x : 0.0f;
                f.b[i][t] = in ? y : 0.0f;
            }
        }
        fma(f);
    }

    // sum over the wave's 64 lanes: the step with offset s (32, 16, ..., 1)
    // pairs lanes that differ in lane bit s; both add their copies of values
    // x and x + s and each keeps the one whose bit s matches that lane bit,
    // so lane l ends with value l = 8i + j
    float v[64];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[8 * i + j] = acc[i][j];
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        const bool hi = (lane & s) != 0;
#pragma unroll
        for (int x = 0; x < s; ++x) {
            const float lo = v[x] + __shfl_xor(v[x], s);
            const float up = v[x + s] + __shfl_xor(v[x + s], s);
            v[x] = hi ? up : lo;
        }
    }
    return v[0];
}

template <int W, bool TA, bool TB>
__global__ void __launch_bounds__(W * 64) sgemm_valu_sk_kernel(GemmArgs g)
{
    typedef VskTraits<W> T;
    constexpr bool KK = !TA && TB;  // both operands k-contiguous
    __shared__ float red[T::LDS_FLOATS];

    if constexpr (kLdsPoison) {
        // LDS race check build: the partial-tile area starts as NaN everywhere
        lds_poison(&red[threadIdx.x], 1);
        lds_poison_done();
        __syncthreads();
    }

    const Work wk = map_work(g);
    locate<TA, TB>(g, wk);
    const int m0 = wk.tm * T::BM, n0 = wk.tn * T::BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    float part;
    if constexpr (KK) part = vsk_kk<W>(g, m0, n0, wave, lane);
    else part = vsk_pairs<W, TA, TB>(g, m0, n0, wave, lane);

    // the waves' partial tiles, added in wave order
    red[wave * 64 + lane] = part;
    __syncthreads();
    if (tid < 64) {
        float s = red[tid];
#pragma unroll
        for (int w = 1; w < W; ++w) s += red[w * 64 + tid];
        const int row = m0 + (KK ? tid >> 3 : 4 * (tid & 1) + (tid >> 4));
        const int col = n0 + (KK ? tid & 7 : (tid >> 1) & 7);
        if (row < g.M && col < g.N) {
            float *p = g.C + (int64_t)row * g.ldc + col;
            *p = g.beta != 0.0f ? g.alpha * s + g.beta * *p : g.alpha * s;
        }
    }
}

}  // namespace sgemm
