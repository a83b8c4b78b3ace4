// Edge strips: the parts of a product that hold at most four rows or four
// columns of C.
//
// A product whose M (or N) is a multiple of the tile height plus a few rows
// spends a whole tile row on those few rows: 4099^2 outputs in 192^2 tiles are
// 484 workgroups, 1.9 rounds of the chip's 256 compute units, where the
// 4096^2 block alone is one round of 256^2 tiles (the tail effect of the DD2360
// workbook "Applied GPU Programming", Module 17, and the wave quantisation of
// "4.1 CUDA GEMM operator performance optimization", section 12.5).  The host
// then runs the tiled kernel on the (M - sm) x (N - sn) block and this kernel
// on the strips that remain:
//
//   row strip     rows M-sm .. M-1, columns 0 .. N-1        (sm <= 4)
//   column strip  rows 0 .. M-sm-1, columns N-sn .. N-1     (sn <= 4)
//
// Each strip is a product out(x, y) = sum_k big(x, k) * small(y, k) with a
// long index x (a column of C in the row strip, a row of C in the column
// strip) and at most four values of y: its cost is streaming the big operand
// (op(B) for the row strip, op(A) for the column strip) once, so it is bound by
// memory bandwidth, and a matrix-core tile would pad its at most 4 rows to 32.
// It runs on vector FMAs.
//
// A workgroup covers a block of x and all of K; its lanes and waves split K,
// and their partial sums are added in a fixed order (a butterfly of lane
// shuffles, then the waves in order through LDS), so a result is the same on
// every run and no workspace is needed.  The small operand is staged through
// LDS in chunks of K, zero for y past the strip and k past K: the 4 values of y
// at k = 4q + e sit at 16-byte slot e * plane + q, so a lane that reads the 4
// successive k of one quad (KC) and its neighbours touch consecutive slots,
// and the planes are padded so that 8 consecutive k (XC) do not collide.  The big operand is read with non-temporal loads in KC order (each
// element is used once, which leaves L2 to the small operand every workgroup
// re-reads), and in XC order when the launch also holds a KC strip (measured:
// 4099^3's strips 1% faster with them, an XC strip alone 15% slower).
//
// big is read in one of two storage orders:
//   XC ("x contiguous"): big(x, k) = big[k * ld_big + x] (B in a row strip,
//       a transposed A in a column strip).  Lanes run along x, 4 floats each,
//       so 8 lanes read one 128-byte row segment; a workgroup covers 32 x, and
//       its 128 K phases are the 8 lane groups of each of 16 waves.
//   KC ("k contiguous"): big(x, k) = big[x * ld_big + k] (a transposed B in a
//       row strip, A in a column strip).  Lanes run along k, 4 floats each; a
//       wave reads 4 rows, and a workgroup covers 32 rows in 8 row groups
//       times 2 K phases.
// Both keep many loads in flight per compute unit (one workgroup of 16 waves
// each, several independent 16-byte loads per lane), which is what a
// streaming kernel's rate depends on.
#pragma once

#include "common.hpp"

namespace sgemm {

constexpr int kStripMax = 4;         // rows (or columns) of C one strip may hold
constexpr int kStripThreads = 1024;  // 16 waves
constexpr int kStripWaves = kStripThreads / 64;
constexpr int kStripKChunk = 4608;   // K values of the small operand staged at once
// 16-byte slots per residue plane of the staged chunk: a quarter of the chunk
// plus 4, so the planes start 4 banks apart and the 8 different k one XC read
// instruction touches (k, k+1, ..., k+7) fall in distinct banks.
constexpr int kStripPlane = kStripKChunk / 4 + 4;

template <bool B> struct StripTag { static constexpr bool value = B; };

struct Strip {
    const float *big;     // XC: big(x, k) = big[k * ld_big + x]; KC: big[x * ld_big + k]
    const float *small;   // small(y, k) = small[y * s_y + k * s_k]
    float *out;           // out(x, y) = out[x * o_x + y * o_y]
    int64_t batch_big, batch_small, batch_out;  // elements between batch entries
    int64_t ld_big, s_y, s_k, o_x, o_y;
    int X;                // x range
    int r;                // y range, 1 .. kStripMax
    int wgs;              // workgroups of this strip (0: no strip)
    int nt;               // XC order: read big with non-temporal loads
    int narrow;           // 1: 16 x per workgroup, else 32 (KC order only: XC keeps
                          // 128-byte row segments); the host's strip_plan decides
};

// Up to two strips in one launch: workgroups [0, s[0].wgs) take strip 0, the
// next s[1].wgs strip 1; blockIdx.y is the batch entry (from z0 on).
struct StripArgs {
    Strip s[2];
    int K;
    int z0;
    float alpha, beta;
};

template <bool KC>
__device__ __forceinline__ void strip_block(const Strip &s, int wg, int K, int z, float alpha,
                                            float beta, f32x4 *stage)
{
    const float *__restrict__ big = s.big + z * s.batch_big;
    const float *__restrict__ small = s.small + z * s.batch_small;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: KC rows in SGPRs
    const int X = s.X;
    // XB x per workgroup.  XC: XQ = XB/4 lanes cover one row segment, so a
    // wave holds 64/XQ lane groups and the workgroup KPH = 16 * 64/XQ K
    // phases.  KC: RG = XB/4 row groups of 4 rows, times KCP = 16/RG K phases.
    const int xq_bits = s.narrow ? 2 : 3;  // log2(XQ) = log2(RG)
    const int XB = 4 << xq_bits;
    const int XQ = 1 << xq_bits;
    const int LG = 64 >> xq_bits;          // XC lane groups per wave
    const int KPH = LG * kStripWaves;      // XC K phases
    const int KCP = kStripWaves >> xq_bits;  // KC K phases
    const int x0 = wg * XB;

    // KC: acc[row][y]; XC: acc[y][x]
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    // XC: lane group kr (XQ lanes, XB consecutive x) of wave w takes k = kr +
    // LG*w (mod KPH).  KC: wave w reads rows x0 + 4*(w % RG) .. +3 at k =
    // 4*lane + 256*(w / RG) (mod 256*KCP); rows past X are clamped to X-1
    // (read, never stored).
    const int xq = lane & (XQ - 1), kr = lane >> xq_bits;
    const int xc = x0 + 4 * xq;
    const bool x_full = xc + 3 < X;
    const int rg = wave & (XQ - 1), kp = wave >> xq_bits;
    const float *rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int x = min(x0 + 4 * rg + i, X - 1);
        rows[i] = big + (int64_t)x * s.ld_big;
    }

    // LDS race check build: this thread's slots of the stage set to NaN (the
    // stage is free here: before the first chunk, or after a chunk's barrier)
    auto poison_slots = [&]() {
        if constexpr (kLdsPoison) {
            for (int slot = tid; slot < kStripKChunk; slot += kStripThreads) {
                constexpr int Q = kStripKChunk / 4;
                lds_poison(reinterpret_cast<float *>(&stage[(slot / Q) * kStripPlane + slot % Q]), 4);
            }
            lds_poison_done();
        }
    };

    for (int c0 = 0; c0 < K; c0 += kStripKChunk) {
        const int clen = min(K - c0, kStripKChunk);
        poison_slots();
        for (int slot = tid; slot < kStripKChunk; slot += kStripThreads) {
            constexpr int Q = kStripKChunk / 4;
            const int k = 4 * (slot % Q) + slot / Q;
            f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (k < clen) {
                const float *q = small + (int64_t)(c0 + k) * s.s_k;
                if (s.s_y == 1 && s.r == 4) {
                    v = *reinterpret_cast<const f32x4u *>(q);
                } else {
#pragma unroll
                    for (int y = 0; y < 4; ++y) v[y] = y < s.r ? q[y * s.s_y] : 0.0f;
                }
            }
            stage[(slot / Q) * kStripPlane + slot % Q] = v;
        }
        __syncthreads();
        if constexpr (KC) {
            // quads wholly inside K, two in flight; then at most one quad per
            // lane (in the last chunk) that reaches past K, masked
            auto quad = [&](int kk, bool masked) {
                const int k = c0 + kk;
                f32x4 sv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[e] = stage[e * kStripPlane + kk / 4];
                f32x4 v[4];
                if (!masked) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        v[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4u *>(rows[i] + k));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[i][e] = k + e < K ? rows[i][k + e] : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int y = 0; y < 4; ++y) acc[i][y] += v[i][e] * sv[e][y];
            };
            const int kfull = min(clen, K - c0 - 3);  // kk < kfull: k + 3 < K
            int kk = 256 * kp + 4 * lane;
#pragma unroll 2
            for (; kk < kfull; kk += 256 * KCP) quad(kk, false);
            if (kk < clen) quad(kk, true);
        } else {
            auto xc_loop = [&](auto nt) {
                constexpr bool NT = decltype(nt)::value;
                const float *p = big + (int64_t)(c0 + kr + LG * wave) * s.ld_big + xc;
                const int64_t step = (int64_t)KPH * s.ld_big;
#pragma unroll 8
                for (int kk = kr + LG * wave; kk < clen; kk += KPH, p += step) {
                    f32x4 v;
                    if (x_full) {
                        if constexpr (NT)
                            v = __builtin_nontemporal_load(reinterpret_cast<const f32x4u *>(p));
                        else
                            v = *reinterpret_cast<const f32x4u *>(p);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = xc + e < X ? p[e] : 0.0f;
                    }
                    const f32x4 sv = stage[(kk & 3) * kStripPlane + (kk >> 2)];
#pragma unroll
                    for (int y = 0; y < 4; ++y)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[y][e] += sv[y] * v[e];
                }
            };
            if (s.nt) xc_loop(StripTag<true>());
            else xc_loop(StripTag<false>());
        }
        __syncthreads();
    }

    // Fixed-order reduction: lanes that share outputs by xor butterflies, then
    // the waves in order through LDS (the stage area, free after the last
    // chunk's barrier).
    float *red = reinterpret_cast<float *>(stage);
    float *__restrict__ out = s.out + z * s.batch_out;
    if constexpr (kLdsPoison) {
        poison_slots();
        __syncthreads();
    }
    if constexpr (KC) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[i][y] += __shfl_xor(acc[i][y], off);
        if (lane == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int y = 0; y < 4; ++y) red[wave * 16 + i * 4 + y] = acc[i][y];
        }
        __syncthreads();
        if (tid < XB * 4) {
            const int xi = tid >> 2, y = tid & 3;
            const int g = xi >> 2, i = xi & 3;
            float sum = red[g * 16 + i * 4 + y];
#pragma unroll
            for (int q = 1; q < kStripWaves / 4; ++q)  // KCP = 2 or 4
                if (q < KCP) sum += red[(g + XQ * q) * 16 + i * 4 + y];
            if (x0 + xi < X && y < s.r) {
                float *p = out + (int64_t)(x0 + xi) * s.o_x + (int64_t)y * s.o_y;
                *p = beta != 0.0f ? alpha * sum + beta * *p : alpha * sum;
            }
        }
    } else {
#pragma unroll
        for (int off = 4; off < 64; off <<= 1) {  // off = XQ .. 32 (XQ = 4 or 8)
            if (off < XQ) continue;
#pragma unroll
            for (int y = 0; y < 4; ++y)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[y][e] += __shfl_xor(acc[y][e], off);
        }
        if (kr == 0) {
#pragma unroll
            for (int y = 0; y < 4; ++y)
#pragma unroll
                for (int e = 0; e < 4; ++e) red[(wave * XQ + xq) * 16 + y * 4 + e] = acc[y][e];
        }
        __syncthreads();
        if (tid < XB * 4) {
            const int y = tid / XB, xi = tid % XB;
            const int q = xi >> 2, e = xi & 3;
            float sum = red[q * 16 + y * 4 + e];
#pragma unroll
            for (int w = 1; w < kStripWaves; ++w) sum += red[(w * XQ + q) * 16 + y * 4 + e];
            if (x0 + xi < X && y < s.r) {
                float *p = out + (int64_t)(x0 + xi) * s.o_x + (int64_t)y * s.o_y;
                *p = beta != 0.0f ? alpha * sum + beta * *p : alpha * sum;
            }
        }
    }
}

// KC0, KC1: storage order of strip 0's and strip 1's big operand.
template <bool KC0, bool KC1>
__global__ void __launch_bounds__(kStripThreads) sgemm_strip_kernel(StripArgs a)
{
    __shared__ __attribute__((aligned(16))) f32x4 stage[4 * kStripPlane];
    const int z = a.z0 + blockIdx.y;
    const int wg = blockIdx.x;
    if (wg < a.s[0].wgs) strip_block<KC0>(a.s[0], wg, a.K, z, a.alpha, a.beta, stage);
    else strip_block<KC1>(a.s[1], wg - a.s[0].wgs, a.K, z, a.alpha, a.beta, stage);
}

}  // namespace sgemm
