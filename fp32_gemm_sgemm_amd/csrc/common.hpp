// Device helpers shared by the GEMM kernels: vector types, the workgroup to
// tile mapping, and buffer resources for edge loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16-byte vectors that only claim 4-byte alignment.  The HSA code objects for
// gfx950 run with unaligned global access enabled (the compiler itself merges
// four consecutive float loads from a dword-aligned pointer into one
// global_load_dwordx4), so rows with any dword-aligned start and stride load
// and store 16 bytes per lane.
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x2u __attribute__((ext_vector_type(2), aligned(4)));

// One GEMM launch, passed to every kernel by value.
//
// The launch computes, for every batch entry z and every K split s,
//   C_z,s[i*ldc + j] = alpha * sum_{k in split s} op(A_z)(i,k) * op(B_z)(k,j)
//                      + beta * C_z,s[i*ldc + j]
// where op(X) is X (row-major, X[r*ld + c]) or its transpose (X[c*ld + r]).
// Without a K split (splits == 1) that is the whole product; with one, the
// host points C at a workspace that receives one partial result per split
// (alpha 1, beta 0) and a second kernel adds them up in a fixed order.
struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int64_t batch_a, batch_b, batch_c;  // elements between batch entries
    int64_t split_c;                    // elements between the partials of splits s and s+1
    int M, N, K;
    int lda, ldb, ldc;
    int k_chunk;                        // K range of one split (>= K when splits == 1)
    int splits;
    int tiles_m, tiles_n;
    int group_m, xcd_remap;
    int wg_base;                        // logical id of this launch's first workgroup
    int direct;                         // operands allow direct global -> LDS loads
    float alpha, beta;
};

// Workgroup -> (tile row, tile column, K split, batch entry).
//
// The dispatcher hands workgroups to the 8 XCDs round-robin by linear id, and
// each XCD has its own L2.  With xcd_remap, the workgroups that land on one
// XCD get a contiguous run of logical ids, so tiles that share A rows and B
// columns share an L2.  A logical id walks the tiles of one (split, batch)
// pair before the next, and inside them, with group_m > 0, groups of group_m
// tile rows column by column, so a run of consecutive ids covers a compact
// block of tiles instead of one long tile row.  Every map is a bijection of
// the launch's workgroups onto [wg_base, wg_base + gridDim.x).
struct Work {
    int tm, tn, split, batch;
};

__device__ __forceinline__ Work map_work(const GemmArgs &g)
{
    int wg = blockIdx.x;
    if (g.xcd_remap) {
        constexpr int NX = 8;
        const int nwg = gridDim.x;
        const int x = wg % NX, idx = wg / NX;
        const int q = nwg / NX, r = nwg % NX;
        wg = x * q + (x < r ? x : r) + idx;
    }
    wg += g.wg_base;
    const int tiles = g.tiles_m * g.tiles_n;
    const int rest = wg / tiles;
    const int t = wg - rest * tiles;
    Work w;
    w.split = rest % g.splits;
    w.batch = rest / g.splits;
    if (g.group_m > 0) {
        const int per_group = g.group_m * g.tiles_n;
        const int grp = t / per_group;
        const int first = grp * g.group_m;
        const int rows = min(g.tiles_m - first, g.group_m);
        const int in = t - grp * per_group;
        w.tm = first + in % rows;
        w.tn = in / rows;
    } else {
        w.tm = t / g.tiles_n;
        w.tn = t - w.tm * g.tiles_n;
    }
    return w;
}

// Moves A, B and C to the batch entry and K split of `w` and narrows K to
// that split's range (the operands' k index runs along rows of B and of a
// transposed A, along columns otherwise).
template <bool TA, bool TB>
__device__ __forceinline__ void locate(GemmArgs &g, const Work &w)
{
    const int kb = w.split * g.k_chunk;
    g.A += w.batch * g.batch_a + (TA ? (int64_t)kb * g.lda : (int64_t)kb);
    g.B += w.batch * g.batch_b + (TB ? (int64_t)kb : (int64_t)kb * g.ldb);
    g.C += w.batch * g.batch_c + w.split * g.split_c;
    g.K = min(g.K - kb, g.k_chunk);
}

// Epilogue: W adjacent results v[0..W-1] of one C row go to p[0..W-1]
// (column col .. col+W-1), masked to columns below N, as alpha * v + beta * old.
// C is read only when beta != 0, so with beta == 0 whatever it held (NaN
// included) is simply overwritten.
template <int W>
__device__ __forceinline__ void store_row(float *p, int col, int N, const float (&v)[W],
                                          float alpha, float beta)
{
    // (no 3-wide vector: 3-element vector stores may be widened to 4)
    static_assert(W == 1 || W == 2 || W == 4, "1, 2 or 4 adjacent results");
    if constexpr (W > 1) {
        if (col + W - 1 < N) {
            typedef float vec_t __attribute__((ext_vector_type(W), aligned(4)));
            vec_t x;
#pragma unroll
            for (int j = 0; j < W; ++j) x[j] = alpha * v[j];
            if (beta != 0.0f) {
                const vec_t old = *reinterpret_cast<const vec_t *>(p);
#pragma unroll
                for (int j = 0; j < W; ++j) x[j] += beta * old[j];
            }
            *reinterpret_cast<vec_t *>(p) = x;
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < W; ++j)
        if (col + j < N) p[j] = beta != 0.0f ? alpha * v[j] + beta * p[j] : alpha * v[j];
}

// LDS race check.  A build with SGEMM_LDS_POISON=1 sets every LDS word to a
// quiet NaN before it is refilled, from the moment the words are free (the
// barrier after their last reads) or just before their fill is issued, and
// waits for those writes before the fill.  A read that comes too early (the
// fill has not landed) or too late (the words were already released) then
// returns NaN, which spreads into the results; bitwise equality with the
// normal build shows that no read of the parity cases raced.  The normal
// build (SGEMM_LDS_POISON=0) compiles none of it.
#ifndef SGEMM_LDS_POISON
#define SGEMM_LDS_POISON 0
#endif
constexpr bool kLdsPoison = SGEMM_LDS_POISON != 0;

// Writes a quiet NaN to n consecutive LDS floats at p.
__device__ __forceinline__ void lds_poison(float *p, int n)
{
    for (int i = 0; i < n; ++i) p[i] = __builtin_nanf("");
}

// Waits for this thread's LDS writes (the poison) to complete, so that a fill
// issued afterwards (a direct load whose data reaches LDS later) lands on top
// of them, and keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void lds_poison_done()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));  // lgkmcnt(0), other counters free
    asm volatile("" ::: "memory");
}

// Timeline build.  With SGEMM_TIMELINE=1 the direct-load kernel reads the
// shader clock (s_memtime) at fixed points and keeps the readings in device
// arrays that sgemm_f32_timeline_read copies out:
//  phase: per workgroup of a call's first launch with id below
//         kTlPhaseWgs, the clock at entry, after the first slice has landed
//         (the loop starts), after the last slice, and once every thread's
//         stores of C are done; then the device's constant-rate real-time
//         counter (s_memrealtime) at entry and at that end;
//  slice: per workgroup below kTlSliceWgs, per wave and per slice below
//         kTlSlices, the clock before and after the wave waits for its own
//         loads of the next slice (the workgroup barrier follows).
// The per-slice readings go to LDS beside the stages and are copied out at
// the end, so the loop issues no global stores; the clock readings are
// scalar reads, whose count the loop waits out right after the second one.
// Shader-clock readings of different compute units come from unrelated
// counters: only differences within one workgroup mean anything.  The
// real-time counter is one for the device, so its readings place the
// workgroups against each other, and against the shader clock they give the
// clock's rate.  The normal build
// (SGEMM_TIMELINE=0) compiles none of it.
#ifndef SGEMM_TIMELINE
#define SGEMM_TIMELINE 0
#endif
#if SGEMM_TIMELINE
constexpr int kTlPhaseWgs = 4096, kTlSliceWgs = 16, kTlWaves = 16, kTlSlices = 256;
constexpr int kTlPhaseValues = 6;
__device__ unsigned long long g_tl_phase[kTlPhaseWgs * kTlPhaseValues];
__device__ uint32_t g_tl_slice[kTlSliceWgs * kTlWaves * kTlSlices * 2];
#endif

// A raw buffer resource over [base, base + bytes): loads at or past its end
// return zero and never fault.  bytes <= 0 gives an empty resource; sizes
// above 4 GiB - 1 are clamped (offsets used with a resource stay below that).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float *base, int64_t bytes)
{
    const int num = (int)(uint32_t)(bytes <= 0 ? 0 : bytes < 0xffffffffll ? bytes : 0xffffffffll);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, num, 0x00020000);
}

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_offset, 0, 0));
}

}  // namespace sgemm
