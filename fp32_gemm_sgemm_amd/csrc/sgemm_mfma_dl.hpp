// Single-precision GEMM on CDNA4 matrix cores with direct global -> LDS loads
// (gfx950 buffer_load_dword[x4] ... lds): the AMD counterpart of the
// multi-stage asynchronous-copy pipeline of "4.1 CUDA GEMM operator
// performance optimization", section 10.  Fetched slices land in LDS without
// passing through registers, so there are no staging registers and no LDS
// write instructions, and STAGES slices can be in flight.
//
// The MFMA part (wave tiles of 32x32 blocks, k permutation, fragment
// ping-pong) is the one of sgemm_mfma.hpp; MB = 16 builds the same tiles from
// 16x16 blocks (v_mfma_f32_16x16x4_f32), four times as many independent
// accumulator chains per wave, which pays when one wave per SIMD runs a small
// wave tile.  What differs from sgemm_mfma.hpp is the LDS layout and the
// fetch:
//
//  * A direct load writes a wave's 64 lanes x EL floats to contiguous LDS
//    (lane l at offset 4*EL*l, checked on the device for EL = 4 and EL = 1),
//    so operand tiles are stored without padding.  EL = 4 (16-byte loads)
//    needs rows that start 16-byte aligned; DW kernels use EL = 1 (4-byte
//    loads), which any row allows, with four times the load instructions.
//  * Each operand is k-contiguous (A, or a transposed B) or index-contiguous
//    (B, or a transposed A) and keeps that storage in LDS (DlOperand below).
//    In a k-contiguous tile, 16-byte chunk p of row r is stored at chunk
//    position p ^ f(r), which keeps the fragment reads (32 consecutive rows,
//    one 16-byte chunk each) free of bank conflicts; a lane loads the global
//    data that belongs at its LDS position.  f uses only row bits 0-3:
//    BK = 16: f(r) = ((r >> 1) ^ (r >> 2)) & 3;
//    BK = 32: f(r) = (r ^ ((r >> 3) & 1)) & 7;
//    BK = 64: f(r) = r & 15 (a row is the 64 banks' width, so 16 rows read
//    16 distinct chunk positions);
//    16x16 blocks (32-deep slices): f(r) = ((r & 2) << 1) | ((r & 4) >> 1),
//    see chunk_swizzle.
//  * Loads go through buffer resources ending at the operands' last
//    elements; rows past the end read as zero, and data wholly past K, M or N
//    gets an offset beyond every resource (also zero).  With 16-byte loads,
//    a slice that holds a chunk only partly inside the data is fetched
//    instead through registers (dword loads and a select) into the same
//    positions, and so is every slice when the rows are not 16-byte aligned
//    (DW kernels exist for that case).
//
// Pipelines (PIPE), one barrier per slice either way:
//  * plain (PIPE & 2 == 0), per slice kt: wait for this thread's fetch of
//    slice kt, barrier (every wave's fetch of kt has landed and every wave has
//    finished slice kt-1), issue the fetch of slice kt+STAGES-1 into the
//    buffer slice kt-1 used, multiply slice kt.
//  * cross-slice (PIPE & 2): the fetch of slice kt+STAGES-1 is
//    interleaved with the MFMAs of slice kt's first k group, the barrier sits
//    before the last k group, and the next slice's first fragments are read
//    in the shadow of that group's MFMAs, so no LDS latency and no burst of
//    load instructions stands between two slices' MFMAs.  In a tile whose
//    every slice takes direct loads, the slices that fetch a slice wholly
//    inside K run a second copy of the loop body with load offsets fixed for
//    the tile and no checks, so no branch separates the loads from the MFMAs
//    they are scheduled among; the last slices keep the general fetch.
//  PIPE & 4 keeps the accumulators in AGPRs.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace sgemm {

// MB = 16 (16x16 blocks, 32-deep slices): f(r) = ((r & 2) << 1) | ((r & 4) >> 1).
// A 16-byte fragment read there takes 16 consecutive rows in each lane
// quarter q, at chunk 4g + q.  With the 32x32 layout's f that read costs 4
// bank-conflict cycles on gfx950 (SQ_LDS_BANK_CONFLICT); among the linear maps
// of row bits 0-3 to a chunk, this one was measured conflict-free for both k
// groups of a slice at every 2 KB offset (the offsets of blocks, waves,
// operands and stages here).
template <int BK, int MB = 32> __device__ __forceinline__ int chunk_swizzle(int r)
{
    if constexpr (MB == 16) {
        static_assert(BK == 32, "16x16 blocks are laid out for 32-deep slices");
        return ((r & 2) << 1) | ((r & 4) >> 1);
    } else if constexpr (BK == 16) {
        return ((r >> 1) ^ (r >> 2)) & 3;
    } else if constexpr (BK == 32) {
        return (r ^ ((r >> 3) & 1)) & 7;
    } else {
        return r & 15;
    }
}

// Three adjacent floats with 4-byte alignment (the compiler picks the LDS
// read instructions that this alignment allows).
struct DlF3 {
    float x[3];
    __device__ __forceinline__ float operator[](int i) const { return x[i]; }
};

// Offset given to chunks that must read as zero: beyond every resource
// (resources are clamped below it when direct loads are used).
constexpr uint32_t kOobOffset = 0x80000000u;

template <bool B> struct DlTag { static constexpr bool value = B; };

// x if e < n, else +0: the sign of e - n as a bit mask, with no compare (a
// compare per element leaves a 64-bit lane mask per element in scalar
// registers, which the compiler hoists and spills).
__device__ __forceinline__ float keep_below(float x, int e, int n)
{
    const uint32_t keep = (uint32_t)((e - n) >> 31);
    uint32_t r;
    // (the AND is opaque: the compiler would turn the mask back into a compare)
    asm volatile("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(__builtin_bit_cast(uint32_t, x)), "v"(keep));
    return __builtin_bit_cast(float, r);
}

template <int W> struct DlVec;
template <> struct DlVec<1> { typedef float T; };
template <> struct DlVec<2> { typedef f32x2 T; };
template <> struct DlVec<3> { typedef DlF3 T; };
template <> struct DlVec<4> { typedef f32x4 T; };

// Fragment vector of an index-contiguous operand (unused, and a plain float,
// for a k-contiguous one).
template <bool XC, int W> struct DlXVec { typedef float T; };
template <int W> struct DlXVec<true, W> { typedef typename DlVec<W>::T T; };

template <int W, typename V>
__device__ __forceinline__ float dl_elem(const V &v, int b)
{
    if constexpr (W == 1) return v;
    else return v[b];
}

// One operand's tile in LDS.  X is the operand's own index (rows of C for A,
// columns of C for B); a tile covers E of them, a wave WT, in W blocks of MB
// (32 or 16).  Block b of a wave holds the indices x = wave_offset + W*l + b,
// l = 0..MB-1 (interleaved), so a lane's W results of one C row or column are
// adjacent.
//
//  KC ("k contiguous": A, or a transposed B): the operand's rows run along k.
//     LDS holds E rows of BK floats; row L holds index P(L) = wave offset +
//     W*(L%MB) + (L%WT)/MB, so the MB rows a fragment read touches are
//     consecutive; chunk p of row L is stored at chunk p ^ f(L).  A fragment
//     read is one 16-byte read per block: 4 successive k of one index.
//  XC ("index contiguous": B, or a transposed A): the operand's rows run
//     along X.  LDS holds BK rows of E floats; a fragment read is one W-wide
//     read per k: the W blocks' values at one k.
template <int E, int BK, int WT, int NW, bool KC, bool DW, int MB = 32>
struct DlOperand {
    static constexpr int W = WT / MB;
    static constexpr int ELEMS = DW ? 1 : 4;            // floats per lane per load
    static constexpr int LOADS = E * BK / ELEMS / (NW * 64);  // per thread per slice
    static constexpr int FLOATS = E * BK;
    static_assert(WT % MB == 0 && W >= 1, "wave tiles must be multiples of the block");
    static_assert(KC || (W >= 1 && W <= 4), "index-contiguous fragments are 1 to 4 wide");
    static_assert(LOADS * NW * 64 * ELEMS == E * BK, "slices must split into whole wave loads");

    // Fetch assignment of load j: byte offset from the slice's base (the
    // tile's first index at the slice's first k) and the first column of the
    // lane's data along the contiguous dimension (k for KC, the index for
    // XC).  The lane's data lands at LDS float (j*NW + wave)*64*ELEMS +
    // lane*ELEMS of the operand's region.
    __device__ __forceinline__ static void assign(int j, int wave, int lane, int ld,
                                                  uint32_t &off, int &col)
    {
        int r, c;
        source(j, wave, lane, r, c);
        col = c;
        off = 4u * ((uint32_t)r * (uint32_t)ld + (uint32_t)c);
    }

    // Load j's offset for a slice that lies wholly inside K, in a tile whose
    // edge along the operand's own index (M for A, N for B) is at `lim`:
    // data of indices at or past it gets kOobOffset.  Such offsets stay fixed
    // for the whole tile, so a run of full slices needs no per-slice checks.
    __device__ __forceinline__ static uint32_t full_slice_off(int j, int wave, int lane, int ld,
                                                             int lim)
    {
        int r, c;
        source(j, wave, lane, r, c);
        const int idx = KC ? r : c;
        return idx < lim ? 4u * ((uint32_t)r * (uint32_t)ld + (uint32_t)c) : kOobOffset;
    }

  private:
    // The global row r and column c (of the operand as stored, relative to the
    // slice's base) whose EL floats load j of this lane brings in.
    __device__ __forceinline__ static void source(int j, int wave, int lane, int &r, int &c)
    {
        const int q = ((j * NW + wave) * 64 + lane) * ELEMS;  // LDS float position
        const int rl = KC ? BK : E;                            // floats per LDS row
        const int row = q / rl;
        c = q % rl;
        r = row;
        if constexpr (KC) {
            c = 4 * ((c / 4) ^ chunk_swizzle<BK, MB>(row)) + c % 4;
            const int in = row % WT;
            r = row - in + W * (in % MB) + in / MB;
        }
    }
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, bool TA, bool TB,
          bool DW = false, int MB = 32>
struct DlTraits {
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int NT = NW * 64;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int RM = WTM / MB;
    static constexpr int NB = WTN / MB;
    typedef DlOperand<BM, BK, WTM, NW, !TA, DW, MB> OpA;
    typedef DlOperand<BN, BK, WTN, NW, TB, DW, MB> OpB;
    static constexpr int A_FLOATS = BM * BK;
    static constexpr int STAGE_FLOATS = BM * BK + BK * BN;
    static constexpr int LDS_FLOATS = STAGES * STAGE_FLOATS;
    static_assert(BK == 16 || BK == 32 || BK == 64, "swizzle defined for BK 16, 32 and 64");
    static_assert(NB == 1 || NB == 2 || NB == 4, "wave tile columns must be 32, 64 or 128");
    static_assert(STAGES >= 2, "at least two LDS stages");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget of one CU");
};


template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, bool TA, bool TB, bool DW,
          int PIPE = 0, int MB = 32>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
sgemm_mfma_dl_kernel(GemmArgs g)
{
    typedef DlTraits<BM, BN, BK, WAVES_M, WAVES_N, STAGES, TA, TB, DW, MB> T;
    typedef typename T::OpA OpA;
    typedef typename T::OpB OpB;
    constexpr int NW = T::NW, WTM = T::WTM, WTN = T::WTN, RM = T::RM, NB = T::NB;
    constexpr int A_LOADS = OpA::LOADS, B_LOADS = OpB::LOADS;
    constexpr int STAGE_FLOATS = T::STAGE_FLOATS, A_FLOATS = T::A_FLOATS;
    static_assert(MB == 32 || MB == 16, "32x32x2 or 16x16x4 blocks");
    constexpr int G = BK / (MB == 32 ? 8 : 16);  // k groups per slice
    constexpr int ACC = MB == 32 ? 16 : 4;        // accumulators per block per lane
    typedef typename std::conditional<MB == 32, f32x16, f32x4>::type acc_t;
    constexpr int EL = DW ? 1 : 4;  // floats per lane per load

#if SGEMM_TIMELINE
    // per-slice clock readings beside the stages (see g_tl_slice)
    static_assert(NW <= kTlWaves, "waves recorded per workgroup");
    __shared__ __attribute__((aligned(1024))) float smem[T::LDS_FLOATS + NW * kTlSlices * 2];
    uint32_t *const tl_lds = reinterpret_cast<uint32_t *>(smem + T::LDS_FLOATS);
    const unsigned long long tl_entry = __builtin_amdgcn_s_memtime();
    const unsigned long long tl_entry_rt = __builtin_amdgcn_s_memrealtime();
    unsigned long long tl_loop0 = 0;
#else
    __shared__ __attribute__((aligned(1024))) float smem[T::LDS_FLOATS];
#endif

    // PIPE bit 2: an (empty) AGPR clobber makes the register allocator keep
    // the accumulators in AGPRs.  It pays with the cross-slice loop; with the
    // plain loop the allocator rotated them through copies at the back-edge.
    if constexpr ((PIPE & 4) != 0) asm volatile("" ::: "a0");

    const Work w = map_work(g);
    locate<TA, TB>(g, w);
    const float *__restrict__ A = g.A;
    const float *__restrict__ B = g.B;
    const int M = g.M, N = g.N, K = g.K, lda = g.lda, ldb = g.ldb;
    const int m0 = w.tm * BM, n0 = w.tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    acc_t acc[RM][NB];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < ACC; ++r) acc[i][j][r] = 0.0f;

    // ---- fetch assignment ------------------------------------------------------
    // Load j of this thread fills EL floats at LDS float (j*NW + wave)*64*EL +
    // lane*EL of the operand's region of a stage.
    uint32_t a_off[A_LOADS], b_off[B_LOADS];
    int a_col[A_LOADS], b_col[B_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) OpA::assign(j, wave, lane, lda, a_off[j], a_col[j]);
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) OpB::assign(j, wave, lane, ldb, b_off[j], b_col[j]);

    // LDS destinations are cast to the LDS address space right at the load:
    // a helper lambda returning such a pointer cannot be compiled for the
    // host, which would silently drop this kernel's host-side stub.
    typedef __attribute__((address_space(3))) void lds_void;

    // LDS race check build: this thread's share of stage s (the words its
    // fetch fills) is set to NaN before the fill is issued.
    auto poison_stage = [&](int s) {
        if constexpr (kLdsPoison) {
#pragma unroll
            for (int j = 0; j < A_LOADS; ++j)
                lds_poison(smem + s * STAGE_FLOATS + ((j * NW + wave) * 64 + lane) * EL, EL);
#pragma unroll
            for (int j = 0; j < B_LOADS; ++j)
                lds_poison(smem + s * STAGE_FLOATS + A_FLOATS + ((j * NW + wave) * 64 + lane) * EL, EL);
            lds_poison_done();
        }
    };

    // Fetch slice kt into stage s.  Per operand: the slice's base (its first
    // index at k0), the resource extent up to the operand's last element, and
    // the limit of the contiguous column (k for KC, the index for XC) below
    // which a chunk holds data.
    auto fetch = [&](int kt, int s) {
        poison_stage(s);
        const int k0 = kt * BK;
        const float *abase = TA ? A + (int64_t)k0 * lda + m0 : A + (int64_t)m0 * lda + k0;
        const float *bbase = TB ? B + (int64_t)n0 * ldb + k0 : B + (int64_t)k0 * ldb + n0;
        const int64_t abytes = TA ? 4 * ((int64_t)(K - 1 - k0) * lda + (M - m0))
                                  : 4 * ((int64_t)(M - 1 - m0) * lda + (K - k0));
        const int64_t bbytes = TB ? 4 * ((int64_t)(N - 1 - n0) * ldb + (K - k0))
                                  : 4 * ((int64_t)(K - 1 - k0) * ldb + (N - n0));
        const int a_lim = TA ? M - m0 : K - k0;
        const int b_lim = TB ? K - k0 : N - n0;
        // (16-byte loads: a slice holding a chunk that is only partly inside
        // the data goes through registers; 4-byte loads are masked one by one)
        const bool partial = !DW && (((a_lim & 3) && a_lim < (TA ? BM : BK)) ||
                                     ((b_lim & 3) && b_lim < (TB ? BK : BN)));
        // One resource per operand serves both paths: with direct loads allowed
        // every in-slice offset of data is below 2^31 (the leading-dimension
        // limits of direct loads), so the extent can stop at kOobOffset,
        // beyond which chunks past the data are sent; otherwise the register
        // path needs the full extent.
        const int64_t cap = g.direct ? (int64_t)kOobOffset : (int64_t)0xffffffff;
        const auto ar = make_rsrc(abase, abytes < cap ? abytes : cap);
        const auto br = make_rsrc(bbase, bbytes < cap ? bbytes : cap);
        if (g.direct && !partial) {
            // (the load size must be a literal: one call per size)
#pragma unroll
            for (int j = 0; j < A_LOADS; ++j) {
                const int off = (int)(a_col[j] < a_lim ? a_off[j] : kOobOffset);
                float *dst = smem + s * STAGE_FLOATS + (j * NW + wave) * 64 * EL;
                if constexpr (DW) __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void *)dst, 4, off, 0, 0, 0);
                else __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void *)dst, 16, off, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < B_LOADS; ++j) {
                const int off = (int)(b_col[j] < b_lim ? b_off[j] : kOobOffset);
                float *dst = smem + s * STAGE_FLOATS + A_FLOATS + (j * NW + wave) * 64 * EL;
                if constexpr (DW) __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)dst, 4, off, 0, 0, 0);
                else __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)dst, 16, off, 0, 0, 0);
            }
        } else {
            // One load's data at a time (loaded, masked, written to LDS), so
            // this rarely used path needs few staging registers.
            auto put = [&](float *dst, const float (&v)[EL]) {
                if constexpr (EL == 4) *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
                else *dst = v[0];
            };
#pragma unroll
            for (int j = 0; j < A_LOADS; ++j) {
                float v[EL];
                const int n_in = a_lim - a_col[j];  // floats of this load inside the data
#pragma unroll
                for (int e = 0; e < EL; ++e) {
                    const float x = buffer_load_f32(ar, a_off[j] + 4u * e);
                    v[e] = keep_below(x, e, n_in);
                }
                put(smem + s * STAGE_FLOATS + ((j * NW + wave) * 64 + lane) * EL, v);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int j = 0; j < B_LOADS; ++j) {
                float v[EL];
                const int n_in = b_lim - b_col[j];  // floats of this load inside the data
#pragma unroll
                for (int e = 0; e < EL; ++e) {
                    const float x = buffer_load_f32(br, b_off[j] + 4u * e);
                    v[e] = keep_below(x, e, n_in);
                }
                put(smem + s * STAGE_FLOATS + A_FLOATS + ((j * NW + wave) * 64 + lane) * EL, v);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // Fetch of a slice wholly inside K in a tile that takes direct loads
    // throughout, with the tile's fixed offsets (full_slice_off): one
    // resource per operand, no checks, nothing that needs a branch.
    auto fetch_full = [&](int kt, int s, const uint32_t (&af)[A_LOADS], const uint32_t (&bf)[B_LOADS]) {
        poison_stage(s);
        const int k0 = kt * BK;
        const float *abase = TA ? A + (int64_t)k0 * lda + m0 : A + (int64_t)m0 * lda + k0;
        const float *bbase = TB ? B + (int64_t)n0 * ldb + k0 : B + (int64_t)k0 * ldb + n0;
        const auto ar = make_rsrc(abase, (int64_t)kOobOffset);
        const auto br = make_rsrc(bbase, (int64_t)kOobOffset);
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j) {
            float *dst = smem + s * STAGE_FLOATS + (j * NW + wave) * 64 * EL;
            if constexpr (DW) __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void *)dst, 4, (int)af[j], 0, 0, 0);
            else __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void *)dst, 16, (int)af[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j) {
            float *dst = smem + s * STAGE_FLOATS + A_FLOATS + (j * NW + wave) * 64 * EL;
            if constexpr (DW) __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)dst, 4, (int)bf[j], 0, 0, 0);
            else __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)dst, 16, (int)bf[j], 0, 0, 0);
        }
    };

    // ---- fragments -----------------------------------------------------------------
    // 32x32 blocks: MFMA step t (0..3) of k group g (8 deep) takes k = 8g + t
    // from lanes 0-31 and k = 8g + 4 + t from lanes 32-63 (h = lane >> 5).
    // 16x16 blocks: step t of k group g (16 deep) takes k = 16g + 4h + t from
    // lane quarter h = lane >> 4.  Both operands use the same k for a lane
    // group, so the permuted order sums the same products.
    //  KC: block b's index for lane l is LDS row wave_offset + MB*b + (l mod
    //      MB), whose k values of step 0..3 are logical chunk KQ*g + h (KQ
    //      chunks per k group), stored at (KQ*g + h) ^ f(row) = KQ*g ^ (h ^
    //      f(l mod MB)) (KQ*g has no bit of h, and f only sees row bits 0-3).
    //  XC: LDS row k, W floats at column wave_offset + W*(l mod MB).
    constexpr int LB = MB - 1;
    constexpr int KQ = MB == 32 ? 2 : 4;  // 16-byte chunks per k group
    const int l31 = lane & LB, h = MB == 32 ? lane >> 5 : lane >> 4;
    const int u = h ^ chunk_swizzle<BK, MB>(l31);
    typedef typename DlXVec<TA, RM>::T xa_t;
    typedef typename DlXVec<!TB, NB>::T xb_t;
    struct Frag {
        f32x4 ka[OpA::W];  // KC A: [block][t]
        xa_t xa[4];        // XC A: [t][block]
        f32x4 kb[OpB::W];
        xb_t xb[4];
    };
    const int a_base = TA ? (4 * h) * BM + wm * WTM + RM * l31 : (wm * WTM + l31) * BK;
    const int b_base = TB ? (wn * WTN + l31) * BK : (4 * h) * BN + wn * WTN + NB * l31;
    auto read_frag = [&](int s, int gi, Frag &f) {
        const float *as = smem + s * STAGE_FLOATS + a_base;
        const float *bs = smem + s * STAGE_FLOATS + A_FLOATS + b_base;
        if constexpr (TA) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                f.xa[t] = *reinterpret_cast<const xa_t *>(as + (4 * KQ * gi + t) * BM);
        } else {
#pragma unroll
            for (int i = 0; i < RM; ++i)
                f.ka[i] = *reinterpret_cast<const f32x4 *>(as + i * MB * BK + 4 * ((KQ * gi) ^ u));
        }
        if constexpr (TB) {
#pragma unroll
            for (int j = 0; j < NB; ++j)
                f.kb[j] = *reinterpret_cast<const f32x4 *>(bs + j * MB * BK + 4 * ((KQ * gi) ^ u));
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                f.xb[t] = *reinterpret_cast<const xb_t *>(bs + (4 * KQ * gi + t) * BN);
        }
    };
    auto mfma_frag = [&](const Frag &f) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    float a, b;
                    if constexpr (TA) a = dl_elem<RM>(f.xa[t], i);
                    else a = f.ka[i][t];
                    if constexpr (TB) b = f.kb[j][t];
                    else b = dl_elem<NB>(f.xb[t], j);
                    if constexpr (MB == 32)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i][j], 0, 0, 0);
                }
    };

    // ---- main loop -------------------------------------------------------------------
    // vmcnt value that leaves the fetches of the STAGES-2 later slices in
    // flight (s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt and
    // lgkmcnt at their maxima so they do not wait).
    constexpr int LOADS = A_LOADS + B_LOADS;
    constexpr int VM = (STAGES - 2) * LOADS;
    static_assert(VM < 64, "vmcnt field holds 6 bits");
    constexpr int WAIT_LATER = (VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14);

    // The barrier is issued bare: a __syncthreads() fence would make the
    // compiler wait for every outstanding load (the direct loads write LDS),
    // draining the later stages.  Instead this thread waits for its own fetch
    // of slice kt (vmcnt) and its own LDS writes (lgkmcnt(0): register-path
    // fetches), then meets the other waves at s_barrier; empty asm statements
    // with a memory clobber keep the compiler from moving LDS accesses
    // across it.
    constexpr int WAIT_ALL = (7 << 4);  // vmcnt(0) lgkmcnt(0)
    constexpr int WAIT_LATER_LGKM0 = WAIT_LATER & ~(15 << 8);
    const int nk = (K + BK - 1) / BK;
    constexpr int LOADS_ALL = A_LOADS + B_LOADS;
    if constexpr ((PIPE & 2) != 0) {
        // Cross-slice pipeline.  Slice kt: the loads of slice kt+STAGES-1 are
        // issued among the MFMAs of k group 0; before the last k group each
        // thread waits for its own loads of slice kt+1 and its LDS reads of
        // slice kt, one barrier follows (every wave's slice kt+1 has landed and
        // every wave has read all of slice kt, whose stage the next slice's
        // loads may then overwrite), and the fragments of slice kt+1's first k
        // group are read in the shadow of the last group's MFMAs.
        static_assert(G % 2 == 0, "fragment buffers alternate per k group");
        Frag f[2];
        if (nk > 0) {
#pragma unroll
            for (int s = 0; s < STAGES - 1; ++s)
                if (s < nk) fetch(s, s);
            if (STAGES - 2 < nk) __builtin_amdgcn_s_waitcnt(WAIT_LATER_LGKM0);
            else __builtin_amdgcn_s_waitcnt(WAIT_ALL);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            read_frag(0, 0, f[0]);
#if SGEMM_TIMELINE
            tl_loop0 = __builtin_amdgcn_s_memtime();
            __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));  // the reading (and the reads above)
#endif
        }
        uint32_t af[A_LOADS], bf[B_LOADS];
        // One slice kt.  FULL: the slice fetched here (kt+STAGES-1) lies wholly
        // inside K and the tile takes direct loads, so the fetch has no branch
        // and its loads can sit among the MFMAs.
        auto slice = [&](int kt, auto full) {
            constexpr bool FULL = decltype(full)::value;
            const int s = kt % STAGES;
            const int s1 = (kt + 1) % STAGES;
            const bool next = FULL || kt + 1 < nk;
            const bool more = FULL || kt + STAGES - 1 < nk;
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                __builtin_amdgcn_sched_barrier(0);
                if (gi + 1 < G) {
                    read_frag(s, gi + 1, f[(gi + 1) & 1]);
                    if (gi == 0) {
                        if constexpr (FULL) fetch_full(kt + STAGES - 1, (kt + STAGES - 1) % STAGES, af, bf);
                        else if (more) fetch(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
                    }
                    mfma_frag(f[gi & 1]);
                    // fragment reads (and in group 0 the loads) among the MFMAs
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    }
                    if (gi == 0) {
#pragma unroll
                        for (int i = 0; i < LOADS_ALL; ++i) {
                            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                        }
                    }
                } else {
                    // own loads of slice kt+1 landed (the later slices' may still
                    // be in flight) and own reads of slice kt done, barrier, then
                    // the next slice's first fragments
#if SGEMM_TIMELINE
                    const uint32_t tl_t0 = (uint32_t)__builtin_amdgcn_s_memtime();
#endif
                    if (more) __builtin_amdgcn_s_waitcnt(WAIT_LATER_LGKM0);
                    else __builtin_amdgcn_s_waitcnt(WAIT_ALL);
#if SGEMM_TIMELINE
                    const uint32_t tl_t1 = (uint32_t)__builtin_amdgcn_s_memtime();
                    // wait for the reading on every path, so that no later
                    // fragment wait has to cover an outstanding scalar read
                    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
                    if (lane == 0 && kt < kTlSlices) {
                        tl_lds[(wave * kTlSlices + kt) * 2] = tl_t0;
                        tl_lds[(wave * kTlSlices + kt) * 2 + 1] = tl_t1;
                    }
#endif
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
                    if (next) read_frag(s1, 0, f[G & 1]);
                    mfma_frag(f[gi & 1]);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        int kt = 0;
        // Tiles whose every slice goes by direct loads (no chunk only partly
        // inside M or N) run the slices that fetch a full slice without checks.
        const int m_lim = M - m0, n_lim = N - n0;
        const bool edge_chunks = !DW && ((TA && (m_lim & 3) && m_lim < BM) ||
                                         (!TB && (n_lim & 3) && n_lim < BN));
        if (g.direct && !edge_chunks) {
#pragma unroll
            for (int j = 0; j < A_LOADS; ++j) af[j] = OpA::full_slice_off(j, wave, lane, lda, m_lim);
#pragma unroll
            for (int j = 0; j < B_LOADS; ++j) bf[j] = OpB::full_slice_off(j, wave, lane, ldb, n_lim);
            const int kend = K / BK - (STAGES - 1);
            for (; kt < kend; ++kt) slice(kt, DlTag<true>());
        }
        for (; kt < nk; ++kt) slice(kt, DlTag<false>());
#if SGEMM_TIMELINE
        if (nk == 0) tl_loop0 = __builtin_amdgcn_s_memtime();
#endif
    } else {
        // Plain pipeline.
#if SGEMM_TIMELINE
        tl_loop0 = __builtin_amdgcn_s_memtime();
#endif
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < nk) fetch(s, s);
        for (int kt = 0; kt < nk; ++kt) {
            const int s = kt % STAGES;
            // this thread's fetch of slice kt has landed once at most the later
            // slices' fetches are outstanding (fewer near the end: wait for all)
            if (kt + STAGES - 2 < nk) __builtin_amdgcn_s_waitcnt(WAIT_LATER_LGKM0);
            else __builtin_amdgcn_s_waitcnt(WAIT_ALL);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if (kt + STAGES - 1 < nk) fetch(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);
            Frag f[2];
            read_frag(s, 0, f[0]);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                if (gi + 1 < G) read_frag(s, gi + 1, f[(gi + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mfma_frag(f[gi & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

#if SGEMM_TIMELINE
    const unsigned long long tl_loop1 = __builtin_amdgcn_s_memtime();
#endif
    // ---- epilogue ----------------------------------------------------------------------
    // Accumulator r of block (i, j) in lane l is D[8*(r/4) + 4*h + r%4][l & 31]
    // of a 32x32 block, D[4*h + r][l & 15] of a 16x16 one (h as above): C row
    // wave_offset + RM*(that row) + i, column wave_offset + NB*(l mod MB) + j,
    // so a lane holds NB adjacent columns.
    float *__restrict__ C = g.C;
    const int ldc = g.ldc;
    const int col = n0 + wn * WTN + NB * l31;
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int r = 0; r < ACC; ++r) {
            const int row = m0 + wm * WTM +
                            RM * (MB == 32 ? 8 * (r >> 2) + 4 * h + (r & 3) : 4 * h + r) + i;
            if (row >= M) continue;
            float v[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) v[j] = acc[i][j][r];
            store_row<NB>(C + (int64_t)row * ldc + col, col, N, v, g.alpha, g.beta);
        }
    }
#if SGEMM_TIMELINE
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores are done
    __syncthreads();
    const unsigned long long tl_end = __builtin_amdgcn_s_memtime();
    const unsigned long long tl_end_rt = __builtin_amdgcn_s_memrealtime();
    if (g.wg_base == 0 && (int)blockIdx.x < kTlSliceWgs) {
        // the slices this workgroup ran (the plain pipeline records none);
        // the LDS slots past them were never written
        const int rec = (PIPE & 2) != 0 ? min(nk, kTlSlices) : 0;
        uint32_t *dst = g_tl_slice + (size_t)blockIdx.x * kTlWaves * kTlSlices * 2;
        for (int i = tid; i < NW * kTlSlices * 2; i += T::NT)
            dst[i] = (i >> 1) % kTlSlices < rec ? tl_lds[i] : 0u;
    }
    if (g.wg_base == 0 && tid == 0 && (int)blockIdx.x < kTlPhaseWgs) {
        unsigned long long *ph = g_tl_phase + (size_t)blockIdx.x * kTlPhaseValues;
        ph[0] = tl_entry;
        ph[1] = tl_loop0;
        ph[2] = tl_loop1;
        ph[3] = tl_end;
        ph[4] = tl_entry_rt;
        ph[5] = tl_end_rt;
    }
#endif
}

}  // namespace sgemm
