// Single-precision GEMM on CDNA4 matrix cores with direct global -> LDS loads
// (gfx950 buffer_load_dwordx4 ... lds): the AMD counterpart of the multi-stage
// asynchronous-copy pipeline of "4.1 CUDA GEMM operator performance
// optimization", section 10.  Fetched slices land in LDS without passing
// through registers, so there are no staging registers and no LDS write
// instructions, and STAGES slices can be in flight.
//
// The MFMA part (wave tiles of 32x32 blocks, k permutation, column
// interleave, fragment ping-pong) is the one of sgemm_mfma.hpp.  What differs is the LDS layout and the fetch:
//
//  * A direct load writes a wave's 64 lanes x 16 bytes to 1 KB of contiguous
//    LDS (lane l at offset 16*l, checked on the device), so the A slice is
//    stored without padding: BM rows of BK floats.  To keep the fragment
//    reads (32 consecutive rows, one 16-byte chunk each) free of bank
//    conflicts, chunk p of row r is stored at chunk position p ^ f(r), and a
//    lane fetching position q of its 1 KB block loads the global chunk that
//    belongs there.  f uses only row bits 0-3, so it is the same for every
//    32-row block:  BK = 16: f(r) = ((r >> 1) ^ (r >> 2)) & 3;
//                   BK = 32: f(r) = (r ^ ((r >> 3) & 1)) & 7.
//    Either makes the 16-byte chunks read by any 8 consecutive lanes fall in
//    distinct 128-byte bank rows' slots, and those of any 16 consecutive lanes
//    in distinct slots of 256 bytes.
//  * B keeps its row-major layout: a 1 KB block is part of one B row.
//  * Loads go through buffer resources ending at the matrices' last
//    elements; rows past M (A) or K (B) read as zero, and a chunk wholly past
//    K (A) or N (B) gets an offset beyond every resource (also zero).  A
//    slice that holds a partial chunk (K or N not a multiple of 4 at the
//    edge) is fetched instead through registers (dword loads and a select)
//    and written to the same swizzled positions.  Operands whose rows are
//    not 16-byte aligned use the register fetch for every slice.
//
// Pipeline, per slice kt: wait for this thread's fetch of slice kt, barrier
// (every wave's fetch of kt has landed and every wave has finished slice
// kt-1), issue the fetch of slice kt+STAGES-1 into the buffer slice kt-1
// used, multiply slice kt.  One barrier per slice.
#pragma once

#include "common.hpp"

namespace sgemm {

template <int BK> __device__ __forceinline__ int chunk_swizzle(int r)
{
    if constexpr (BK == 16) return ((r >> 1) ^ (r >> 2)) & 3;
    else return (r ^ ((r >> 3) & 1)) & 7;
}

template <int NB> struct DlFragB;
template <> struct DlFragB<1> { typedef float T; };
template <> struct DlFragB<2> { typedef f32x2 T; };
template <> struct DlFragB<4> { typedef f32x4 T; };

template <int NB>
__device__ __forceinline__ float dl_frag_elem(const typename DlFragB<NB>::T &v, int cb)
{
    if constexpr (NB == 1) return v;
    else return v[cb];
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES>
struct DlTraits {
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int NT = NW * 64;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = BN / WAVES_N;
    static constexpr int RM = WTM / 32;
    static constexpr int NB = WTN / 32;
    static constexpr int CPR = BK / 4;                 // 16-byte chunks per A row
    static constexpr int A_LOADS = BM * BK / 4 / NT;   // per thread per slice
    static constexpr int B_LOADS = BK * BN / 4 / NT;
    static constexpr int A_FLOATS = BM * BK;
    static constexpr int STAGE_FLOATS = BM * BK + BK * BN;
    static constexpr int LDS_FLOATS = STAGES * STAGE_FLOATS;
    static_assert(BK == 16 || BK == 32, "swizzle defined for BK 16 and 32");
    static_assert(WTM % 32 == 0 && RM >= 1, "wave tile rows must be a multiple of 32");
    static_assert(NB == 1 || NB == 2 || NB == 4, "wave tile columns must be 32, 64 or 128");
    static_assert(A_LOADS * NT * 4 == BM * BK && B_LOADS * NT * 4 == BK * BN,
                  "slices must split into whole 1 KB blocks per wave");
    static_assert(STAGES >= 2, "at least two LDS stages");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget of one CU");
};

// Offset given to chunks that must read as zero: beyond every resource
// (resources are clamped below it when direct loads are used).
constexpr uint32_t kOobOffset = 0x80000000u;

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
sgemm_mfma_dl_kernel(int M, int N, int K,
                     const float *__restrict__ A, int lda,
                     const float *__restrict__ B, int ldb,
                     float *__restrict__ C, int ldc,
                     int tiles_m, int tiles_n, int group_m, int xcd_remap, int direct)
{
    typedef DlTraits<BM, BN, BK, WAVES_M, WAVES_N, STAGES> T;
    constexpr int NW = T::NW, WTM = T::WTM, WTN = T::WTN, RM = T::RM, NB = T::NB;
    constexpr int CPR = T::CPR, A_LOADS = T::A_LOADS, B_LOADS = T::B_LOADS;
    constexpr int STAGE_FLOATS = T::STAGE_FLOATS, A_FLOATS = T::A_FLOATS;
    constexpr int G = BK / 8;
    constexpr int BCH = BN / 4;  // 16-byte chunks per B row
    typedef typename DlFragB<NB>::T fragb_t;

    __shared__ __attribute__((aligned(1024))) float smem[T::LDS_FLOATS];

    // (No AGPR hint here: with no staging registers the accumulators fit in
    // ArchVGPRs, and with the hint the allocator rotates them through copies
    // at the loop back-edge.)

    int tm, tn;
    map_tile(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, xcd_remap, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    f32x16 acc[RM][NB];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // ---- fetch assignment ------------------------------------------------------
    // Load j of this thread fills 16 bytes at LDS chunk q = (j*NW + wave)*64 +
    // lane of the A (or B) region of a stage.
    uint32_t a_off[A_LOADS], b_off[B_LOADS];
    int a_col[A_LOADS], b_colv[B_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int q = (j * NW + wave) * 64 + lane;
        const int r = q / CPR, p = (q % CPR) ^ chunk_swizzle<BK>(r);
        a_col[j] = 4 * p;
        a_off[j] = 4u * ((uint32_t)r * (uint32_t)lda + 4u * (uint32_t)p);
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int q = (j * NW + wave) * 64 + lane;
        const int kr = q / BCH, c = q % BCH;
        b_colv[j] = 4 * c;
        b_off[j] = 4u * ((uint32_t)kr * (uint32_t)ldb + 4u * (uint32_t)c);
    }
    // LDS destinations are cast to the LDS address space right at the load:
    // a helper lambda returning such a pointer cannot be compiled for the
    // host, which would silently drop this kernel's host-side stub.
    typedef __attribute__((address_space(3))) void lds_void;

    // Fetch slice kt into stage s.
    auto fetch = [&](int kt, int s) {
        const int k0 = kt * BK;
        const float *abase = A + (int64_t)m0 * lda + k0;
        const float *bbase = B + (int64_t)k0 * ldb + n0;
        const int64_t abytes = 4 * ((int64_t)(M - 1 - m0) * lda + (K - k0));
        const int64_t bbytes = 4 * ((int64_t)(K - 1 - k0) * ldb + (N - n0));
        const bool partial = ((K & 3) && k0 + BK > K) || ((N & 3) && n0 + BN > N);
        if (direct && !partial) {
            const auto ar = make_rsrc(abase, abytes < (int64_t)kOobOffset ? abytes : (int64_t)kOobOffset);
            const auto br = make_rsrc(bbase, bbytes < (int64_t)kOobOffset ? bbytes : (int64_t)kOobOffset);
#pragma unroll
            for (int j = 0; j < A_LOADS; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ar, (lds_void *)(smem + s * STAGE_FLOATS + (j * NW + wave) * 256), 16,
                    (int)(k0 + a_col[j] < K ? a_off[j] : kOobOffset), 0, 0, 0);
#pragma unroll
            for (int j = 0; j < B_LOADS; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    br, (lds_void *)(smem + s * STAGE_FLOATS + A_FLOATS + (j * NW + wave) * 256), 16,
                    (int)(n0 + b_colv[j] < N ? b_off[j] : kOobOffset), 0, 0, 0);
        } else {
            const auto ar = make_rsrc(abase, abytes);
            const auto br = make_rsrc(bbase, bbytes);
            f32x4 va[A_LOADS], vb[B_LOADS];
#pragma unroll
            for (int j = 0; j < A_LOADS; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = buffer_load_f32(ar, a_off[j] + 4u * e);
                    va[j][e] = (k0 + a_col[j] + e < K) ? x : 0.0f;
                }
#pragma unroll
            for (int j = 0; j < B_LOADS; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = buffer_load_f32(br, b_off[j] + 4u * e);
                    vb[j][e] = (n0 + b_colv[j] + e < N) ? x : 0.0f;
                }
#pragma unroll
            for (int j = 0; j < A_LOADS; ++j)
                *reinterpret_cast<f32x4 *>(smem + s * STAGE_FLOATS + ((j * NW + wave) * 64 + lane) * 4) = va[j];
#pragma unroll
            for (int j = 0; j < B_LOADS; ++j)
                *reinterpret_cast<f32x4 *>(smem + s * STAGE_FLOATS + A_FLOATS + ((j * NW + wave) * 64 + lane) * 4) = vb[j];
        }
    };

    // ---- fragments -----------------------------------------------------------------
    // A: row R = wm*WTM + 32i + (lane & 31), logical chunk 2g + (lane >> 5),
    // stored at chunk (2g + h) ^ f(R) = 2g ^ (h ^ f(R)) (2g is even), and
    // f(R) = f(lane & 31) since 32i and wm*WTM only change row bits >= 5.
    const int l31 = lane & 31;
    const int u = (lane >> 5) ^ chunk_swizzle<BK>(l31);
    const int a_row0 = (wm * WTM + l31) * BK;
    const int b_base = (4 * (lane >> 5)) * BN + wn * WTN + NB * l31;
    struct Frag {
        f32x4 a[RM];
        fragb_t b[4];
    };
    auto read_frag = [&](int s, int g, Frag &f) {
        const float *as = smem + s * STAGE_FLOATS + a_row0 + 4 * ((2 * g) ^ u);
        const float *bs = smem + s * STAGE_FLOATS + A_FLOATS + b_base + 8 * g * BN;
#pragma unroll
        for (int i = 0; i < RM; ++i)
            f.a[i] = *reinterpret_cast<const f32x4 *>(as + i * 32 * BK);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            f.b[t] = *reinterpret_cast<const fragb_t *>(bs + t * BN);
    };
    auto mfma_frag = [&](const Frag &f) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < RM; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        f.a[i][t], dl_frag_elem<NB>(f.b[t], j), acc[i][j], 0, 0, 0);
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
        for (int g = 0; g < G; ++g) {
            if (g + 1 < G) read_frag(s, g + 1, f[(g + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_frag(f[g & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- epilogue (as sgemm_mfma.hpp) ------------------------------------------------
    const int col = n0 + wn * WTN + NB * l31;
#pragma unroll
    for (int i = 0; i < RM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row >= M) continue;
            float *p = C + (int64_t)row * ldc + col;
            if (NB == 4 && col + 3 < N) {
                f32x4 v = {acc[i][0][r], acc[i][NB > 1 ? 1 : 0][r],
                           acc[i][NB > 2 ? 2 : 0][r], acc[i][NB > 3 ? 3 : 0][r]};
                *reinterpret_cast<f32x4u *>(p) = v;
            } else if (NB == 2 && col + 1 < N) {
                f32x2 v = {acc[i][0][r], acc[i][NB > 1 ? 1 : 0][r]};
                *reinterpret_cast<f32x2u *>(p) = v;
            } else {
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    if (col + j < N) p[j] = acc[i][j][r];
            }
        }
    }
}

}  // namespace sgemm
