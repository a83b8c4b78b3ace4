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

// Linear workgroup id -> (tile row, tile column).
//
// The dispatcher hands workgroups to the 8 XCDs round-robin by linear id, and
// each XCD has its own L2.  With xcd_remap, the workgroups that land on one
// XCD get a contiguous run of logical ids, so tiles that share A rows and B
// columns share an L2.  group_m > 0 then walks the logical ids down groups of
// group_m tile rows, column by column, so a run of consecutive ids covers a
// compact block of tiles instead of one long tile row.  Both maps are
// bijections of [0, tiles_m * tiles_n).
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
