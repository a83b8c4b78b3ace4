// Second pass of a K-split product, and the scaling pass of an empty one.
//
// Splitting K across workgroups and adding the partial results afterwards
// turns a grid of few output tiles into one that fills the chip (the split-K
// stage of the "cuda-kernels" README: one 128x128 tile with K = 32768 is one
// workgroup on one compute unit however fast the inner loop is).  Here each
// split writes its partial product to a workspace and this kernel computes
//
//   C = alpha * (P_0 + P_1 + ... + P_{S-1}) + beta * C
//
// with one thread per 4 adjacent outputs adding the partials in split order
// 0, 1, 2, ...: no atomics, so a given configuration gives bitwise the same
// C on every run whatever order the splits' workgroups ran in.  With S = 0 it
// computes C = beta * C (alpha times an empty sum), which is how a product
// with K = 0 or alpha = 0 is finished without reading A or B.
#pragma once

#include "common.hpp"

namespace sgemm {

struct ReduceArgs {
    const float *P;    // partials: [batch][split][M][ldp], rows 16-byte aligned
    float *C;
    int64_t split_p;   // elements between splits (M * ldp)
    int64_t batch_p;   // elements between batch entries (splits * M * ldp)
    int64_t batch_c;
    int64_t quads;     // M * ldp / 4: 4-wide groups per batch entry
    int M, N, ldp, ldc, splits;
    float alpha, beta;
};

__global__ void __launch_bounds__(256) splitk_reduce_kernel(ReduceArgs r)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= r.quads) return;
    const int z = blockIdx.y;
    const int qpr = r.ldp >> 2;
    const int row = (int)(q / qpr);
    const int col = 4 * (int)(q - (int64_t)row * qpr);
    if (col >= r.N) return;
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    if (r.splits > 0) {
        const float *p = r.P + z * r.batch_p + (int64_t)row * r.ldp + col;
        s = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll 4
        for (int t = 1; t < r.splits; ++t) s += *reinterpret_cast<const f32x4 *>(p + t * r.split_p);
    }
    const float v[4] = {s[0], s[1], s[2], s[3]};
    store_row<4>(r.C + z * r.batch_c + (int64_t)row * r.ldc + col, col, r.N, v, r.alpha, r.beta);
}

}  // namespace sgemm
