// Measurement probes (libsgemm_probes.so), kept apart from the product
// library: they exist only to put the GEMM's numbers in context.
//
// sgemm_probe_mfma_peak: every wave runs `iters` rounds of 8 independent
// v_mfma_f32_32x32x2_f32 chains on register operands (no memory traffic in
// the loop), so the launch measures the matrix-core FP32 ceiling the chip
// sustains at its actual clock: FLOPs = iters * 8 * 4096 * waves.  Each thread
// writes one float (a sum of its accumulators) so nothing is optimised away.
//
// sgemm_probe_empty: a launch that does nothing but write one float per
// workgroup, with the grid of the small products (256 workgroups of 512
// threads: the 512^3 plan), so its time is the floor any launch of that
// shape pays (dispatch of the waves, completion) before doing work.
//
// sgemm_probe_valu_peak: every thread runs `iters` rounds of 16 independent
// single-precision FMA chains (x = x * a + b) on registers, the vector-ALU
// counterpart: FLOPs = iters * 16 * 2 * threads.  The library is built with
// packed FP32 disabled, so these are plain v_fma_f32 / v_fmac_f32, the same
// instruction the vector-FMA comparison kernel uses.
#include <hip/hip_runtime.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, float *out)
{
    const float a = 1.0f + 1e-7f * (float)(threadIdx.x & 7);
    const float b = 1.0f - 1e-7f * (float)(threadIdx.x >> 3 & 7);
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ void __launch_bounds__(512) empty_kernel(float *out)
{
    if (threadIdx.x == 0) out[blockIdx.x] = (float)blockIdx.x;
}

__global__ void __launch_bounds__(256) valu_peak_kernel(int iters, float *out)
{
    const float a = 1.0f - 1e-7f * (float)(1 + (threadIdx.x & 7));
    const float b = 1e-3f * (float)(threadIdx.x >> 3 & 7);
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = (float)j;
#pragma unroll 4
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = __builtin_fmaf(x[j], a, b);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += x[j];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

extern "C" {

// Launch `workgroups` workgroups of 4 waves (256 threads).  `out` must hold
// workgroups * 256 floats of device memory.  Returns the hipError_t of the
// launch; the work is asynchronous on `stream`.
int sgemm_probe_mfma_peak(int workgroups, int iters, float *out, hipStream_t stream)
{
    if (workgroups <= 0 || iters <= 0 || !out) return hipErrorInvalidValue;
    void *args[] = {&iters, &out};
    return hipLaunchKernel((const void *)&mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256),
                           args, 0, stream);
}

// FLOPs done by one probe launch.
double sgemm_probe_mfma_peak_flops(int workgroups, int iters)
{
    return (double)workgroups * 4.0 * (double)iters * 8.0 * 4096.0;
}

// The vector-FMA probe: `workgroups` workgroups of 256 threads; `out` must
// hold workgroups * 256 floats of device memory.  Asynchronous on `stream`.
int sgemm_probe_valu_peak(int workgroups, int iters, float *out, hipStream_t stream)
{
    if (workgroups <= 0 || iters <= 0 || !out) return hipErrorInvalidValue;
    void *args[] = {&iters, &out};
    return hipLaunchKernel((const void *)&valu_peak_kernel, dim3((unsigned)workgroups), dim3(256),
                           args, 0, stream);
}

double sgemm_probe_valu_peak_flops(int workgroups, int iters)
{
    return (double)workgroups * 256.0 * (double)iters * 16.0 * 2.0;
}

// The empty launch: `workgroups` workgroups of 512 threads; `out` must hold
// `workgroups` floats of device memory.  Asynchronous on `stream`.
int sgemm_probe_empty(int workgroups, float *out, hipStream_t stream)
{
    if (workgroups <= 0 || !out) return hipErrorInvalidValue;
    void *args[] = {&out};
    return hipLaunchKernel((const void *)&empty_kernel, dim3((unsigned)workgroups), dim3(512),
                           args, 0, stream);
}

}  // extern "C"
