"""MI355X-native single-precision GEMM (row-major) behind a C ABI.

The compute path is the HIP library libsgemm.so (built from csrc/ for gfx950):
C = alpha * op(A) x op(B) + beta * C with optional transposed operands, strided
batches and K split across workgroups.  This package holds its thin ctypes
binding (binding.py), the seeded input generators (inputs.py) and host-side
counting (metrics.py).  libsgemm_lds_poison.so is the same code built as an
LDS race check, for the tests; libsgemm_timeline.so is the same code with
clock readings inside the direct-load kernel, which timeline.py reports.  The
library is loaded on first use; if it is missing, every entry point raises.
"""
from .binding import (  # noqa: F401
    SgemmCfg, SgemmError, load, sgemm, sgemm_batched, sgemm_f32, sgemm_f32_cfg_geometry,
    sgemm_f32_ex, sgemm_f32_ex_noalloc, sgemm_f32_gemm, sgemm_f32_num_variants, sgemm_f32_plan, sgemm_f32_query,
    sgemm_f32_strided_batched, sgemm_f32_variant, sgemm_f32_variant_ops, sgemm_f32_version,
    sgemm_f32_workspace_size, library, LIB_PATH, POISON_LIB_PATH, TIMELINE_LIB_PATH,
    SGEMM_KERNEL_MFMA, SGEMM_KERNEL_VALU, SGEMM_OP_N, SGEMM_OP_T, SGEMM_SCRATCH_BYTES,
)
