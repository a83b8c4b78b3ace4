"""Host-side counting for single-precision GEMM: work, bytes, intensity, peak,
and launch geometry.  Integer and float bookkeeping only; no product arithmetic.

* Work: 2*M*N*K floating-point operations ("4.1 CUDA GEMM operator
  performance optimization", section 1.1; throughput as defined in its
  section 1.3).
* Compulsory bytes: read A and B once, write C once, 4 bytes per float (the
  "ideal matmul" count of the DD2360 workbook, Module 4 exercises).
* Block-tile intensity: BM*BN / (2*(BM+BN)) FLOP per byte ("4.1 ...",
  section 4.3).
* Peak: units x FLOP per clock x clock (DD2360 workbook, Module 3: peak
  FP32 = cores x 2 x clock).  MI355X: 256 CUs x 256 FP32 matrix FLOP per
  clock per CU x 2.4 GHz = 157.3 TFLOP/s.
* Geometry: round-up grid sizing with a guard (DD2360 workbook, Module 6,
  section 6.3, and its 2-D worked example in section 6.5).
"""
from dataclasses import dataclass

MI355X_CUS = 256
MI355X_CLOCK_HZ = 2.4e9
MI355X_FP32_MATRIX_FLOP_PER_CLK_PER_CU = 256
MI355X_FP32_MATRIX_PEAK_TFLOPS = 157.3        # published figure
MI355X_HBM_PEAK_GBPS = 8000.0                 # published figure (8 TB/s)


def ceil_div(a: int, b: int) -> int:
    if b <= 0:
        raise ValueError("divisor must be positive")
    return -(-a // b)


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def compulsory_bytes(M: int, N: int, K: int, elem: int = 4) -> int:
    """Read A (M x K) and B (K x N) once and write C (M x N) once."""
    return elem * (M * K + K * N + M * N)


def arithmetic_intensity(M: int, N: int, K: int) -> float:
    return gemm_flops(M, N, K) / compulsory_bytes(M, N, K)


def block_tile_intensity(BM: int, BN: int) -> float:
    """FLOP per byte of a BM x BN block tile that loads BM*BK + BK*BN floats
    per BK-slice; BK cancels."""
    return BM * BN / (2.0 * (BM + BN))


def tile_operand_bytes(M: int, N: int, K: int, BM: int, BN: int, elem: int = 4) -> int:
    """Bytes that all block tiles together read from the cache hierarchy when
    every tile reads its A strip and B strip once (ragged tiles counted
    whole): elem * K * (ceil(N/BN)*M + ceil(M/BM)*N)."""
    return elem * K * (ceil_div(N, BN) * M + ceil_div(M, BM) * N)


def fp32_matrix_peak_tflops(cus: int = MI355X_CUS, clock_hz: float = MI355X_CLOCK_HZ,
                            flop_per_clk_per_cu: int = MI355X_FP32_MATRIX_FLOP_PER_CLK_PER_CU) -> float:
    return cus * flop_per_clk_per_cu * clock_hz / 1e12


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    return gemm_flops(M, N, K) / seconds / 1e12


@dataclass(frozen=True)
class Grid2D:
    """A 2-D launch with one thread per output element, Tx x Ty threads per
    block, x over columns and y over rows."""
    grid_x: int
    grid_y: int
    blocks: int
    threads: int
    useful: int
    idle: int
    phases: int          # steps along the shared dimension for a square tile


def one_thread_per_output_grid(rows: int, cols: int, tx: int, ty: int,
                               shared: int = 0, tile_k: int = 0) -> Grid2D:
    gx, gy = ceil_div(cols, tx), ceil_div(rows, ty)
    blocks = gx * gy
    threads = blocks * tx * ty
    useful = rows * cols
    phases = ceil_div(shared, tile_k) if tile_k else 0
    return Grid2D(gx, gy, blocks, threads, useful, threads - useful, phases)


def wave_utilisation(n_workgroups: int, slots: int) -> float:
    """Fraction of workgroup slots busy over the whole launch when every
    workgroup takes the same time: n / (ceil(n/slots) * slots)."""
    if n_workgroups <= 0:
        return 0.0
    return n_workgroups / (ceil_div(n_workgroups, slots) * slots)
