"""Host-side counting helpers pinned to numbers the pages print
(tests/golden/worked_examples.json holds each number with its citation)."""
import json
import os

import pytest

from fp32_gemm_sgemm_amd import metrics as m


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_examples.json")) as f:
        return json.load(f)


def test_flop_and_byte_counts(golden):
    e = golden["flop_byte"][0]
    assert round(m.gemm_flops(e["M"], e["N"], e["K"]) / 1e9) == e["gflop_rounded"]
    # "data" = A, B and C once each
    assert round(m.compulsory_bytes(e["M"], e["N"], e["K"]) / 1e6) == e["megabytes_rounded"]
    e = golden["flop_byte"][1]
    assert float(f"{m.gemm_flops(e['M'], e['N'], e['K']):.3g}") == e["flops_3sig"]
    naive_reads = 2 * e["M"] * e["N"] * e["K"]
    assert float(f"{naive_reads:.3g}") == e["naive_reads_3sig"]
    assert float(f"{naive_reads / e['tiled_T']:.2g}") == e["tiled_reads_2sig"]
    e = golden["flop_byte"][2]
    assert round(m.arithmetic_intensity(e["n"], e["n"], e["n"])) == e["ideal_ai_rounded"]


def test_tile_intensity(golden):
    for e in golden["tile_intensity"]:
        assert m.block_tile_intensity(e["BM"], e["BN"]) == e["ai"]


def test_ridge(golden):
    for e in golden["ridge"]:
        assert round(e["peak_gflops"] / e["bw_gbps"], 1) == e["ridge_1dp"]


def test_grid_geometry(golden):
    g0, g1, g2 = golden["geometry"]
    g = m.one_thread_per_output_grid(g0["rows"], g0["cols"], g0["tx"], g0["ty"])
    assert [g.grid_x, g.grid_y] == g0["grid"]
    assert (g.blocks, g.threads, g.useful, g.idle) == (g0["blocks"], g0["threads"], g0["useful"], g0["idle"])
    g = m.one_thread_per_output_grid(g1["rows"], g1["cols"], g1["T"], g1["T"], g1["shared"], g1["T"])
    assert [g.grid_x, g.grid_y] == g1["grid"]
    assert (g.blocks, g.threads, g.useful, g.phases) == (g1["blocks"], g1["threads"], g1["writers"], g1["phases"])
    assert m.ceil_div(g2["n"], g2["tpb"]) == g2["blocks"]


def test_wave_utilisation(golden):
    e = golden["waves"][0]
    assert round(m.wave_utilisation(e["workgroups"], e["slots"]), 2) == e["utilisation_2sig"]


def test_mi355x_peak():
    assert abs(m.fp32_matrix_peak_tflops() - m.MI355X_FP32_MATRIX_PEAK_TFLOPS) < 0.05
    assert m.tile_operand_bytes(256, 256, 16, 128, 128) == 4 * 16 * (2 * 256 + 2 * 256)
