"""FLOP/byte accounting against the worked examples the pages print (CPU only)."""

import json
import os

from io_aware_exact_attention_amd import accounting as acc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _close(value, printed, tol):
    """Within one unit of the last digit the page prints (it truncates as often as it rounds)."""
    return abs(value - printed) <= tol


def test_standard_attention_worked_io():
    g = GOLDEN["standard_attention_io_n4096_d128_bf16"]
    p = g["printed"]
    io = acc.standard_attention_io(g["n"], g["d"], g["elem_bytes"])
    assert _close(io["score_matrix_bytes"] / 1e6, p["score_matrix_MB"], 0.1)
    assert _close(io["score_round_trip_bytes"] / 1e6, p["score_round_trip_MB"], 1)
    assert _close(io["qkvo_bytes"] / 1e6, p["qkvo_MB"], 1)
    assert _close(100 * io["intermediate_share"], p["intermediate_share_percent"], 1)
    assert _close(io["flops"] / 1e9, p["flops_G"], 0.1)
    assert _close(io["bytes_moved"] / 1e6, p["bytes_moved_MB"], 1)
    assert _close(io["arithmetic_intensity"], p["arithmetic_intensity_flop_per_byte"], 1)
    assert io["arithmetic_intensity"] < p["a100_balance_flop_per_byte"]  # bandwidth-bound


def test_score_matrix_at_128k():
    g = GOLDEN["score_matrix_n131072"]
    b = acc.standard_attention_io(g["n"], 128, g["elem_bytes"])["score_matrix_bytes"]
    assert b == g["printed"]["score_matrix_GB"] * 2**30


def test_sfu_budget():
    g = GOLDEN["sfu_tile_budget_h100"]
    p = g["printed"]
    r = acc.sfu_tile_budget(g["block_m"], g["block_n"], g["d"], g["mma_flops_per_clk"], g["exp_per_clk"])
    assert _close(r["mma_flops"] / 1e6, p["mma_MFLOP"], 0.1)
    assert r["mma_cycles"] == p["mma_cycles"]
    assert r["exps"] == p["exps_k"] * 1024
    assert r["exp_cycles"] == p["exp_cycles"]
    assert 100 * r["exp_cycles"] / r["mma_cycles"] == p["exp_share_of_gemm_percent"]


def test_pairs_and_forward_flops_match_worked_compute():
    # one head, one sample, non-causal: 4 n^2 d
    assert acc.flops_fwd(acc.pairs(4096, 4096, False), 128) == 4 * 4096 * 4096 * 128
    assert acc.pairs(5, 5, True) == 15          # lower triangle incl. diagonal
    assert acc.pairs(4, 7, False) == 28


def test_headline_counts():
    c = acc.dense_counts(8, 16, 4096, 128, True)
    assert c["pairs"] == 8 * 16 * 4096 * 4097 // 2
    assert abs(c["flops_fwd"] / 1e9 - 549.9) < 0.1
    assert abs((c["flops_fwd"] + c["flops_bwd"]) / 1e12 - 1.925) < 0.001
    assert c["bytes_fwd"] == 8 * 4096 * 16 * (8 * 128 + 4)


def test_varlen_counts_reduce_to_dense():
    a = acc.varlen_counts([300, 300], 4, 64, True)
    b = acc.dense_counts(2, 4, 300, 64, True)
    assert a == b
