"""Consistency of the figures the pages print (tests/golden/pages_figures.json) with
the MI355X FP8 dense peak the benchmark divides by.

MI355X: 256 compute units x 4 SIMDs at 2.4 GHz.  The pages' block of 32 queries x
128 keys at head dim 128 is 2 matmuls x 2*32*128*128 FLOP and takes 1024 matrix
cycles; that fixes 2048 FP8 FLOP per clock per SIMD, i.e. the 5.03 PFLOP/s dense
peak, and 2672 TFLOP/s is then the printed 53%.
"""
import json
import os

from fp8_causal_prefill_tiled_amd.workloads import WORKLOADS

HERE = os.path.dirname(os.path.abspath(__file__))
FIG = {k: v["value"] for k, v in json.load(open(os.path.join(HERE, "golden", "pages_figures.json"))).items()
       if not k.startswith("_")}

FP8_PEAK_TFLOPS = 5033.165  # 256 CU * 4 SIMD * 2048 FLOP/clk * 2.4 GHz


def test_cycle_model_fixes_the_fp8_peak():
    flop = 2 * (2 * FIG["block_queries"] * FIG["block_keys"] * 128)
    per_simd_clk = flop / FIG["mfma_cycles_per_block_fp8_d128"]
    assert per_simd_clk == 2048
    peak = 256 * 4 * per_simd_clk * 2.4e9 / 1e12
    assert abs(peak - FP8_PEAK_TFLOPS) < 1e-3
    assert round(FIG["zyfa_fp8_tflops_d128_32k_gaussian"] / peak, 2) == FIG["zyfa_fp8_share_of_peak"]
    assert round(FIG["aiter_fp8_tflops_d128_32k_gaussian"] / peak, 2) == FIG["aiter_fp8_share_of_peak"]


def test_valu_budget_per_score():
    scores = FIG["block_queries"] * FIG["block_keys"]
    # wave64 VALU instructions issue over 4 cycles on a 16-lane SIMD
    assert FIG["exact_softmax_valu_cycles_per_block"] / 4 / (scores / 64) == 3.5
    assert FIG["lean_p_valu_cycles_per_block"] / 4 / (scores / 64) == 1.5


def test_causal_flop_formula():
    w = WORKLOADS["gauss32k"]
    assert w.causal_flops == 2 * 1 * 32 * 32768 ** 2 * 256 / 2
    assert abs(w.causal_flops / 1e12 - 8.796) < 1e-3
