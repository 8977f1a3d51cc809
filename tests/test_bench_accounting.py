"""The benchmark's FLOP, byte and throughput accounting, pinned to figures
printed on the pages (tests/golden/page_figures.txt)."""
import pytest

import bench
from golden_io import page_figures

F = page_figures()


def test_flops_match_the_4096_cycle_identity():
    # 1550 TFLOP/s at 4096^3 is 88.7 microseconds
    t = bench.gemm_flops(4096, 4096, 4096) / (F["p1_tflops_4096"] * 1e12)
    assert t * 1e6 == pytest.approx(F["p1_us_4096"], rel=2e-3)
    # 512 CTAs x 64 k-tiles over 160 SMs
    assert 512 * 64 / 160 == pytest.approx(F["p1_ktiles_per_sm"], rel=3e-3)


def test_naive_ladder_rate():
    tf = bench.gemm_flops(1024, 1024, 1024) / (F["p2_naive_ms_1024"] * 1e-3) / 1e12
    assert tf == pytest.approx(F["p2_naive_tflops_1024"], rel=0.02)


def test_ideal_intensity():
    assert bench.ideal_intensity(1024, 1024, 1024, 4) == pytest.approx(1024 / 6)
    assert bench.ideal_intensity(1024, 1024, 1024, 4) == pytest.approx(
        F["p2_ideal_intensity_1024_fp32"], rel=3e-3)
    assert bench.ideal_intensity(1, 4096, 4096, 2) == pytest.approx(
        F["p2_ideal_intensity_m1_fp16"], rel=1e-3)


def test_prefill_flop_ledger():
    flop = 2 * F["p4_params"] * F["p4_tokens"]
    assert flop == pytest.approx(F["p4_prefill_flop"], rel=0.02)
    # the 7B-like stack's projection weights are consistent with that ledger
    weights = 32 * (4 * 4096 * 4096 + 2 * 11008 * 4096 + 4096 * 11008)
    assert weights == pytest.approx(F["p4_params"], rel=0.07)


def test_alg_bytes_and_dequant_bytes():
    assert bench.gemm_alg_bytes(4096, 4096, 4096, 2, 2) == 3 * 4096 * 4096 * 2
    assert bench.dequant_alg_bytes(11008, 4096) == 11008 * 4096 * (18 / 32 + 2)


def test_stack_tokens_per_s():
    assert bench.prefill_stack_tokens_per_s(1e-6, 2e-6, 3e-6) == pytest.approx(
        2048 / (32 * (4e-6 + 4e-6 + 3e-6)))


def test_source_hash_ignores_comments_only():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "x // y"; char q = \'"\';\n'
    assert bench._strip_comments(src) == 'int a = 1;\n const char* s = "x // y"; char q = \'"\';'
    assert bench._strip_comments("a /* x */ + b // y\n") == "a  + b"
