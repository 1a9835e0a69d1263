"""Pin the FLOP, byte and roofline arithmetic against numbers the pages
print (tests/golden/page_numbers.json names the page and section of each)."""
import json
import os

import pytest

from bf16_gemm_decode_amd import roofline as rf

HERE = os.path.dirname(os.path.abspath(__file__))
P = json.load(open(os.path.join(HERE, "golden", "page_numbers.json")))


def close(a, b, rel):
    return abs(a - b) <= rel * abs(b)


def test_contest_flops():
    g = P["gemm_contest"]
    assert close(rf.gemm_flop(g["M"], g["N"], g["K"]), g["flop_approx"], g["rel_tol"])
    assert rf.gemm_flop(g["M"], g["N"], g["K"]) == 2 * 8192 * 8192 * 16384


def test_contest_kernel_time():
    g, t = P["gemm_contest"], P["gemm_contest_time"]
    ms = rf.seconds_at(rf.gemm_flop(g["M"], g["N"], g["K"]), t["tflops"] * 1e12) * 1e3
    assert close(ms, t["ms_approx"], t["rel_tol"])


def test_roofline_low_and_high_intensity():
    lo, hi = P["roofline_low_intensity"], P["roofline_high_intensity"]
    assert close(rf.attainable_tflops(lo["peak_tflops"], lo["hbm_GBps"], lo["intensity"]),
                 lo["attainable_tflops"], lo["rel_tol"])
    assert rf.bound(lo["peak_tflops"], lo["hbm_GBps"], lo["intensity"]) == lo["bound"]
    assert close(rf.bandwidth_roof_tflops(hi["hbm_GBps"], hi["intensity"]),
                 hi["bandwidth_roof_tflops"], hi["rel_tol"])
    assert rf.attainable_tflops(hi["peak_tflops"], hi["hbm_GBps"], hi["intensity"]) == \
        hi["attainable_tflops"]
    assert rf.bound(hi["peak_tflops"], hi["hbm_GBps"], hi["intensity"]) == hi["bound"]


def test_ridge():
    r = P["ridge"]
    assert close(rf.ridge(r["peak_tflops"], r["hbm_GBps"]), r["ridge_flop_per_byte"], r["rel_tol"])


def test_decode_weight_io_estimate():
    d = P["decode_weight_io"]
    assert close(d["weight_GB"] / d["hbm_TBps"], d["io_ms"], d["rel_tol"])
    assert close(rf.seconds_at(d["flop_G"] * 1e9, d["peak_tflops"] * 1e12) * 1e3,
                 d["compute_ms"], 0.05)


def test_gemv_bytes_and_intensity():
    s = P["gate_up_shape"]
    m, k = s["m"], s["k"]
    assert rf.gemv_bytes(m, k, 1) == 2 * (m * k + k + m)
    assert m * k * 2 == 356_515_840
    # decode is about 1 FLOP per byte: far below any ridge point
    assert 0.99 < rf.intensity(rf.gemv_flop(m, k, 1), rf.gemv_bytes(m, k, 1)) < 1.0
    assert rf.bound(2500.0, 8000.0, 1.0) == "hbm"


def test_rows_per_block_sweep_rates():
    # Derived: bytes of W over the page's times give the effective bandwidth.
    s, w = P["rows_per_block_sweep"], P["gate_up_shape"]
    gbps = [w["m"] * w["k"] * 2 / (t * 1e-3) / 1e9 for t in s["ms"]]
    assert max(range(4), key=lambda i: gbps[i]) == s["rows"].index(8)
    assert close(gbps[2], 1018.6, 0.002)


def test_mi355x_peaks():
    assert rf.MI355X["mfma_bf16_tflops"] == 2500.0 and rf.MI355X["hbm_GBps"] == 8000.0
    # dense FP16/BF16 MFMA: 256 CUs x 4096 FLOP/clk x 2.4 GHz
    assert close(256 * 4096 * 2.4e9 / 1e12, 2516.6, 1e-4)


def test_attention_segment_table():
    # the section 7 table and its stated conclusions: 32 segments lose at 8K,
    # win by about 10% at 16K and about 21% at 32K, so 32 segments pay off
    # only above a length between 8K and 16K (the page sets 12,288)
    a = P["attention_segments"]
    assert a["ms_32"]["8192"] > a["ms_16"]["8192"]
    for L, stated in (("16384", a["stated_speedup_16k"]), ("32768", a["stated_speedup_32k"])):
        gain = 1.0 - a["ms_32"][L] / a["ms_16"][L]
        assert abs(gain - stated) <= a["speedup_tol"], (L, gain)
    assert 8192 < a["use_32_from_length"] <= 16384
    assert a["heads_q"] % a["heads_kv"] == 0
