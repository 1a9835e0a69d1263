"""GPU parity of the 8-bit GEMMs (OCP FP8 E4M3 / E5M2 and INT8 inputs, A
k-major, BF16 output of scale x sum) through the C ABI against the CPU
oracle: every output at small and ragged sizes on each tile, INT8 bit-exact
(including sums that FP32 cannot hold), FP8 within the FP32-accumulation
bound, non-finite FP8 inputs by class, and sampled outputs of the
8192 x 8192 x 16384 product in the launch configuration the report times."""
import numpy as np
import pytest

import oracle
import synth
from helpers import gemm_tn_q_gpu

pytestmark = pytest.mark.gpu

FMTS = ["f8e4m3", "f8e5m2", "i8"]
TILES = [0, 9, 10, 13]
SHAPES = [(300, 200, 272), (513, 129, 1040), (64, 64, 16), (1000, 37, 2064), (17, 600, 48)]


def _check(got, ref, fmt, what):
    if fmt == "i8":
        assert np.array_equal(got, ref.bits), "%s: %d of %d differ" % (
            what, int(np.sum(got != ref.bits)), got.size)
    else:
        ok, rep = oracle.check(got, ref, "bf16")
        assert ok, "%s: %s" % (what, rep)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("fmt", FMTS)
def test_each_tile_ragged(tile, fmt):
    for i, (M, N, K) in enumerate(SHAPES):
        print("case q8", fmt, tile, M, N, K, flush=True)
        At, B = synth.q8_operands(M, N, K, fmt, seed=300 + i)
        scale = 0.0625 if fmt == "i8" else 0.75
        got, guards, unchanged = gemm_tn_q_gpu(At, B, M, N, K, fmt, scale, tile)
        assert guards and unchanged
        _check(got, oracle.gemm_tn_q(At, B, M, N, K, fmt, scale), fmt, "%s tile %d %s" % (fmt, tile, (M, N, K)))


@pytest.mark.parametrize("fmt", ["f8e4m3", "f8e5m2"])
def test_fp8_wide_tile_ragged(fmt):
    # tile 17: whole 64-unit steps on the double-rate 16x16x128 FP8 MFMA
    # (K = 16 or 48 bytes: one stage with a leading zero half; 160 and 192:
    # two stages, fewer than the ring holds; 272: three)
    for i, (M, N, K) in enumerate(SHAPES + [(520, 264, 4096), (256, 128, 128), (264, 130, 160), (300, 140, 192)]):
        print("case q8 wide", fmt, M, N, K, flush=True)
        At, B = synth.q8_operands(M, N, K, fmt, seed=500 + i)
        got, guards, unchanged = gemm_tn_q_gpu(At, B, M, N, K, fmt, 0.75, 17)
        assert guards and unchanged
        _check(got, oracle.gemm_tn_q(At, B, M, N, K, fmt, 0.75), fmt, "%s tile 17 %s" % (fmt, (M, N, K)))


def test_fp8_wide_tile_non_finite():
    M, N, K = 64, 40, 256
    At, B = synth.q8_operands(M, N, K, "f8e5m2", seed=53)
    At[0] = 0x7C                                     # +inf in row 0
    At[K + 130] = 0x7D                               # NaN in row 1, second stage
    B[5 * K + 200] = 0xFC                            # -inf in column 5
    got, _, _ = gemm_tn_q_gpu(At, B, M, N, K, "f8e5m2", 1.0, 17)
    _check(got, oracle.gemm_tn_q(At, B, M, N, K, "f8e5m2", 1.0), "f8e5m2", "wide e5m2 non-finite")
    At, B = synth.q8_operands(M, N, K, "f8e4m3", seed=54)
    At[:K] = 0x7E                                    # row 0 of A: 448 everywhere
    got, _, _ = gemm_tn_q_gpu(At, B, M, N, K, "f8e4m3", 1.0, 17)
    _check(got, oracle.gemm_tn_q(At, B, M, N, K, "f8e4m3", 1.0), "f8e4m3", "wide e4m3 extremes")


def test_int8_large_sums_exact():
    # all entries +-127: sums up to K * 16129 exceed 2^24 and go through FP32
    rng = np.random.default_rng(41)
    M, N, K = 256, 256, 4096
    At = (rng.integers(0, 2, M * K) * 254 - 127).astype(np.int8).view(np.uint8)
    B = np.full(N * K, 127, np.int8).view(np.uint8)
    for scale in (1.0, 1.0 / 3.0):
        got, g, _ = gemm_tn_q_gpu(At, B, M, N, K, "i8", scale)
        assert g
        _check(got, oracle.gemm_tn_q(At, B, M, N, K, "i8", scale), "i8", "large sums scale %g" % scale)


def test_fp8_extremes_and_non_finite():
    # E4M3 extremes (448, smallest subnormal) and E5M2 infinities / NaN
    M, N, K = 32, 32, 64
    At, B = synth.q8_operands(M, N, K, "f8e4m3", seed=51)
    At[:K] = 0x7E                                    # row 0 of A: 448 everywhere
    At[K:2 * K] = 0x01                               # row 1: 2^-9
    got, _, _ = gemm_tn_q_gpu(At, B, M, N, K, "f8e4m3", 1.0)
    _check(got, oracle.gemm_tn_q(At, B, M, N, K, "f8e4m3", 1.0), "f8e4m3", "e4m3 extremes")
    At, B = synth.q8_operands(M, N, K, "f8e5m2", seed=52)
    At[0] = 0x7C                                     # +inf in row 0
    At[K + 3] = 0x7D                                 # NaN in row 1
    got, _, _ = gemm_tn_q_gpu(At, B, M, N, K, "f8e5m2", 1.0)
    _check(got, oracle.gemm_tn_q(At, B, M, N, K, "f8e5m2", 1.0), "f8e5m2", "e5m2 non-finite")


@pytest.mark.parametrize("fmt", FMTS)
def test_headline_size_sampled(fmt):
    M = N = 8192
    K = 16384
    print("case q8 headline", fmt, flush=True)
    At, B = synth.q8_operands(M, N, K, fmt, seed=61)
    scale = 2.0 ** -10 if fmt == "i8" else 1.0
    got, g, _ = gemm_tn_q_gpu(At, B, M, N, K, fmt, scale)
    assert g
    idx = synth.sample_indices(M, N, 61, 2048)
    _check(got[idx], oracle.gemm_tn_q(At, B, M, N, K, fmt, scale, idx=idx), fmt, "headline sampled")
