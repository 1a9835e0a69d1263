"""Pins of the oracle's 8-bit GEMM (OCP FP8 E4M3 / E5M2 and INT8 inputs, k-major
A, BF16 output of scale x sum): the decoders against torch's own float8 types
and closed forms, the sums against brute force, the addressing against the
swapped product, the INT8 output's FP32 steps against numpy float32, the
special values, and the small-integer operands of the large-operand GPU tests
(their 8-bit codes, and the product restricted to sampled rows and columns)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

FMTS = ["f8e4m3", "f8e5m2", "i8"]


def test_decode8_exhaustive_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    for fmt, dt in (("f8e4m3", torch.float8_e4m3fn), ("f8e5m2", torch.float8_e5m2)):
        want = torch.from_numpy(codes.copy()).view(dt).to(torch.float64).numpy()
        got = oracle.decode8(codes, fmt)
        assert np.array_equal(np.isnan(got), np.isnan(want)), fmt
        ok = ~np.isnan(want)
        assert np.array_equal(got[ok], want[ok]), fmt
    assert np.array_equal(oracle.decode8(codes, "i8"), codes.view(np.int8).astype(np.float64))


def test_decode8_closed_forms():
    e4 = lambda c: oracle.decode8(np.array([c], np.uint8), "f8e4m3")[0]
    e5 = lambda c: oracle.decode8(np.array([c], np.uint8), "f8e5m2")[0]
    assert e4(0x38) == 1.0 and e4(0xB8) == -1.0 and e4(0x7E) == 448.0
    assert e4(0x01) == 2.0 ** -9 and e4(0x08) == 2.0 ** -6 and e4(0x07) == 7 * 2.0 ** -9
    assert math.isnan(e4(0x7F)) and math.isnan(e4(0xFF)) and e4(0x78) == 256.0
    assert e5(0x3C) == 1.0 and e5(0x7B) == 57344.0 and e5(0x01) == 2.0 ** -16
    assert e5(0x04) == 2.0 ** -14 and e5(0x7C) == math.inf and e5(0xFC) == -math.inf
    assert math.isnan(e5(0x7D)) and math.isnan(e5(0x7F))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_q_brute_force(fmt):
    M, N, K = 5, 4, 48
    At, B = synth.q8_operands(M, N, K, fmt, seed=3)
    a = oracle.decode8(At, fmt).reshape(M, K)
    b = oracle.decode8(B, fmt).reshape(N, K)
    r = oracle.gemm_tn_q(At, B, M, N, K, fmt, 1.0)
    assert r.macs == M * N * K
    for n in range(N):
        for m in range(M):
            want = math.fsum(float(a[m, k]) * float(b[n, k]) for k in range(K))
            assert r.exact[m + n * M] == (float(np.float32(want)) if fmt == "i8" else want)
            assert r.sabs[m + n * M] == math.fsum(abs(float(a[m, k]) * float(b[n, k])) for k in range(K))


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_q_swapped_operands_transpose(fmt):
    M, N, K = 7, 11, 32
    At, B = synth.q8_operands(M, N, K, fmt, seed=4)
    c = oracle.gemm_tn_q(At, B, M, N, K, fmt, 1.0).exact.reshape(N, M)
    ct = oracle.gemm_tn_q(B, At, N, M, K, fmt, 1.0).exact.reshape(M, N)
    assert np.array_equal(c, ct.T)


def test_int8_output_goes_through_fp32():
    # 1040 products 127 * 127 plus 127 * 24 and 9 * 1 sum to 2^24 + 1, which
    # is not an FP32 value: it becomes 2^24 before the scale.  The FP32
    # product with a scale is checked against numpy float32.
    At = np.concatenate([np.full(1040, 127), [127, 9], np.zeros(14)]).astype(np.int8)
    Bv = np.concatenate([np.full(1040, 127), [24, 1], np.zeros(14)]).astype(np.int8)
    K = At.size
    assert K % 16 == 0 and int(np.dot(At.astype(np.int64), Bv.astype(np.int64))) == 2 ** 24 + 1
    r = oracle.gemm_tn_q(At.view(np.uint8), Bv.view(np.uint8), 1, 1, K, "i8", 1.0)
    assert r.exact[0] == 2.0 ** 24 and r.bits[0] == 0x4B80
    r = oracle.gemm_tn_q(At.view(np.uint8), Bv.view(np.uint8), 1, 1, K, "i8", 0.1)
    assert r.exact[0] == float(np.float32(np.float32(2.0 ** 24 + 1) * np.float32(0.1)))


@pytest.mark.parametrize("fmt", ["f8e4m3", "f8e5m2"])
def test_fp8_scale_is_exactly_linear(fmt):
    M, N, K = 6, 5, 64
    At, B = synth.q8_operands(M, N, K, fmt, seed=6)
    r1 = oracle.gemm_tn_q(At, B, M, N, K, fmt, 1.0)
    r2 = oracle.gemm_tn_q(At, B, M, N, K, fmt, 2.0)
    r3 = oracle.gemm_tn_q(At, B, M, N, K, fmt, -0.5)
    assert np.array_equal(r2.exact, 2.0 * r1.exact) and np.array_equal(r3.exact, -0.5 * r1.exact)
    assert np.array_equal(r2.sabs, 2.0 * r1.sabs)


def test_fp8_special_values():
    # E5M2: inf * 0 is NaN, inf * 1 is inf; E4M3: a NaN input makes a NaN sum
    K = 16
    At = np.zeros(K, np.uint8)
    B = np.zeros(K, np.uint8)
    At[0], B[0] = 0x7C, 0x3C          # inf * 1
    r = oracle.gemm_tn_q(At, B, 1, 1, K, "f8e5m2", 1.0)
    assert r.exact[0] == math.inf and r.bits[0] == 0x7F80
    B[0] = 0x00                       # inf * 0
    assert math.isnan(oracle.gemm_tn_q(At, B, 1, 1, K, "f8e5m2", 1.0).exact[0])
    At[0], B[0] = 0x7F, 0x38          # E4M3 NaN * 1
    assert math.isnan(oracle.gemm_tn_q(At, B, 1, 1, K, "f8e4m3", 1.0).exact[0])


def test_sampled_entries_match_full():
    M, N, K = 33, 17, 80
    for fmt in FMTS:
        At, B = synth.q8_operands(M, N, K, fmt, seed=8)
        full = oracle.gemm_tn_q(At, B, M, N, K, fmt, 0.25)
        idx = np.array([0, 5, M * N - 1, 100, 257], np.int64)
        part = oracle.gemm_tn_q(At, B, M, N, K, fmt, 0.25, idx=idx)
        assert np.array_equal(part.bits, full.bits[idx]) and np.array_equal(part.exact, full.exact[idx])


@pytest.mark.parametrize("fmt", FMTS)
def test_to_q8_exact_on_small_integers(fmt):
    # the large-operand GPU tests store the integers -2..2 with synth.to_q8
    v = np.arange(-8, 9, dtype=np.float64)
    assert np.array_equal(oracle.decode8(synth.to_q8(v, fmt), fmt), v)


@pytest.mark.parametrize("fmt", FMTS)
def test_mod5_rows_and_columns_restrict_the_product(fmt):
    # the reference construction of the large-operand GPU tests: the operands
    # assembled from five repeated rows / columns, and the product restricted
    # to some rows and columns rebuilt from the formula, agree with the full
    # product at those entries
    M, N, K = 40, 30, 48
    kk = np.arange(K)
    arows = [synth.to_q8(synth.mod5_pattern(c, kk, 1, 3), fmt) for c in range(5)]
    bcols = [synth.to_q8(synth.mod5_pattern(kk, c, 1, 1), fmt) for c in range(5)]
    At = np.concatenate([arows[m % 5] for m in range(M)])
    B = np.concatenate([bcols[2 * n % 5] for n in range(N)])
    full = oracle.gemm_tn_q(At, B, M, N, K, fmt, 1.0).bits.reshape(N, M).T
    ms, ns = np.array([0, 3, 17, 39]), np.array([0, 1, 12, 29])
    Asub = synth.to_q8(synth.mod5_pattern(ms[:, None], kk[None, :], 1, 3).ravel(), fmt)
    Bsub = synth.to_q8(synth.mod5_pattern(kk[None, :], ns[:, None], 1, 2).ravel(), fmt)
    sub = oracle.gemm_tn_q(Asub, Bsub, len(ms), len(ns), K, fmt, 1.0).bits.reshape(len(ns), len(ms)).T
    assert np.array_equal(full[np.ix_(ms, ns)], sub)
    # and every entry is the exact integer sum, rounded once to BF16
    ref = np.array([[np.sum(synth.mod5_pattern(m, kk, 1, 3) * synth.mod5_pattern(kk, n, 1, 2)) for n in ns]
                    for m in ms])
    assert np.array_equal(synth.to_bits(ref.ravel(), "bf16").reshape(ref.shape), sub)
