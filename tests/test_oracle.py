"""Pins for the CPU oracle, against things other than the oracle itself:
numpy/torch conversions, closed-form rounding ties, numpy's float64 matmul,
exact integer arithmetic, identity and permutation matrices, brute force on
tiny inputs, and a hand-worked example of the grouped tile ordering.
Each test is chosen so that a plausible slip in ``oracle/oracle.c`` (a
dropped term, a transposed operand, a wrong index stride, a wrong rounding
mode or a double rounding) fails at least one of them."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def colmajor(flat, rows, cols):
    return np.asarray(flat).reshape(cols, rows).T


def as_flat_colmajor(mat):
    return np.asarray(mat).ravel(order="F")


# ---- codecs ------------------------------------------------------------------

def test_decode_fp16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    want = t.to(torch.float32).numpy().astype(np.float64)
    got = oracle.decode(bits, "bf16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


@pytest.mark.parametrize("x,expect", [
    (1.0 + 2.0 ** -11, 0x3C00),          # tie between 1 and 1+2^-10 -> even (1.0)
    (1.0 + 3 * 2.0 ** -11, 0x3C02),      # tie between 1+2^-10 and 1+2^-9 -> even
    (1.0 + 2.0 ** -11 + 2.0 ** -30, 0x3C01),  # just above the tie -> up
    (65504.0, 0x7BFF),                   # largest finite
    (65519.99, 0x7BFF),                  # below the overflow tie
    (65520.0, 0x7C00),                   # overflow tie rounds to even = Inf
    (-1e6, 0xFC00),
    (2.0 ** -24, 0x0001),                # smallest subnormal
    (2.0 ** -25, 0x0000),                # tie between 0 and 2^-24 -> even (0)
    (3 * 2.0 ** -25, 0x0002),            # tie between 2^-24 and 2^-23 -> even
    (2.0 ** -14 - 2.0 ** -25, 0x0400),   # tie between max subnormal and min normal -> even
    (-0.0, 0x8000),
    (0.0, 0x0000),
])
def test_encode_fp16_closed_form(x, expect):
    assert int(oracle.encode([x], "f16")[0]) == expect


@pytest.mark.parametrize("x,expect", [
    (1.0 + 2.0 ** -8, 0x3F80),           # tie -> even (1.0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),       # tie -> even (1+2^-6)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # above the tie only in float64: must round up
    (3.3895313892515355e38, 0x7F7F),     # largest finite bfloat16
    (3.4e38, 0x7F80),                    # rounds past the largest finite -> Inf
    (2.0 ** -133, 0x0001),               # smallest subnormal
    (2.0 ** -134, 0x0000),               # tie -> even (0)
    (-2.5, 0xC020),
])
def test_encode_bf16_closed_form(x, expect):
    assert int(oracle.encode([x], "bf16")[0]) == expect


def test_encode_nan_inf_classes():
    for fmt in ("f16", "bf16"):
        out = oracle.decode(oracle.encode([np.nan, np.inf, -np.inf], fmt), fmt)
        assert np.isnan(out[0]) and out[1] == np.inf and out[2] == -np.inf


def test_encode_fp16_sweep_vs_numpy():
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.uniform(-70000, 70000, 20000),
        rng.normal(0, 1, 20000),
        rng.normal(0, 1e-5, 20000),       # subnormal range
        np.ldexp(rng.uniform(1, 2, 20000), rng.integers(-30, 17, 20000)),
    ])
    # exact float16 midpoints, both signs
    h = rng.integers(0, 0x7BFF, 5000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    x = np.concatenate([x, (lo + hi) / 2, -(lo + hi) / 2])
    assert np.array_equal(oracle.encode(x, "f16"), x.astype(np.float16).view(np.uint16))


def test_encode_bf16_sweep_vs_torch():
    # On float32-representable inputs one rounding from float64 equals
    # torch's float32 -> bfloat16 nearest-even conversion.
    rng = np.random.default_rng(7)
    x32 = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 1e-38, 5000),
        np.ldexp(rng.uniform(1, 2, 20000), rng.integers(-140, 128, 20000)),
    ]).astype(np.float32)
    x32 = x32[np.isfinite(x32)]
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode(x32.astype(np.float64), "bf16"), want)


def test_roundtrip_all_finite_patterns():
    for fmt in ("f16", "bf16"):
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        v = oracle.decode(bits, fmt)
        fin = np.isfinite(v)
        assert np.array_equal(oracle.encode(v[fin], fmt), bits[fin])


# ---- GEMM triple loop ----------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (16, 9, 33), (31, 17, 64), (7, 1, 100)])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_gemm_matches_numpy_matmul(M, N, K, fmt):
    A, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), seed=M * 1000 + N * 10 + K)
    r = oracle.gemm(A, B, M, N, K, fmt)
    a = colmajor(oracle.decode(A, fmt), M, K)
    b = colmajor(oracle.decode(B, fmt), K, N)
    ref = a @ b
    got = colmajor(r.exact, M, N)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * (np.abs(a) @ np.abs(b)).max())
    assert np.allclose(colmajor(r.sabs, M, N), np.abs(a) @ np.abs(b), rtol=1e-12)
    assert np.array_equal(r.bits, oracle.encode(r.exact, fmt))
    assert r.macs == M * N * K


def test_gemm_brute_force_tiny():
    # Pure-Python loops with exactly rounded sums (math.fsum) on tiny inputs.
    rng = np.random.default_rng(5)
    for (M, N, K) in [(2, 3, 4), (4, 2, 3), (1, 4, 5), (3, 3, 1)]:
        A = synth.to_bits(rng.normal(0, 1, M * K), "f16")
        B = synth.to_bits(rng.normal(0, 1, K * N), "f16")
        av = A.view(np.float16).astype(float)
        bv = B.view(np.float16).astype(float)
        r = oracle.gemm(A, B, M, N, K, "f16")
        for n in range(N):
            for m in range(M):
                terms = [av[m + k * M] * bv[k + n * K] for k in range(K)]
                exact = math.fsum(terms)
                # few exact products of normal(0,1) values: the float64
                # running sum is itself exact, so it must equal fsum.
                assert r.exact[m + n * M] == exact
                assert r.bits[m + n * M] == np.float64(exact).astype(np.float16).view(np.uint16)


def test_gemm_identity_and_permutation_bit_exact():
    n, N = 24, 7
    rng = np.random.default_rng(11)
    for fmt in ("f16", "bf16"):
        X = synth.to_bits(rng.normal(0, 3, n * N), fmt)          # n x N, column-major
        I = synth.to_bits(synth.identity_colmajor(n), fmt)
        # A = I: C == B bit for bit
        assert np.array_equal(oracle.gemm(I, X, n, N, n, fmt).bits, X)
        # B = I: C == A bit for bit (A is N x n here)
        Xt = synth.to_bits(rng.normal(0, 3, N * n), fmt)         # N x n
        assert np.array_equal(oracle.gemm(Xt, I, N, n, n, fmt).bits, Xt)
        # A = cyclic shift P with P(i, (i+s) mod n) = 1: (P X)(i, :) = X((i+s) mod n, :)
        for s in (1, 5):
            P = synth.to_bits(synth.cyclic_shift_colmajor(n, s), fmt)
            got = colmajor(oracle.gemm(P, X, n, N, n, fmt).bits, n, N)
            want = np.roll(colmajor(X, n, N), -s, axis=0)
            assert np.array_equal(got, want)


def test_gemm_transpose_identity_on_integers():
    # (A B)^T = B^T A^T, on integer data where every sum is exact.
    rng = np.random.default_rng(3)
    M, N, K = 9, 13, 21
    a = synth.small_ints(rng, M * K, -3, 3)
    b = synth.small_ints(rng, K * N, -3, 3)
    A, B = synth.to_bits(a, "f16"), synth.to_bits(b, "f16")
    C = colmajor(oracle.gemm(A, B, M, N, K, "f16").exact, M, N)
    At = as_flat_colmajor(colmajor(a, M, K).T)
    Bt = as_flat_colmajor(colmajor(b, K, N).T)
    Ct = colmajor(oracle.gemm(synth.to_bits(Bt, "f16"), synth.to_bits(At, "f16"),
                              N, M, K, "f16").exact, N, M)
    assert np.array_equal(C.T, Ct)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_gemm_small_integers_exact(fmt):
    rng = np.random.default_rng(17)
    M, N, K = 33, 29, 64
    a = synth.small_ints(rng, M * K, -3, 3)
    b = synth.small_ints(rng, K * N, -3, 3)
    r = oracle.gemm(synth.to_bits(a, fmt), synth.to_bits(b, fmt), M, N, K, fmt)
    want = colmajor(a, M, K).astype(np.int64) @ colmajor(b, K, N).astype(np.int64)
    assert np.array_equal(colmajor(r.exact, M, N), want)
    # |C| <= 9*64 = 576: exact in both formats only up to 256 for bf16
    ok = np.abs(want) <= (2048 if fmt == "f16" else 256)
    assert np.array_equal(colmajor(oracle.decode(r.bits, fmt), M, N)[ok], want[ok])


def test_gemm_k_split_additivity():
    rng = np.random.default_rng(19)
    M, N, K, k1 = 10, 6, 40, 17
    a = colmajor(synth.small_ints(rng, M * K, -4, 4), M, K)
    b = colmajor(synth.small_ints(rng, K * N, -4, 4), K, N)

    def run(aa, bb):
        m, k = aa.shape
        n = bb.shape[1]
        return colmajor(oracle.gemm(synth.to_bits(as_flat_colmajor(aa), "f16"),
                                    synth.to_bits(as_flat_colmajor(bb), "f16"),
                                    m, n, k, "f16").exact, m, n)
    assert np.array_equal(run(a, b), run(a[:, :k1], b[:k1]) + run(a[:, k1:], b[k1:]))


def test_gemm_output_rounding_ties():
    # K=2, a = [1, 3*2^-11], b = [1, 1]: exact sum 1 + 3*2^-11 is a binary16
    # tie; nearest-even gives 1 + 2^-9 (truncation would give 1 + 2^-10).
    A = synth.to_bits([1.0, 3 * 2.0 ** -11], "f16")
    B = synth.to_bits([1.0, 1.0], "f16")
    assert int(oracle.gemm(A, B, 1, 1, 2, "f16").bits[0]) == 0x3C02
    A = synth.to_bits([1.0, 3 * 2.0 ** -8], "bf16")
    B = synth.to_bits([1.0, 1.0], "bf16")
    assert int(oracle.gemm(A, B, 1, 1, 2, "bf16").bits[0]) == 0x3F82


def test_gemm_degenerate_k0():
    r = oracle.gemm(np.zeros(0, np.uint16), np.zeros(0, np.uint16), 3, 2, 0, "f16")
    assert np.array_equal(r.bits, np.zeros(6, np.uint16)) and r.macs == 0


def test_gemm_nonfinite_propagation():
    # An Inf in A row 0 makes C(0, n) non-finite; other rows stay finite.
    M, N, K = 3, 2, 4
    a = np.ones(M * K)
    a[0 + 2 * M] = np.inf
    r = oracle.gemm(synth.to_bits(a, "f16"), synth.to_bits(np.ones(K * N), "f16"), M, N, K, "f16")
    v = colmajor(oracle.decode(r.bits, "f16"), M, N)
    assert np.all(np.isinf(v[0])) and np.all(v[1:] == 4.0)


def test_gemm_sampled_equals_full():
    M, N, K = 37, 23, 50
    A, B = synth.gemm_operands(M, N, K, "bf16", ("normal", 1.0, 1.0), seed=9)
    full = oracle.gemm(A, B, M, N, K, "bf16")
    idx = synth.sample_indices(M, N, seed=9, count=100)
    s = oracle.gemm_sampled(A, B, M, N, K, idx, "bf16")
    assert np.array_equal(s.bits, full.bits[idx])
    assert np.array_equal(s.exact, full.exact[idx])
    assert s.macs == idx.size * K


def test_sample_indices_contract():
    idx = synth.sample_indices(8192, 8192, seed=1)
    assert 4096 <= idx.size <= 4100
    assert idx.min() == 0 and idx.max() == 8192 * 8192 - 1
    assert np.array_equal(idx, np.unique(idx))
    assert np.array_equal(idx, synth.sample_indices(8192, 8192, seed=1))


# ---- GEMV ---------------------------------------------------------------------

@pytest.mark.parametrize("M,K,n", [(5, 7, 1), (64, 33, 4), (19, 130, 16)])
def test_gemv_matches_numpy(M, K, n):
    W, X = synth.gemv_operands(M, K, n, seed=M + K + n)
    r = oracle.gemv(W, X, M, K, n)
    w = oracle.decode(W, "bf16").reshape(M, K)
    x = oracle.decode(X, "bf16").reshape(n, K)
    ref = x @ w.T                       # Y = X W^T, [n, M]
    assert np.allclose(r.exact.reshape(n, M), ref, rtol=1e-12, atol=1e-13)
    assert np.allclose(r.sabs.reshape(n, M), np.abs(x) @ np.abs(w).T, rtol=1e-12)
    assert r.macs == n * M * K


def test_gemv_one_hot_selects_column():
    M, K = 40, 50
    W, _ = synth.gemv_operands(M, K, 1, seed=2)
    for k in (0, 13, K - 1):
        x = np.zeros(K)
        x[k] = 1.0
        r = oracle.gemv(W, synth.to_bits(x, "bf16"), M, K, 1)
        assert np.array_equal(r.bits, W.reshape(M, K)[:, k])


def test_gemv_equals_gemm_with_one_row():
    # y[1, M] = x[1, K] W^T is the column-major GEMM with A = x (1 x K),
    # B(k, j) = W[j*K + k] (W row-major is B column-major), C = y.
    M, K = 30, 70
    W, X = synth.gemv_operands(M, K, 1, seed=4)
    g = oracle.gemv(W, X, M, K, 1)
    c = oracle.gemm(X, W, 1, M, K, "bf16")
    assert np.array_equal(g.bits, c.bits)


# ---- grouped tile ordering -------------------------------------------------------

def test_grouped_tile_hand_worked_example():
    rows = np.loadtxt(os.path.join(HERE, "golden", "grouped_tile_5x3_g2.txt"), dtype=np.int64)
    table = oracle.grouped_order(5, 3, 2)
    for pid, pm, pn in rows:
        assert oracle.grouped_tile(int(pid), 5, 3, 2) == (pm, pn)
        assert table[pid] == (pm, pn)


def test_grouped_tile_one_group_is_column_major():
    # GROUP_M >= num_pid_m: one group holding every tile row, so the ordering
    # walks the grid column by column (pid -> (pid % rows, pid // rows))
    for npm, npn, gm in ((5, 3, 5), (5, 3, 8), (1, 4, 2)):
        assert oracle.grouped_order(npm, npn, gm) == [(p % npm, p // npm) for p in range(npm * npn)]


@pytest.mark.parametrize("group_m", [1, 2, 3, 4, 8, 16])
def test_grouped_tile_bijection(group_m):
    for npm in (1, 2, 5, 8, 13):
        for npn in (1, 3, 7, 16):
            seen = {oracle.grouped_tile(p, npm, npn, group_m) for p in range(npm * npn)}
            assert seen == {(i, j) for i in range(npm) for j in range(npn)}


def test_grouped_tile_group1_is_column_order():
    # GROUP_M = 1: each group is one tile row, walked along n.
    assert [oracle.grouped_tile(p, 3, 4, 1) for p in range(5)] == \
        [(0, 0), (0, 1), (0, 2), (0, 3), (1, 0)]
