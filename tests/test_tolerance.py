"""The acceptance rule |C - C_ref| <= 2e-3 * S_abs + ulp_out(C_ref): its
closed-form justification, a positive control (a CPU FP32 sum in an
arbitrary order passes) and negative controls (a planted error fails)."""
import numpy as np
import pytest

import oracle
import synth


def gamma(K, u=2.0 ** -24):
    """Higham, Accuracy and Stability of Numerical Algorithms, section 3.1:
    the FP32 summation error bound gamma_K = K u / (1 - K u)."""
    return K * u / (1 - K * u)


@pytest.mark.parametrize("K", [512, 4100, 5120, 16384])
def test_tolerance_covers_any_fp32_order(K):
    assert 2e-3 >= 2 * gamma(K)


def test_gamma_values():
    assert abs(gamma(16384) - 9.77e-4) < 1e-6
    assert abs(gamma(5120) - 3.05e-4) < 1e-6
    assert abs(gamma(4100) - 2.44e-4) < 1e-6


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_ulp_out_values(fmt):
    mb = 10 if fmt == "f16" else 7
    emin = -14 if fmt == "f16" else -126
    assert oracle.ulp_out([1.0], fmt)[0] == 2.0 ** -mb
    assert oracle.ulp_out([1.5], fmt)[0] == 2.0 ** -mb
    assert oracle.ulp_out([-3.0], fmt)[0] == 2.0 ** (1 - mb)
    assert oracle.ulp_out([0.0], fmt)[0] == 2.0 ** (emin - mb)
    assert oracle.ulp_out([2.0 ** (emin - 3)], fmt)[0] == 2.0 ** (emin - mb)


def _fp32_sum_colmajor(A, B, M, N, K, fmt, reverse):
    a = synth.from_bits(A, fmt).reshape(K, M).T.astype(np.float32)
    b = synth.from_bits(B, fmt).reshape(N, K).T.astype(np.float32)
    acc = np.zeros((M, N), np.float32)
    ks = range(K - 1, -1, -1) if reverse else range(K)
    for k in ks:
        acc += np.outer(a[:, k], b[k, :]).astype(np.float32)
    return synth.to_bits(acc.T.ravel().astype(np.float64), fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("reverse", [False, True])
def test_positive_control_fp32_sum_passes(fmt, reverse):
    M, N, K = 24, 20, 300
    A, B = synth.gemm_operands(M, N, K, fmt, ("uniform", 1.0, 1.0), seed=21)
    ref = oracle.gemm(A, B, M, N, K, fmt)
    got = _fp32_sum_colmajor(A, B, M, N, K, fmt, reverse)
    ok, rep = oracle.check(got, ref, fmt)
    assert ok, rep


def test_negative_control_perturbation_fails():
    M, N, K = 16, 16, 200
    A, B = synth.gemm_operands(M, N, K, "f16", ("uniform", 1.0, 1.0), seed=22)
    ref = oracle.gemm(A, B, M, N, K, "f16")
    v = oracle.decode(ref.bits, "f16")
    i = 37
    v[i] += 1e-2 * ref.sabs[i]
    ok, rep = oracle.check(synth.to_bits(v, "f16"), ref, "f16")
    assert not ok and rep["first_bad"] == [i]


def test_negative_control_transposed_result_fails():
    M, N, K = 12, 12, 64
    A, B = synth.gemm_operands(M, N, K, "bf16", ("normal", 1.0, 1.0), seed=23)
    ref = oracle.gemm(A, B, M, N, K, "bf16")
    wrong = ref.bits.reshape(N, M).T.ravel()       # C^T stored as C
    ok, _ = oracle.check(wrong, ref, "bf16")
    assert not ok


def test_negative_control_truncating_rounding_fails_tie_case():
    # exact sum 1 + 3*2^-11 is a binary16 tie; truncation gives 1 + 2^-10,
    # which is within one ulp -- the tolerance alone cannot see it, so the
    # rounding mode is pinned by the bit-exact test instead.
    A = synth.to_bits([1.0, 3 * 2.0 ** -11], "f16")
    B = synth.to_bits([1.0, 1.0], "f16")
    ref = oracle.gemm(A, B, 1, 1, 2, "f16")
    assert int(ref.bits[0]) == 0x3C02
    assert int(ref.bits[0]) != 0x3C01


def test_nonfinite_class_rule():
    ref = oracle.GemmResult(np.array([0x7C00, 0x7E00, 0x3C00], np.uint16), None,
                            np.array([1.0, 1.0, 1.0]), 0)
    ok, _ = oracle.check(np.array([0x7C00, 0x7E01, 0x3C00], np.uint16), ref, "f16")
    assert ok
    ok, _ = oracle.check(np.array([0xFC00, 0x7E00, 0x3C00], np.uint16), ref, "f16")
    assert not ok
    ok, _ = oracle.check(np.array([0x7C00, 0x7C00, 0x3C00], np.uint16), ref, "f16")
    assert not ok
