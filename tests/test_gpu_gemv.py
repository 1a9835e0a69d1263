"""GPU parity of gemv_bf16 (through the C ABI) against the CPU oracle:
every element of the 34816 x 5120 decode shape at n = 1, 4, 16, sampled rows
(all tokens) at n = 2, 64, 128, 256, ragged shapes and token counts on every
automatic route, the one-hot exact case, agreement with the GEMM at n = 1,
and bit-identical results across rows_per_block."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_parity, gemm_gpu, gemv_gpu

pytestmark = pytest.mark.gpu


def _case(M, K, n, seed, rows_per_block=0):
    W, X = synth.gemv_operands(M, K, n, seed=seed)
    got, guards, unchanged = gemv_gpu(W, X, M, K, n, rows_per_block)
    assert guards, "write outside Y"
    assert unchanged, "inputs modified"
    ref = oracle.gemv(W, X, M, K, n)
    assert ref.macs == n * M * K
    return got, assert_parity(got, ref, "bf16", "gemv %s" % ((M, K, n, rows_per_block),))


def test_small_shapes():
    for (M, K, n) in [(1, 8, 1), (2, 512, 1), (8, 520, 2), (33, 1000, 3), (64, 5120, 1)]:
        print("case", M, K, n, flush=True)
        _case(M, K, n, seed=M + K + n)


def test_ragged_shapes_and_token_counts():
    # with K a multiple of 8 and M < 16384: 1 and 2 tokens the vector
    # kernel, 3 and 4 the 4x4x4 MFMA kernel, 5..32 the batch kernel, 33..128
    # the row-balanced kernel, more the full-line GEMM tile; K % 8 != 0
    # always the vector kernel (gemv_route reports each choice)
    from bf16_gemm_decode_amd import binding
    seen = set()
    for (M, K) in [(7, 13), (100, 512), (129, 1031), (1000, 5120), (77, 5128), (31, 4096)]:
        for n in (1, 2, 3, 4, 5, 8, 9, 16, 17, 33, 130):
            seen.add(binding.gemv_route(1 << 20, 1 << 30, 1 << 40, M, K, n)[1])
            print("case", M, K, n, flush=True)
            _case(M, K, n, seed=M * 7 + K + n)
    assert seen == {1, 9, 14, 15, 18}, seen


@pytest.mark.parametrize("n", [1, 4, 16])
def test_decode_shape_full(n):
    w = synth.WORKLOADS["gemv_34816x5120_bf16"]
    print("case decode n", n, flush=True)
    _, rep = _case(w["M"], w["K"], n, seed=w["seed"])
    print("n", n, "max err/bound", rep["max_ratio"])


@pytest.mark.parametrize("n,route", [(2, 18), (64, 18), (128, 19), (256, 19)])
def test_decode_shape_sampled_rows(n, route):
    # the row-balanced kernels' decode shape (136 rows per workgroup) at more
    # tokens than the full oracle finishes quickly: 512 random rows, the rows
    # around the first workgroup boundaries and the last workgroup, every
    # token, against the oracle GEMV of those rows
    from bf16_gemm_decode_amd import binding
    w = synth.WORKLOADS["gemv_34816x5120_bf16"]
    M, K = w["M"], w["K"]
    assert binding.gemv_route(1 << 20, 1 << 30, 1 << 40, M, K, n)[1] == route
    W, X = synth.gemv_operands(M, K, n, seed=w["seed"])
    got, guards, unchanged = gemv_gpu(W, X, M, K, n)
    assert guards and unchanged
    rows = np.unique(np.concatenate([np.random.default_rng(n).choice(M, 512, replace=False),
                                     np.arange(120, 152), np.arange(264, 280), np.arange(M - 144, M)]))
    ref = oracle.gemv(W.reshape(M, K)[rows].ravel(), X, rows.size, K, n)
    print("case decode sampled n", n, "rows", rows.size, flush=True)
    rep = assert_parity(got.reshape(n, M)[:, rows].ravel(), ref, "bf16", "decode sampled n=%d" % n)
    print("n", n, "max err/bound", rep["max_ratio"])


@pytest.mark.parametrize("n", [1, 4, 16])
def test_rows_per_block_bit_identical(n):
    M, K = 4099, 5120
    W, X = synth.gemv_operands(M, K, n, seed=8)
    outs = []
    for r in (2, 4, 8, 16, 32):
        got, guards, _ = gemv_gpu(W, X, M, K, n, r)
        assert guards
        outs.append(got)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert_parity(outs[0], oracle.gemv(W, X, M, K, n), "bf16", "rows_per_block")


def test_every_route_against_the_vector_kernel():
    # the automatic routes at M = 2051 (the 4x4x4 MFMA kernel for 3 and 4
    # tokens, the batch kernel for 5..32, the row-balanced kernel for
    # 33..128, the GEMM tile beyond) and the vector kernel (rows_per_block
    # given) both meet the oracle's bound at the decode width
    M, K = 2051, 5120
    for n in (3, 6, 8, 12, 40, 100, 129):
        print("case route n", n, flush=True)
        W, X = synth.gemv_operands(M, K, n, seed=40 + n)
        ref = oracle.gemv(W, X, M, K, n)
        auto, g1, _ = gemv_gpu(W, X, M, K, n, 0)
        vec, g2, _ = gemv_gpu(W, X, M, K, n, 2)
        assert g1 and g2
        assert_parity(auto, ref, "bf16", "automatic n=%d" % n)
        assert_parity(vec, ref, "bf16", "vector n=%d" % n)


def test_one_hot_selects_column_exactly():
    M, K = 34816, 5120
    W, _ = synth.gemv_operands(M, K, 1, seed=3)
    for k in (0, 1234, K - 1):
        x = np.zeros(K)
        x[k] = 1.0
        got, _, _ = gemv_gpu(W, synth.to_bits(x, "bf16"), M, K, 1)
        assert np.array_equal(got, W.reshape(M, K)[:, k])


def test_matches_gemm_with_one_row():
    # y = x W^T is the column-major GEMM with A = x (1 x K) and B = W read as
    # K x M column-major; both GPU paths must pass against the one oracle.
    M, K = 34816, 5120
    W, X = synth.gemv_operands(M, K, 1, seed=3)
    g, _, _ = gemv_gpu(W, X, M, K, 1)
    c, _, _ = gemm_gpu(X, W, 1, M, K, "bf16")
    ref = oracle.gemv(W, X, M, K, 1)
    assert_parity(g, ref, "bf16", "gemv")
    assert_parity(c, ref, "bf16", "gemm M=1")
    diff = np.abs(oracle.decode(g, "bf16") - oracle.decode(c, "bf16"))
    assert np.all(diff <= 2 * (2e-3 * ref.sabs + oracle.ulp_out(oracle.decode(ref.bits, "bf16"), "bf16")))


def test_k_zero_writes_zero():
    got, guards, _ = gemv_gpu(np.zeros(0, np.uint16), np.zeros(0, np.uint16), 50, 0, 3)
    assert guards and np.all(got == 0)


def test_hbm_probe_checksum():
    # every word read exactly once: whole 8 KiB chunks, and a ragged tail
    import torch
    from bf16_gemm_decode_amd import hbm_read, hbm_read_sink_words
    for n in (1 << 24, (1 << 22) + 12, 4):
        print("case probe words", n, flush=True)
        buf = torch.randint(0, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda")
        sink = torch.zeros(hbm_read_sink_words(), dtype=torch.int32, device="cuda")
        hbm_read(buf, sink)
        torch.cuda.synchronize()
        x = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
        assert x == want, n
