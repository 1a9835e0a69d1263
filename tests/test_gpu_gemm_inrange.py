"""The full-line tiles (9-13, 16 and 17) load through global addresses
when every load of the launch lies inside A and B (16-byte rows, M and N
multiples of the tile, K a multiple of 64) and through range-checked buffer
loads otherwise.  Both kinds of load must give the same bits: each product
computed in range is compared with the same rows or columns of a product one
ragged block larger (other loads; the extra rows and columns hold other
data), and with the oracle.

The tiles with 64-row wave tiles also pass C through LDS and store whole
128-byte lines when C lies on a 16-byte boundary and M is a multiple of 8
(in range or ragged); with C moved by 8 bytes they store each output
directly.  Both must give the same bits."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_parity, gemm_gpu, gemm_tn_gpu, gemm_tn_q_gpu, kmajor_to_colmajor

pytestmark = pytest.mark.gpu

FMTS = ["f16", "bf16"]


def _extra(rng, n, like):
    return rng.integers(0, 1 << 14, size=n).astype(like.dtype)


@pytest.mark.parametrize("tile", [16, 10, 9, 12, 11, 13])
@pytest.mark.parametrize("fmt", FMTS)
def test_column_major_in_range_equals_ragged(tile, fmt):
    M, N, K = 512, 512, 1024
    A, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), 2100 + tile)
    rng = np.random.default_rng(7)
    print("case in-range", tile, fmt, flush=True)
    c, guards, _ = gemm_gpu(A, B, M, N, K, fmt, tile=tile)
    assert guards
    assert_parity(c, oracle.gemm(A, B, M, N, K, fmt), fmt, "in range tile %d" % tile)
    # 8 more rows of A (A(m,k) = A[m + k*M]): the first 512 rows of C agree
    A2 = np.concatenate([A.reshape(K, M), _extra(rng, K * 8, A).reshape(K, 8)], axis=1).reshape(-1)
    c2, _, _ = gemm_gpu(A2, B, M + 8, N, K, fmt, tile=tile)
    assert np.array_equal(c2.reshape(N, M + 8)[:, :M], c.reshape(N, M)), "ragged M"
    # 8 more columns of B: the first 512 columns of C agree
    B2 = np.concatenate([B, _extra(rng, K * 8, B)])
    c3, _, _ = gemm_gpu(A, B2, M, N + 8, K, fmt, tile=tile)
    assert np.array_equal(c3[:M * N], c), "ragged N"


@pytest.mark.parametrize("tile", [10, 9, 12, 13])
@pytest.mark.parametrize("fmt", FMTS)
def test_k_major_in_range_equals_ragged(tile, fmt):
    M, N, K = 512, 512, 1024
    At, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), 2200)
    rng = np.random.default_rng(8)
    print("case in-range tn", fmt, flush=True)
    c, guards, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=tile)
    assert guards
    assert_parity(c, oracle.gemm(kmajor_to_colmajor(At, M, K), B, M, N, K, fmt), fmt, "in range tn tile %d" % tile)
    # 8 more rows of At (A(m,k) = At[k + m*K])
    At2 = np.concatenate([At, _extra(rng, K * 8, At)])
    c2, _, _ = gemm_tn_gpu(At2, B, M + 8, N, K, fmt, tile=tile)
    assert np.array_equal(c2.reshape(N, M + 8)[:, :M], c.reshape(N, M)), "ragged M"


@pytest.mark.parametrize("fmt,tile", [("f8e4m3", 17), ("f8e5m2", 17), ("i8", 10), ("i8", 9), ("f8e4m3", 13)])
def test_8bit_in_range_equals_ragged(fmt, tile):
    M, N, K = 512, 256, 1024
    At, B = synth.q8_operands(M, N, K, fmt, seed=2300)
    print("case in-range q8", fmt, tile, flush=True)
    c, guards, _ = gemm_tn_q_gpu(At, B, M, N, K, fmt, 0.5, tile)
    assert guards
    ref = oracle.gemm_tn_q(At, B, M, N, K, fmt, 0.5)
    if fmt == "i8":
        assert np.array_equal(c, ref.bits)
    else:
        ok, rep = oracle.check(c, ref, "bf16")
        assert ok, rep
    At2, _ = synth.q8_operands(M + 16, N, K, fmt, seed=2301)
    At2 = np.concatenate([np.asarray(At).reshape(-1), np.asarray(At2).reshape(-1)[M * K:]])
    c2, _, _ = gemm_tn_q_gpu(At2, B, M + 16, N, K, fmt, 0.5, tile)
    assert np.array_equal(c2.reshape(N, M + 16)[:, :M], c.reshape(N, M)), "ragged M"


STAGED_SHAPES = [(512, 512, 1024), (520, 264, 1024), (1032, 136, 512), (516, 260, 256)]


@pytest.mark.parametrize("tile", [16, 10, 9, 13])
@pytest.mark.parametrize("shape", STAGED_SHAPES)
def test_column_major_staged_c_equals_direct(tile, shape):
    M, N, K = shape
    fmt = "bf16" if tile % 2 else "f16"
    A, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), 2400 + tile)
    print("case staged C", tile, shape, flush=True)
    c, guards, _ = gemm_gpu(A, B, M, N, K, fmt, tile=tile)
    c2, guards2, _ = gemm_gpu(A, B, M, N, K, fmt, tile=tile, c_shift=4)
    assert guards and guards2
    assert np.array_equal(c, c2), "staged and direct stores differ"
    assert_parity(c, oracle.gemm(A, B, M, N, K, fmt), fmt, "staged C tile %d %s" % (tile, shape))


@pytest.mark.parametrize("tile", [10, 9, 13])
@pytest.mark.parametrize("shape", STAGED_SHAPES[:3])
def test_k_major_staged_c_equals_direct(tile, shape):
    M, N, K = shape
    fmt = "bf16"
    At, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), 2500 + tile)
    print("case staged C tn", tile, shape, flush=True)
    c, guards, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=tile)
    c2, guards2, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=tile, c_shift=4)
    assert guards and guards2
    assert np.array_equal(c, c2), "staged and direct stores differ"
    assert_parity(c, oracle.gemm(kmajor_to_colmajor(At, M, K), B, M, N, K, fmt), fmt,
                  "staged C tn tile %d %s" % (tile, shape))


@pytest.mark.parametrize("fmt,tile", [("f8e4m3", 17), ("i8", 10), ("f8e5m2", 13)])
@pytest.mark.parametrize("shape", [(512, 256, 1024), (520, 264, 1024)])
def test_8bit_staged_c_equals_direct(fmt, tile, shape):
    M, N, K = shape
    At, B = synth.q8_operands(M, N, K, fmt, seed=2600)
    print("case staged C q8", fmt, tile, shape, flush=True)
    c, guards, _ = gemm_tn_q_gpu(At, B, M, N, K, fmt, 0.5, tile)
    c2, guards2, _ = gemm_tn_q_gpu(At, B, M, N, K, fmt, 0.5, tile, c_shift=4)
    assert guards and guards2
    assert np.array_equal(c, c2), "staged and direct stores differ"
    ref = oracle.gemm_tn_q(At, B, M, N, K, fmt, 0.5)
    if fmt == "i8":
        assert np.array_equal(c, ref.bits)
    else:
        ok, rep = oracle.check(c, ref, "bf16")
        assert ok, rep


@pytest.mark.parametrize("tile", [10, 16, 9, 13, 12, 11])
@pytest.mark.parametrize("kmajor", [False, True])
@pytest.mark.parametrize("shape", [(520, 264, 1024), (264, 600, 128), (8, 8, 64), (4000, 520, 512)])
def test_ragged_global_loads_equal_buffer_loads(tile, kmajor, shape):
    # ragged M or N, 16-byte rows, K a multiple of 64: the full-line tiles load
    # through global addresses (lanes past M or N re-reading the tile's first
    # row or column); the same A placed 8 bytes later (rows no longer 16-byte
    # aligned) takes the range-checked buffer loads.  Same bits.
    import torch
    from bf16_gemm_decode_amd import binding
    from helpers import dev, Guarded
    if tile == 16 and kmajor:
        pytest.skip("the ping-pong tile takes an m-major A only")
    M, N, K = shape
    fmt = "bf16"
    A, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), 2700 + M + N)
    print("case ragged global vs buffer", tile, kmajor, shape, flush=True)
    fn = binding.gemm_tn_ex_ptr if kmajor else binding.gemm_ex_ptr
    outs = []
    for shift in (0, 4):
        dA = dev(np.concatenate([np.zeros(shift, np.uint16), A]))
        dB = dev(B)
        C = Guarded(M * N)
        code = fn(binding.BF16, dA.data_ptr() + 2 * shift, dB.data_ptr(), C.ptr, M, N, K, tile, 0, 1)
        assert code == 0, code
        torch.cuda.synchronize()
        assert C.guards_intact()
        outs.append(C.out())
    assert np.array_equal(outs[0], outs[1]), "global and buffer loads differ"
    ref_a = kmajor_to_colmajor(A, M, K) if kmajor else A
    assert_parity(outs[0], oracle.gemm(ref_a, B, M, N, K, fmt), fmt, "ragged %s tile %d" % (shape, tile))


@pytest.mark.parametrize("fmt,tile", [("i8", 10), ("f8e4m3", 17), ("f8e5m2", 17)])
@pytest.mark.parametrize("shape", [(520, 264, 1024), (4000, 136, 512), (8, 8, 128)])
def test_8bit_ragged_global_loads_match_oracle(fmt, tile, shape):
    # 8-bit operands always have 16-byte rows, so ragged M or N with K a
    # multiple of 128 takes the global loads with the edge lanes re-reading
    # the tile's first row or column: INT8 must equal the oracle bit for
    # bit, FP8 within its bound; C's guard bands stay intact.  (The
    # in-range-against-ragged test above compares such launches with
    # in-range ones bit for bit.)
    M, N, K = shape
    At, B = synth.q8_operands(M, N, K, fmt, seed=2800 + M)
    print("case 8-bit ragged global", fmt, tile, shape, flush=True)
    c, guards, unchanged = gemm_tn_q_gpu(At, B, M, N, K, fmt, 0.5, tile)
    assert guards and unchanged
    ref = oracle.gemm_tn_q(At, B, M, N, K, fmt, 0.5)
    if fmt == "i8":
        assert np.array_equal(c, ref.bits)
    else:
        ok, rep = oracle.check(c, ref, "bf16")
        assert ok, rep
