"""GPU parity of gemm_tn_* (A supplied k-major: A(m,k) = At[k + m*K]) through
the C ABI against the CPU oracle, which takes the same matrix column-major:
every element at small sizes, K tails inside a 64-k stage, ragged M and N,
bit-identical agreement with gemm_ex on the same tile (same MFMA order), and
the DCU page's Y = X W^T in its own row-major layout for a batch of tokens,
and the decode tiles (14, 15, 18, 19) at their token blocks and ragged edges."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_parity, gemm_gpu, gemm_tn_gpu, gemv_gpu, kmajor_to_colmajor

pytestmark = pytest.mark.gpu

FMTS = ["f16", "bf16"]
TN_TILES = [0, 7, 8, 9, 10, 11, 12, 13, 20]


def _tn_case(M, N, K, fmt, seed, tile=0, dist=("normal", 1.0, 1.0)):
    rng_seed = seed
    At, B = synth.gemm_operands(M, N, K, fmt, dist, rng_seed)   # At drawn as M*K values
    got, guards, unchanged = gemm_tn_gpu(At, B, M, N, K, fmt, tile=tile)
    assert guards, "write outside C for %s" % ((M, N, K, fmt, tile),)
    assert unchanged, "inputs modified"
    ref = oracle.gemm(kmajor_to_colmajor(At, M, K), B, M, N, K, fmt)
    assert_parity(got, ref, fmt, "tn %s tile %d" % ((M, N, K, fmt), tile))
    return At, B, got


@pytest.mark.parametrize("tile", TN_TILES)
@pytest.mark.parametrize("fmt", FMTS)
def test_tn_each_tile_ragged(tile, fmt):
    print("case tn tile", tile, fmt, flush=True)
    _tn_case(520, 600, 200, fmt, seed=800 + tile, tile=tile)


@pytest.mark.parametrize("fmt", FMTS)
def test_tn_small_tile_eight_waves(fmt):
    # tile 20 with a k-major A where K is split over 8 waves (at most 256
    # output tiles and K >= 1024): K tails inside a 32-k step, more steps than
    # waves, ragged M and N
    for i, (M, N, K) in enumerate([(300, 200, 1032), (64, 64, 4104), (31, 129, 2048), (513, 40, 1024)]):
        print("case tn small tile 8 waves", (M, N, K), fmt, flush=True)
        _tn_case(M, N, K, fmt, seed=1700 + i, tile=20)


@pytest.mark.parametrize("tile", [7, 9, 10, 11, 12, 13, 20])
def test_tn_short_and_ragged_k(tile):
    for i, K in enumerate([8, 32, 40, 64, 72, 96, 136, 264, 520]):
        fmt = FMTS[i % 2]
        print("case tn tile", tile, "K", K, fmt, flush=True)
        _tn_case(300, 264, K, fmt, seed=900 + K, tile=tile)


@pytest.mark.parametrize("tile", [0, 7, 9, 10, 11, 13])
def test_tn_4byte_rows_and_k_tail(tile):
    # K = 2, 4, 6 mod 8: rows of At and B start at 4-byte offsets, the k loop
    # stops at a multiple of 8 and the last k are added after it
    for i, (M, N, K) in enumerate([(300, 264, 202), (130, 70, 100), (264, 300, 1038)]):
        fmt = FMTS[i % 2]
        print("case tn 4-byte rows", tile, (M, N, K), fmt, flush=True)
        _tn_case(M, N, K, fmt, seed=1300 + K + tile, tile=tile)


def test_tn_k_tail_keeps_rows_apart():
    # an infinity at the start of At's row 7 must not reach row 6 through
    # the last 16-byte piece of row 6 (K = 4 mod 8)
    M, N, K = 264, 40, 100
    at = np.ones(M * K)
    at[7 * K] = np.inf
    b = np.ones(K * N)
    for fmt in FMTS:
        At, B = synth.to_bits(at, fmt), synth.to_bits(b, fmt)
        for tile in (0, 9, 10):
            print("case tn k tail non-finite", fmt, tile, flush=True)
            got, _, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=tile)
            ref = oracle.gemm(kmajor_to_colmajor(At, M, K), B, M, N, K, fmt)
            assert_parity(got, ref, fmt, "tn k tail %s tile %d" % (fmt, tile))


def test_tn_small_and_odd_shapes():
    for (M, N, K) in [(1, 1, 8), (17, 5, 16), (255, 257, 64), (257, 31, 128), (64, 1000, 24)]:
        for fmt in FMTS:
            print("case tn", M, N, K, fmt, flush=True)
            _tn_case(M, N, K, fmt, seed=M + N + K)


def test_tn_matches_column_major_path_bit_for_bit():
    # same tile, same MFMA order over k: the two layouts of A must give the
    # same bits
    M, N, K = 1024, 768, 1000
    for fmt in FMTS:
        At, B = synth.gemm_operands(M, N, K, fmt, ("uniform", 1.0, 1.0), seed=31)
        A = kmajor_to_colmajor(At, M, K)
        for tile in (7, 8, 10, 11, 12, 13, 20):
            print("case bitwise tile", tile, fmt, flush=True)
            tn, _, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=tile)
            cm, _, _ = gemm_gpu(A, B, M, N, K, fmt, tile=tile)
            assert np.array_equal(tn, cm), "tile %d %s" % (tile, fmt)


def test_tn_small_integers_exact():
    rng = np.random.default_rng(17)
    M, N, K = 520, 392, 128
    for fmt in FMTS:
        At = synth.to_bits(synth.small_ints(rng, M * K, -3, 3), fmt)
        B = synth.to_bits(synth.small_ints(rng, K * N, -3, 3), fmt)
        want = oracle.gemm(kmajor_to_colmajor(At, M, K), B, M, N, K, fmt).bits
        for tile in TN_TILES:
            got, _, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=tile)
            assert np.array_equal(got, want), (tile, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_skinny_tile_every_token_count_and_ragged_edges(fmt):
    # tile 14 (W straight into 4x4x4 MFMA registers, 128-wide k chunks): token
    # counts across the 4-slot groups, rows off the 8-row wave blocks, K tails
    # inside a chunk and K shorter than one chunk
    for (M, N, K) in [(100, 1, 64), (37, 3, 40), (64, 5, 520), (300, 8, 264), (260, 7, 136),
                      (96, 6, 8), (1000, 8, 1000), (33, 4, 24), (7, 2, 128), (9, 8, 5120)]:
        print("case skinny", M, N, K, fmt, flush=True)
        _tn_case(M, N, K, fmt, seed=1000 + M + N + K, tile=14)


def test_skinny_matches_exact_integers():
    rng = np.random.default_rng(23)
    M, N, K = 520, 7, 1024
    for fmt in FMTS:
        At = synth.to_bits(synth.small_ints(rng, M * K, -3, 3), fmt)
        B = synth.to_bits(synth.small_ints(rng, K * N, -3, 3), fmt)
        want = oracle.gemm(kmajor_to_colmajor(At, M, K), B, M, N, K, fmt).bits
        got, _, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=14)
        assert np.array_equal(got, want), fmt


@pytest.mark.parametrize("fmt", FMTS)
def test_batch_tile_token_blocks_and_ragged_edges(fmt):
    # tile 15 (W straight into 16x16x32 MFMA registers, the token block of B
    # staged in LDS, 128-wide k chunks, chunk count padded to a multiple of
    # 4): every token-block width (16, 32, 64, 128) with ragged token counts,
    # rows off the 64-row workgroup block, K tails inside a chunk, K shorter
    # than one chunk, padded and unpadded chunk counts
    for (M, N, K) in [(100, 9, 64), (37, 16, 40), (64, 17, 520), (300, 32, 264), (260, 33, 136),
                      (96, 64, 8), (1000, 65, 1000), (33, 100, 24), (130, 128, 1160),
                      (9, 128, 5120), (2051, 40, 5120), (65, 1, 128)]:
        print("case batch", M, N, K, fmt, flush=True)
        _tn_case(M, N, K, fmt, seed=2000 + M + N + K, tile=15)


def test_batch_matches_exact_integers():
    rng = np.random.default_rng(29)
    M, N, K = 520, 77, 1032
    for fmt in FMTS:
        At = synth.to_bits(synth.small_ints(rng, M * K, -3, 3), fmt)
        B = synth.to_bits(synth.small_ints(rng, K * N, -3, 3), fmt)
        want = oracle.gemm(kmajor_to_colmajor(At, M, K), B, M, N, K, fmt).bits
        got, _, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=15)
        assert np.array_equal(got, want), fmt


@pytest.mark.parametrize("fmt", FMTS)
def test_batch_rows_tile_token_blocks_and_ragged_edges(fmt):
    # tile 18 (W's rows cut evenly over the workgroups, R = ceil(M / 256)
    # rounded up to 8 and capped at 144, 9 waves of 16 rows; 64-wide k
    # chunks, 2 to 8 in flight and the chunk count padded to that): every
    # token-block width (16 .. 256) with ragged token counts, workgroups of 8
    # rows (one wave, half live), of a few waves and of all 9, more than one
    # workgroup per CU (M > 36864), ragged last workgroups, K tails inside a
    # chunk, K shorter than one chunk
    for (M, N, K) in [(100, 2, 64), (37, 17, 40), (2051, 33, 520), (300, 64, 264), (20000, 65, 136),
                      (36000, 128, 72), (40000, 129, 64), (1000, 256, 200), (9, 200, 5120),
                      (2051, 1, 5120), (130, 255, 1160), (16400, 16, 8), (36871, 3, 584)]:
        print("case batch rows", M, N, K, fmt, flush=True)
        _tn_case(M, N, K, fmt, seed=3000 + M + N + K, tile=18)


def test_batch_rows_matches_exact_integers():
    rng = np.random.default_rng(31)
    for M, N, K in ((520, 77, 1032), (4100, 250, 200), (33000, 8, 648)):
        for fmt in FMTS:
            print("case batch rows exact", M, N, K, fmt, flush=True)
            At = synth.to_bits(synth.small_ints(rng, M * K, -3, 3), fmt)
            B = synth.to_bits(synth.small_ints(rng, K * N, -3, 3), fmt)
            want = oracle.gemm(kmajor_to_colmajor(At, M, K), B, M, N, K, fmt).bits
            got, _, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=18)
            assert np.array_equal(got, want), (M, N, K, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_batch_wide_tile_token_blocks_and_ragged_edges(fmt):
    # tile 19 (the same rows per workgroup as tile 18; 8 waves in row groups
    # of 5 and 4 tiles times four token groups; 64-wide k chunks loaded
    # straight into a 4-stage (128 tokens) or 3-stage (256 tokens) LDS ring):
    # both token blocks with ragged token counts, workgroups of 8 rows (most
    # row tiles empty), of a few tiles and of all 9, more than one workgroup
    # per CU (M > 36864), ragged last workgroups, K tails inside a chunk, K
    # shorter than one chunk and shorter than the ring
    for (M, N, K) in [(100, 65, 64), (37, 1, 40), (2051, 128, 520), (300, 129, 264), (20000, 200, 136),
                      (36000, 256, 72), (40000, 100, 64), (9, 256, 5120), (130, 255, 1160),
                      (16400, 16, 8), (36871, 250, 584), (34816, 130, 128)]:
        print("case batch wide", M, N, K, fmt, flush=True)
        _tn_case(M, N, K, fmt, seed=4000 + M + N + K, tile=19)


def test_batch_wide_matches_exact_integers():
    rng = np.random.default_rng(37)
    for M, N, K in ((520, 77, 1032), (4100, 250, 200), (33000, 130, 648)):
        for fmt in FMTS:
            print("case batch wide exact", M, N, K, fmt, flush=True)
            At = synth.to_bits(synth.small_ints(rng, M * K, -3, 3), fmt)
            B = synth.to_bits(synth.small_ints(rng, K * N, -3, 3), fmt)
            want = oracle.gemm(kmajor_to_colmajor(At, M, K), B, M, N, K, fmt).bits
            got, _, _ = gemm_tn_gpu(At, B, M, N, K, fmt, tile=19)
            assert np.array_equal(got, want), (M, N, K, fmt)


def test_row_balanced_tiles_agree_bit_for_bit():
    # tiles 18 and 19 add the same 32-k MFMA steps in the same order into
    # FP32, so their outputs agree bit for bit
    M, N, K = 34816, 200, 1024
    At, B = synth.gemm_operands(M, N, K, "bf16", ("normal", 0.02, 1.0), 77)
    g18, _, _ = gemm_tn_gpu(At, B, M, N, K, "bf16", tile=18)
    g19, _, _ = gemm_tn_gpu(At, B, M, N, K, "bf16", tile=19)
    assert np.array_equal(g18, g19)


def test_tn_is_the_decode_product_for_a_token_batch():
    # gemm_tn(At = W, B = X, C = Y) is Y = X W^T with W, X, Y row-major: the
    # GEMV's layout.  16 tokens of the decode shape: sampled entries against
    # the oracle GEMV, and agreement with gemv_bf16 within the tolerance.
    M, K, n = 34816, 5120, 16
    W, X = synth.gemv_operands(M, K, n, seed=3)
    print("case tn decode batch", M, K, n, flush=True)
    got, guards, unchanged = gemm_tn_gpu(W, X, M, n, K, "bf16")
    assert guards and unchanged
    idx = synth.sample_indices(M, n, 3, 2048)
    ref = oracle.gemm_sampled(kmajor_to_colmajor(W, M, K), X, M, n, K, idx, "bf16")
    assert_parity(got[idx], ref, "bf16", "tn decode batch sampled")
    gv, _, _ = gemv_gpu(W, X, M, K, n)
    refv = oracle.gemv(W, X, M, K, n, "bf16")
    assert_parity(gv, refv, "bf16", "gemv decode batch")
    # both are within the oracle's bound of the same exact value; directly,
    # they differ by at most twice the bound
    a = synth.from_bits(got, "bf16").astype(np.float64)
    b = synth.from_bits(gv, "bf16").astype(np.float64)
    bound = 2 * (2e-3 * refv.sabs + oracle.ulp_out(refv.exact, "bf16"))
    assert np.all(np.abs(a - b) <= bound)
