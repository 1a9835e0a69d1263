"""GPU parity of gemm_f16 / gemm_bf16 (through the C ABI) against the CPU
oracle: every element at small sizes and for the 512^3 workload, 4096 seeded
samples plus full tail strips at the large sizes, bit-exact classes (integer
data, identity and permutation operands, rounding ties), guard bands around
C, inputs unchanged, and bit-identical results across tile orderings."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_parity, dev, gemm_gpu, Guarded, host

pytestmark = pytest.mark.gpu

FMTS = ["f16", "bf16"]


def _full_case(M, N, K, fmt, seed, dist=("normal", 1.0, 1.0), **cfg):
    A, B = synth.gemm_operands(M, N, K, fmt, dist, seed)
    got, guards, unchanged = gemm_gpu(A, B, M, N, K, fmt, **cfg)
    assert guards, "write outside C for %s" % ((M, N, K, fmt, cfg),)
    assert unchanged, "inputs modified"
    ref = oracle.gemm(A, B, M, N, K, fmt)
    assert ref.macs == M * N * K
    assert_parity(got, ref, fmt, "%s %s" % ((M, N, K, fmt), cfg))
    return got


@pytest.mark.parametrize("fmt", FMTS)
def test_tiny_and_single_tile(fmt):
    for (M, N, K) in [(1, 1, 1), (16, 16, 32), (64, 64, 64), (128, 128, 64), (17, 5, 3)]:
        print("case", M, N, K, fmt, flush=True)
        _full_case(M, N, K, fmt, seed=M + N + K)


SWEEP = [1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


@pytest.mark.parametrize("fmt", FMTS)
def test_shape_sweep_each_dimension(fmt):
    # every sweep value in each dimension, the other two fixed at ragged sizes
    cases = [(v, 65, 129) for v in SWEEP] + [(129, v, 65) for v in SWEEP] + \
            [(65, 129, v) for v in SWEEP]
    for i, (M, N, K) in enumerate(cases):
        print("case", M, N, K, fmt, flush=True)
        _full_case(M, N, K, fmt, seed=100 + i)


def test_shape_sweep_random_triples():
    rng = np.random.default_rng(42)
    for i in range(24):
        M, N, K = (int(v) for v in rng.choice(SWEEP, 3))
        fmt = FMTS[i % 2]
        print("case", M, N, K, fmt, flush=True)
        _full_case(M, N, K, fmt, seed=200 + i)


ALL_TILES = list(range(1, 14)) + [16, 20]
FULL_LINE_TILES = [7, 8, 9, 10, 11, 12, 13, 16]


@pytest.mark.parametrize("tile", ALL_TILES)
@pytest.mark.parametrize("fmt", FMTS)
def test_each_tile_config_ragged(tile, fmt):
    # M, K multiples of 8 (the 256-row tiles need 16-byte loads); N ragged,
    # several tiles in each direction, partial last tiles, K tail.
    print("case tile", tile, fmt, flush=True)
    _full_case(520, 600, 200, fmt, seed=300 + tile, tile=tile)


@pytest.mark.parametrize("tile", FULL_LINE_TILES)
def test_full_line_tiles_short_and_ragged_k(tile):
    # few sub-steps (the ring never fills: waits fall back to "all landed"),
    # odd sub-step counts (leading zero sub-step, B stage straddling k = 0),
    # K tails inside a 64-k B stage, and N past the tile edge
    for i, K in enumerate([8, 32, 40, 64, 72, 96, 136, 200, 264, 520]):
        fmt = FMTS[i % 2]
        print("case tile", tile, "K", K, fmt, flush=True)
        _full_case(264, 300, K, fmt, seed=700 + K, tile=tile)


@pytest.mark.parametrize("tile", FULL_LINE_TILES)
def test_full_line_tiles_4byte_rows(tile):
    # rows only 4-byte aligned: K = 2, 4, 6 mod 8 (B columns start at any
    # 4-byte offset; the k loop stops at a multiple of 8 and the last k are
    # added after it) and M = 2 mod 8 (A's k rows)
    for i, (M, N, K) in enumerate([(264, 300, 202), (266, 130, 100), (520, 264, 1036), (258, 70, 70)]):
        fmt = FMTS[i % 2]
        print("case tile", tile, (M, N, K), fmt, flush=True)
        _full_case(M, N, K, fmt, seed=900 + K + tile, tile=tile)


def test_small_tile_shapes_and_k():
    # tile 20 (32x32 per workgroup, K split over 4 waves, or 8 for at most
    # 256 tiles with K >= 1024; operands straight from memory, partials
    # summed in LDS): any M for an m-major A (2-byte loads), ragged N, K from
    # one 8-element piece to several thousand with tails inside a 32-k step,
    # more k steps than waves and fewer
    for i, (M, N, K) in enumerate([(513, 511, 520), (1, 1, 8), (33, 17, 40), (100, 70, 200), (31, 129, 4104),
                                   (512, 512, 512), (7, 300, 72), (250, 5, 2048), (64, 64, 1032),
                                   (300, 200, 1024)]):
        for fmt in FMTS:
            print("case small tile", (M, N, K), fmt, flush=True)
            _full_case(M, N, K, fmt, seed=1500 + i, tile=20)


def test_k_tail_keeps_columns_apart():
    # K = 4 mod 8 on the full-line tiles: the last 16-byte piece of a B
    # column would also hold the next column's first elements; an infinity
    # there must stay in its own column (and a NaN in A's last k row in its
    # own row)
    M, N, K = 264, 40, 100
    a = np.ones(M * K)
    a[7 + (K - 1) * M] = np.nan   # row 7, last k
    b = np.ones(K * N)
    b[0 + 5 * K] = np.inf         # column 5, k = 0
    for fmt in FMTS:
        A, B = synth.to_bits(a, fmt), synth.to_bits(b, fmt)
        for tile in (0, 9, 10, 13, 16):
            print("case k tail non-finite", fmt, tile, flush=True)
            got, _, _ = gemm_gpu(A, B, M, N, K, fmt, tile=tile)
            assert_parity(got, oracle.gemm(A, B, M, N, K, fmt), fmt, "k tail %s tile %d" % (fmt, tile))


def test_misaligned_vector_widths():
    # odd M and K force element loads; M, K = 2 mod 4 force 4-byte loads
    for (M, N, K) in [(33, 40, 65), (34, 40, 66), (130, 70, 258), (258, 130, 100)]:
        for fmt in FMTS:
            print("case", M, N, K, fmt, flush=True)
            _full_case(M, N, K, fmt, seed=M * N + K)


def test_workload_512_f16_full():
    w = synth.WORKLOADS["gemm_512_f16"]
    A, B = synth.workload_operands("gemm_512_f16")
    got, guards, unchanged = gemm_gpu(A, B, w["M"], w["N"], w["K"], "f16")
    assert guards and unchanged
    ref = oracle.gemm(A, B, w["M"], w["N"], w["K"], "f16")
    rep = assert_parity(got, ref, "f16", "512^3")
    print("512^3 max err/bound", rep["max_ratio"])


def _sampled_case(name, extra_strips=False):
    w = synth.WORKLOADS[name]
    M, N, K, fmt = w["M"], w["N"], w["K"], w["fmt"]
    print("generating", name, flush=True)
    A, B = synth.workload_operands(name)
    print("running", name, flush=True)
    got, guards, unchanged = gemm_gpu(A, B, M, N, K, fmt)
    assert guards and unchanged
    idx = synth.sample_indices(M, N, w["seed"])
    ref = oracle.gemm_sampled(A, B, M, N, K, idx, fmt)
    assert ref.macs == idx.size * K
    rep = assert_parity(got[idx], ref, fmt, name + " samples")
    print(name, "samples", idx.size, "max err/bound", rep["max_ratio"])
    if extra_strips:
        # every element of the last partial row block and column block of
        # the tile the automatic plan launches (256 x 256 here: 136 rows and
        # 184 columns at 5000 x 3000)
        from bf16_gemm_decode_amd import binding
        code, plan = binding.gemm_plan(binding.F16 if fmt == "f16" else binding.BF16, 1 << 20, 1 << 21,
                                       1 << 40, M, N, K)
        assert code == 0, code
        tm, tn = plan["tile_m"], plan["tile_n"]
        m_last = np.arange(M - (M % tm or tm), M)
        n_last = np.arange(N - (N % tn or tn), N)
        print(name, "tile", plan["tile"], "last blocks", m_last.size, "rows,", n_last.size, "columns", flush=True)
        rows = (m_last[:, None] + np.arange(N)[None, :] * M).ravel()
        cols = (np.arange(M)[:, None] + n_last[None, :] * M).ravel()
        strip = np.unique(np.concatenate([rows, cols]))
        ref = oracle.gemm_sampled(A, B, M, N, K, strip, fmt)
        rep = assert_parity(got[strip], ref, fmt, name + " tail strips")
        print(name, "tail strips", strip.size, "max err/bound", rep["max_ratio"])
    return A, B, got


def test_workload_ragged_5000x3000x4100_bf16():
    _sampled_case("gemm_5000x3000x4100_bf16", extra_strips=True)


def test_workload_8192x8192x16384_f16_sampled():
    _sampled_case("gemm_8192x8192x16384_f16")


def test_workload_prefill_4096x34816x5120_bf16_sampled():
    _sampled_case("prefill_4096x34816x5120_bf16")


@pytest.mark.parametrize("fmt", FMTS)
def test_integer_exact_full_size(fmt):
    # entries in {-1, 0, 1}: every FP32 partial sum is an exact integer, so any
    # correct summation order gives the same C, and the final rounding is
    # deterministic -- the GPU must match bit for bit.  Checked on 4096 oracle
    # samples and on ALL entries through exact integer checksums C r = A (B r).
    M, N, K = 8192, 8192, 16384
    rng = np.random.default_rng(7 + (fmt == "bf16"))
    # bfloat16 holds integers exactly only up to 256: sparser entries keep
    # every |C| below that (sigma = sqrt(K p) = 31 for p = 0.06)
    p = [1 / 3] * 3 if fmt == "f16" else [0.03, 0.94, 0.03]
    a = rng.choice(np.array([-1, 0, 1], np.int8), M * K, p=p)
    b = rng.choice(np.array([-1, 0, 1], np.int8), K * N, p=p)
    A, B = synth.to_bits(a.astype(np.float64), fmt), synth.to_bits(b.astype(np.float64), fmt)
    print("running integer", fmt, flush=True)
    got, guards, unchanged = gemm_gpu(A, B, M, N, K, fmt)
    assert guards and unchanged
    idx = synth.sample_indices(M, N, 77)
    ref = oracle.gemm_sampled(A, B, M, N, K, idx, fmt)
    assert np.array_equal(got[idx], ref.bits)
    C = oracle.decode(got, fmt).reshape(N, M).T            # exact small integers
    assert np.all(np.abs(C) <= (2048 if fmt == "f16" else 256)), "outside the exact range"
    am = a.reshape(K, M).T.astype(np.int64)                # A (M x K)
    bm = b.reshape(N, K).T.astype(np.int64)                # B (K x N)
    for trial in range(2):
        r = rng.integers(-3, 4, N).astype(np.int64)
        want = am @ (bm @ r)
        assert np.array_equal(C.astype(np.int64) @ r, want)
        l = rng.integers(-3, 4, M).astype(np.int64)
        assert np.array_equal(l @ C.astype(np.int64), (l @ am) @ bm)


@pytest.mark.parametrize("fmt", FMTS)
def test_small_integers_exact_every_tile(fmt):
    rng = np.random.default_rng(5)
    for tile in ALL_TILES:
        M, N, K = 520, 392, 64
        a = synth.small_ints(rng, M * K, -3, 3)
        b = synth.small_ints(rng, K * N, -3, 3)
        A, B = synth.to_bits(a, fmt), synth.to_bits(b, fmt)
        got, _, _ = gemm_gpu(A, B, M, N, K, fmt, tile=tile)
        assert np.array_equal(got, oracle.gemm(A, B, M, N, K, fmt).bits), tile


@pytest.mark.parametrize("fmt", FMTS)
def test_identity_and_permutation_bit_exact(fmt):
    rng = np.random.default_rng(9)
    for n in (64, 1000, 1024):
        N = 300
        X = synth.to_bits(rng.normal(0, 2, n * N), fmt)
        I = synth.to_bits(synth.identity_colmajor(n), fmt)
        got, _, _ = gemm_gpu(I, X, n, N, n, fmt)
        assert np.array_equal(got, X), "A = I"
        Xt = synth.to_bits(rng.normal(0, 2, N * n), fmt)
        got, _, _ = gemm_gpu(Xt, I, N, n, n, fmt)
        assert np.array_equal(got, Xt), "B = I"
        P = synth.to_bits(synth.cyclic_shift_colmajor(n, 3), fmt)
        got, _, _ = gemm_gpu(P, X, n, N, n, fmt)
        want = np.roll(X.reshape(N, n).T, -3, axis=0).T.ravel()
        assert np.array_equal(got, want), "A = P"


def test_rounding_is_nearest_even():
    # exact FP32 sum 1 + 3*2^-11 (resp. 1 + 3*2^-8) is a tie of the output
    # format: nearest-even gives 0x3C02 (0x3F82); truncation would give 0x3C01.
    for fmt, a1, want in (("f16", 3 * 2.0 ** -11, 0x3C02), ("bf16", 3 * 2.0 ** -8, 0x3F82)):
        A = synth.to_bits([1.0, a1], fmt)
        B = synth.to_bits([1.0, 1.0], fmt)
        got, _, _ = gemm_gpu(A, B, 1, 1, 2, fmt)
        assert int(got[0]) == want, (fmt, hex(int(got[0])))
        # and through a full-size tile path
        M, N, K = 256, 256, 64
        a = np.zeros(M * K)
        a[0], a[M] = 1.0, a1
        b = np.zeros(K * N)
        b[0], b[1] = 1.0, 1.0
        got, _, _ = gemm_gpu(synth.to_bits(a, fmt), synth.to_bits(b, fmt), M, N, K, fmt)
        assert int(got[0]) == want


def test_nonfinite_propagation():
    M, N, K = 64, 48, 96
    a = np.ones(M * K)
    a[5 + 7 * M] = np.inf         # row 5
    a[9 + 2 * M] = np.nan         # row 9
    b = np.ones(K * N)
    b[3 + 11 * K] = -np.inf       # column 11
    for fmt in FMTS:
        A, B = synth.to_bits(a, fmt), synth.to_bits(b, fmt)
        got, _, _ = gemm_gpu(A, B, M, N, K, fmt)
        assert_parity(got, oracle.gemm(A, B, M, N, K, fmt), fmt, "non-finite " + fmt)


def test_k_zero_writes_zero_and_empty_is_noop():
    import torch
    from bf16_gemm_decode_amd import binding
    C = Guarded(7 * 5)
    assert binding.gemm_f16_ptr(0, 0, C.ptr, 7, 5, 0) == 0
    torch.cuda.synchronize()
    assert np.all(C.out() == 0) and C.guards_intact()
    C = Guarded(16)
    A = dev(np.ones(16, np.uint16))
    assert binding.gemm_bf16_ptr(A.data_ptr(), A.data_ptr(), C.ptr, 0, 4, 4) == 0
    torch.cuda.synchronize()
    assert np.all(C.out() == 0xFFFF)


def test_tile_orderings_bit_identical_and_repeatable():
    # the ordering changes which workgroup computes a tile, never the
    # arithmetic inside it: any difference means a race.
    M, N, K = 2048, 4352, 1024
    A, B = synth.gemm_operands(M, N, K, "bf16", ("normal", 1.0, 0.02), seed=11)
    base = None
    for tile in (1, 2, 5, 7, 9, 10, 11, 13, 16):
        outs = []
        for gm in (1, 4, 8, 16):
            for xcd in (0, 1):
                got, guards, _ = gemm_gpu(A, B, M, N, K, "bf16", tile=tile, group_m=gm, xcd_remap=xcd)
                assert guards
                outs.append(got)
        got2, _, _ = gemm_gpu(A, B, M, N, K, "bf16", tile=tile, group_m=8, xcd_remap=1)
        outs.append(got2)
        for o in outs[1:]:
            assert np.array_equal(o, outs[0]), "tile %d differs across orderings" % tile
        if base is None:
            base = outs[0]
            idx = synth.sample_indices(M, N, 11, 512)
            assert_parity(base[idx], oracle.gemm_sampled(A, B, M, N, K, idx, "bf16"), "bf16", "orderings")


def test_pingpong_tile_bit_identical_to_tile_10():
    # tile 16 issues the same MFMAs as tile 10 on the same fragments, each
    # accumulator taking its k sub-steps in the same order (and the k tail
    # first), so the two schedules must agree bit for bit: a stage read too
    # early or refilled too soon would show here as a difference
    for i, (M, N, K) in enumerate([(520, 600, 200), (264, 300, 72), (1024, 768, 1036), (2048, 2304, 4096),
                                   (258, 70, 70)]):
        fmt = FMTS[i % 2]
        A, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), seed=40 + i)
        print("case pingpong vs tile 10", (M, N, K), fmt, flush=True)
        g10, guards10, _ = gemm_gpu(A, B, M, N, K, fmt, tile=10)
        g16, guards16, unchanged = gemm_gpu(A, B, M, N, K, fmt, tile=16)
        assert guards10 and guards16 and unchanged
        assert np.array_equal(g16, g10), (M, N, K, fmt)


def test_pingpong_tile_bit_identical_random_shapes():
    # the same property over seeded random shapes (M even: the tile takes
    # 4-byte rows), a race detector for the ping-pong schedule's waits
    rng = np.random.default_rng(2024)
    for i in range(24):
        M = 2 * int(rng.integers(1, 700))
        N = int(rng.integers(1, 1300))
        K = 2 * int(rng.integers(0, 600))
        fmt = FMTS[i % 2]
        A, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), seed=900 + i)
        print("case pingpong random", (M, N, K), fmt, flush=True)
        g10, _, _ = gemm_gpu(A, B, M, N, K, fmt, tile=10)
        g16, guards, _ = gemm_gpu(A, B, M, N, K, fmt, tile=16)
        assert guards
        assert np.array_equal(g16, g10), (M, N, K, fmt)


def test_pingpong_edge_global_loads_bit_identical_to_tile_10():
    # ragged M or N with 16-byte rows and K a multiple of 64: tile 16 loads
    # through global addresses, the lanes past M or N re-reading the tile's
    # first row or column (tile 10 takes the range-checked buffer loads);
    # the results must agree bit for bit, and C's guard bands stay intact
    for i, (M, N, K) in enumerate([(520, 264, 1024), (1032, 136, 512), (264, 600, 128), (8, 8, 64),
                                   (776, 1000, 192), (2056, 520, 256), (256, 200, 1024)]):
        fmt = FMTS[i % 2]
        A, B = synth.gemm_operands(M, N, K, fmt, ("normal", 1.0, 1.0), seed=70 + i)
        print("case pingpong edge", (M, N, K), fmt, flush=True)
        g10, guards10, _ = gemm_gpu(A, B, M, N, K, fmt, tile=10)
        g16, guards16, unchanged = gemm_gpu(A, B, M, N, K, fmt, tile=16)
        assert guards10 and guards16 and unchanged
        assert np.array_equal(g16, g10), (M, N, K, fmt)
        if i == 0:
            assert_parity(g16, oracle.gemm(A, B, M, N, K, fmt), fmt, "pingpong edge %s" % ((M, N, K),))


def test_tensor_wrapper_and_stream():
    import torch
    from bf16_gemm_decode_amd import gemm
    M, N, K = 300, 200, 130
    A, B = synth.gemm_operands(M, N, K, "f16", ("uniform", 1.0, 1.0), seed=3)
    tA = dev(A).view(torch.float16).reshape(K, M).t()      # column-major M x K
    tB = dev(B).view(torch.float16).reshape(N, K).t()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C = gemm(tA, tB)
    s.synchronize()
    got = host(C.t().contiguous().view(torch.int16)).ravel()
    assert_parity(got, oracle.gemm(A, B, M, N, K, "f16"), "f16", "tensor wrapper")
    with pytest.raises(ValueError):
        gemm(tA.contiguous(), tB)          # row-major A is rejected
