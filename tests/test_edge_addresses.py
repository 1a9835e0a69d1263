"""Bounds of the 256x256 tiles' global-address loads on ragged launches
(gemm.hip, gemm_fl_kernel with EDGE; tiles 10 and 16): a model of the kernel's per-lane load
offsets, with the lanes past M or N moved to the tile's row 0 or column 0,
enumerated for every tile, wave, lane, and the first and last sub-step and
stage (addresses grow with k, so those bound the rest).  Every 16-byte load
must lie inside A (M*K*2 bytes) and B (N*K*2 bytes).  Host logic only: the
tile constants below are those of the 256x256 tiles (4x2 waves; an m-major A
in sub-steps of 32 k rows, a k-major A and B in stages of 64 k)."""
import pytest

BM, BN, WGM, WGN, BK = 256, 256, 4, 2, 32
NW = WGM * WGN
LA = BK * BM * 2 // (1024 * NW)          # A loads per wave per sub-step
LB = BN * 128 // (1024 * NW)             # B loads per wave per 64-k stage


def swz_a(kk):
    return (((kk & 7) << 1) ^ (kk & 8)) & (BM // 8 - 1)


def kmajor_a_loads(M, K):
    # k-major A (A(m,k) = A[k + m*K]): stage of 64 k, load q of 2*LA per
    # stage fills rows 8(q NW + wave) + l/8 with 16-byte piece x
    ks = K & ~7
    P_ = ((((ks + BK - 1) // BK) + 1) & ~1) // 2
    la = BM * 128 // (2048 * NW)
    for m0 in range(0, M, BM):
        for wave in range(NW):
            for lane in range(64):
                for q in range(2 * la):
                    c = 8 * (q * NW + wave) + (lane >> 3)
                    x = (lane & 7) ^ ((c >> 1) & 7)
                    off = (c * K + 8 * x) * 2 if m0 + c < M else 8 * x * 2
                    for pp in {0, max(P_ - 1, 0)} if P_ else ():
                        yield "A", (m0 * K + pp * 2 * BK) * 2 + off


def edge_loads(M, N, K, bn=BN):
    lb = bn * 128 // (1024 * NW)
    ks = K & ~7
    J = (((ks + BK - 1) // BK) + 1) & ~1
    P_ = J // 2
    for m0 in range(0, M, BM):
        for n0 in range(0, N, bn):
            for wave in range(NW):
                for lane in range(64):
                    for q in range(LA):
                        P = (q * NW + wave) * 1024 + lane * 16
                        kk, b = P // (BM * 2), P % (BM * 2)
                        m = ((b >> 4) ^ swz_a(kk)) << 3
                        off = (kk * M + m0 + m) * 2 if m0 + m < M else kk * M * 2
                        for jj in {0, max(J - 1, 0)} if J else ():
                            yield "A", jj * BK * M * 2 + off
                    c0 = 8 * wave + (lane >> 3)
                    x = (lane & 7) ^ ((c0 >> 1) & 7)
                    for q in range(lb):
                        col = n0 + c0 + 8 * q * NW
                        off = (c0 * K + 8 * x) * 2 + 8 * q * NW * K * 2 if col < N else 8 * x * 2
                        for pp in {0, max(P_ - 1, 0)} if P_ else ():
                            yield "B", (n0 * K + pp * 2 * BK) * 2 + off


@pytest.mark.parametrize("bn", [256, 128])        # 256x256 tiles; the 256x128 FP8 tile (B side)
@pytest.mark.parametrize("M,N,K", [(520, 264, 1024), (264, 136, 128), (8, 8, 64), (1032, 136, 512),
                                   (776, 1000, 192), (2056, 520, 256), (256, 200, 1024), (5000, 3000, 64)])
def test_edge_clamped_loads_stay_inside_operands(M, N, K, bn):
    assert (K & ~7) % 64 == 0 and M % 8 == 0          # the planner's condition for these launches
    size = {"A": M * K * 2, "B": N * K * 2}
    n = 0
    for which, addr in edge_loads(M, N, K, bn):
        assert 0 <= addr and addr + 16 <= size[which], (which, addr, size[which])
        n += 1
    assert n > 0


@pytest.mark.parametrize("M,N,K", [(520, 264, 1024), (264, 136, 128), (8, 8, 64), (4000, 520, 512), (776, 1000, 192)])
def test_edge_clamped_kmajor_a_loads_stay_inside_a(M, N, K):
    size = M * K * 2
    n = 0
    for _, addr in kmajor_a_loads(M, K):
        assert 0 <= addr and addr + 16 <= size, (addr, size)
        n += 1
    assert n > 0


def test_unclamped_loads_would_leave_the_operands():
    # the clamp matters: without it a ragged tile reads past the end of B
    M, N, K = 520, 264, 1024
    n0 = 256                                        # the last column tile
    worst = max((n0 * K + (K - 2 * BK)) * 2 + (c0 * K + 8 * 7) * 2 + 8 * q * NW * K * 2
                for c0 in range(64) for q in range(LB))
    assert worst + 16 > N * K * 2


def generic_edge_loads(bm, bn, wgm, wgn, M, N, K, kmajor):
    # the same model for any full-line tile: bm x bn, wgm x wgn waves
    nw = wgm * wgn
    ks = K & ~7
    J = (((ks + BK - 1) // BK) + 1) & ~1
    P_ = J // 2
    la_m, la_k, lb = BK * bm * 2 // (1024 * nw), bm * 128 // (2048 * nw), bn * 128 // (1024 * nw)

    def swz(kk):
        return (((kk & 7) << 1) ^ (kk & 8)) & (bm // 8 - 1)
    for m0 in range(0, M, bm):
        for n0 in range(0, N, bn):
            for wave in range(nw):
                for lane in range(64):
                    if not kmajor:
                        for q in range(la_m):
                            P = (q * nw + wave) * 1024 + lane * 16
                            kk, b = P // (bm * 2), P % (bm * 2)
                            m = ((b >> 4) ^ swz(kk)) << 3
                            off = (kk * M + m0 + m) * 2 if m0 + m < M else kk * M * 2
                            for jj in {0, max(J - 1, 0)} if J else ():
                                yield "A", jj * BK * M * 2 + off
                    else:
                        for q in range(2 * la_k):
                            c = 8 * (q * nw + wave) + (lane >> 3)
                            x = (lane & 7) ^ ((c >> 1) & 7)
                            off = (c * K + 8 * x) * 2 if m0 + c < M else 8 * x * 2
                            for pp in {0, max(P_ - 1, 0)} if P_ else ():
                                yield "A", (m0 * K + pp * 2 * BK) * 2 + off
                    c0 = 8 * wave + (lane >> 3)
                    x = (lane & 7) ^ ((c0 >> 1) & 7)
                    for q in range(lb):
                        col = n0 + c0 + 8 * q * nw
                        off = (c0 * K + 8 * x) * 2 + 8 * q * nw * K * 2 if col < N else 8 * x * 2
                        for pp in {0, max(P_ - 1, 0)} if P_ else ():
                            yield "B", (n0 * K + pp * 2 * BK) * 2 + off


@pytest.mark.parametrize("tile", [(256, 128, 4, 1), (128, 128, 2, 2), (64, 32, 2, 1), (64, 64, 2, 1)])
@pytest.mark.parametrize("kmajor", [False, True])
@pytest.mark.parametrize("M,N,K", [(520, 264, 1024), (8, 8, 64), (136, 40, 128), (1000, 1000, 256)])
def test_edge_clamped_loads_four_wave_tiles(tile, kmajor, M, N, K):
    size = {"A": M * K * 2, "B": N * K * 2}
    n = 0
    for which, addr in generic_edge_loads(*tile, M, N, K, kmajor):
        assert 0 <= addr and addr + 16 <= size[which], (which, addr, size[which])
        n += 1
    assert n > 0
