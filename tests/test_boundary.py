"""The C-ABI library on the CPU: it loads, exports every function the header
declares, rejects bad arguments before touching the GPU, and its tile
scheduler is a bijection that reduces to the grouped ordering of the
FlagGems Hygon page when the XCD renumbering is off."""
import ctypes
import os
import re

import pytest

import oracle
from bf16_gemm_decode_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "migemm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M))


def test_library_exports_every_declared_function():
    L = binding.lib()
    names = header_functions()
    assert {"gemm_f16", "gemm_bf16", "gemv_bf16"} <= names
    for n in names:
        assert hasattr(L, n), n
    assert names == set(binding.SIGNATURES), names ^ set(binding.SIGNATURES)
    assert L.migemm_abi_version() == 3


P = 0x10000        # a fake, aligned device address: never dereferenced on error paths


@pytest.mark.parametrize("fn", ["gemm_f16", "gemm_bf16"])
def test_gemm_argument_errors(fn):
    f = getattr(binding.lib(), fn)
    assert f(P, P + 0x100000, P + 0x200000, -1, 4, 4, None) == -1
    assert f(P, P + 0x100000, P + 0x200000, 4, 4, -2, None) == -1
    assert f(None, P + 0x100000, P + 0x200000, 4, 4, 4, None) == -2
    assert f(P, None, P + 0x200000, 4, 4, 4, None) == -2
    assert f(P, P + 0x100000, None, 4, 4, 4, None) == -2
    assert f(P + 1, P + 0x100000, P + 0x200000, 4, 4, 4, None) == -4
    assert f(P, P + 0x100000, P + 0x200001, 4, 4, 4, None) == -4
    # C overlaps A (A spans 4*4*2 = 32 bytes from P)
    assert f(P, P + 0x100000, P + 16, 4, 4, 4, None) == -3
    # C overlaps B
    assert f(P, P + 0x100000, P + 0x100000 - 8, 4, 4, 4, None) == -3
    # just touching is not overlapping: C starts where A ends (checked via plan, no launch)
    code, _ = binding.gemm_plan(0, P, P + 0x100000, P + 32, 4, 4, 4)
    assert code == 0
    assert f(P, P + 0x100000, P + 0x200000, 1 << 24, 4, 4, None) == -6
    assert f(P, P + 0x100000, P + 0x200000, 4, 4, 1 << 22, None) == -6


def test_gemm_empty_output_is_a_noop_without_gpu():
    L = binding.lib()
    # M == 0 or N == 0: nothing to write, returns before any HIP call
    assert L.gemm_f16(None, P + 0x100000, None, 0, 4, 4, None) == 0
    assert L.gemm_bf16(P, None, None, 4, 0, 4, None) == 0


def test_gemm_ex_config_errors():
    L = binding.lib()
    args = (P, P + 0x100000, P + 0x200000, 64, 64, 64)
    assert L.gemm_ex(2, *args, 0, 0, 1, None) == -5
    assert L.gemm_ex(0, *args, 99, 0, 1, None) == -5
    assert L.gemm_ex(0, *args, -1, 0, 1, None) == -5
    assert L.gemm_ex(0, *args, 0, -1, 1, None) == -5
    assert L.gemm_ex(0, *args, 0, 0, 2, None) == -5
    # 256-row tiles need 16-byte loads: M = 5000 has them, K = 4100 does not
    assert L.gemm_ex(1, P, P + 0x10000000, P + 0x20000000, 5000, 3000, 4100, 1, 0, 1, None) == -5


def test_every_tile_plan_fits_lds():
    # every explicit tile plans at a wide shape, fits the 160 KiB of LDS, and
    # reports its own tile extents
    want = {1: (256, 256), 2: (256, 128), 3: (128, 128), 4: (256, 256), 5: (256, 256),
            6: (256, 256), 7: (256, 256), 8: (256, 256), 9: (256, 128), 10: (256, 256),
            11: (64, 32), 12: (64, 64), 13: (128, 128), 16: (256, 256)}
    for tile, (tm, tn) in want.items():
        code, p = binding.gemm_plan(0, P, P + 2 ** 30, P + 2 ** 31, 1024, 1024, 1024, tile)
        assert code == 0, tile
        assert (p["tile_m"], p["tile_n"], p["tile_k"]) == (tm, tn, 32), tile
        assert 0 < p["lds_bytes"] <= 160 * 1024, tile
    # the full-line tiles: A ring of 4 x 32 k plus B ring of 64 k stages
    assert binding.gemm_plan(0, P, P + 2 ** 30, P + 2 ** 31, 1024, 1024, 1024, 7)[1]["lds_bytes"] == \
        4 * 32 * 256 * 2 + 3 * 64 * 256 * 2
    assert binding.gemm_plan(0, P, P + 2 ** 30, P + 2 ** 31, 1024, 1024, 1024, 9)[1]["lds_bytes"] == \
        4 * 32 * 256 * 2 + 4 * 64 * 128 * 2
    # the ping-pong tile: the rings of tile 10, 8 waves, m-major A only
    code, p = binding.gemm_plan(0, P, P + 2 ** 30, P + 2 ** 31, 1024, 1024, 1024, 16)
    assert code == 0 and p["lds_bytes"] == 160 * 1024 and p["waves"] == 8


def test_tn_plan_and_errors():
    L = binding.lib()
    # automatic tile: the least estimated time over rounds of workgroups
    code, p = binding.gemm_plan(0, P, P + 2 ** 30, P + 2 ** 31, 8192, 8192, 16384, a_kmajor=True)
    assert code == 0 and (p["tile_m"], p["tile_n"], p["vec_a"], p["vec_b"]) == (256, 256, 8, 8)
    assert p["lds_bytes"] == 2 * 64 * 256 * 2 + 3 * 64 * 256 * 2 and p["waves"] == 8
    # (K % 8 != 0: 4-byte rows, so the decode tiles are out and the GEMM's
    # estimate decides)
    code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 34816, 200, 5122, a_kmajor=True)
    assert code == 0 and (p["tile_m"], p["tile_n"]) == (256, 256) and p["grid"] == 136   # one round
    code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 2816, 2816, 4096, a_kmajor=True)
    assert code == 0 and (p["tile_m"], p["tile_n"]) == (256, 128) and p["grid"] == 242   # one round
    code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 2048, 2048, 4096, a_kmajor=True)
    assert code == 0 and (p["tile"], p["grid"]) == (13, 256)
    # at most 512 tiles of 32x32 (16-byte rows, K a multiple of 64; 768
    # otherwise): the small-problem kernel; fewer than 128 tiles of 128x128 with 16-byte
    # rows and K a multiple of 64: the 64x32 tile up to K = 2048, beyond it
    # the 128x128 tile; both layouts
    for kmaj in (False, True):
        for (M, N, K), (tile, grid) in (((512, 512, 512), (20, 256)), ((1024, 512, 4096), (20, 512)),
                                       ((768, 768, 768), (11, 288)), ((768, 768, 4096), (13, 36)), ((1024, 768, 64), (11, 384)),
                                       ((1056, 768, 64), (11, 408)), ((1024, 1024, 1024), (11, 512)),
                                       ((1152, 1408, 256), (11, 792)), ((1000, 1000, 4096), (13, 64)),
                                       ((1536, 1536, 256), (13, 144)),
                                       ((1544, 1536, 256), (13, 156)),
                                       ((512, 512, 131072), (20, 256))):
            code, p = binding.gemm_plan(0, P, P + 2 ** 30, P + 2 ** 31, M, N, K, a_kmajor=kmaj)
            assert code == 0 and (p["tile"], p["grid"]) == (tile, grid), (M, N, K, kmaj, p)
    # 16-byte rows and K a multiple of 64: the full-line 256x128 and 128x128
    # tiles, which then load through global addresses, in range or with the
    # lanes past M or N re-reading the tile's first row or column
    for (M, N, K), tile in (((8192, 1024, 16384), 9), ((8200, 1024, 16384), 16), ((2048, 2048, 16384), 13),
                            ((2056, 2048, 16384), 9), ((4096, 1024, 32768), 13), ((4096, 4096, 4096), 16),
                            ((8000, 1000, 16384), 9), ((2000, 2000, 16384), 13), ((3000, 3000, 4096), 16)):
        code, p = binding.gemm_plan(0, P, P + 2 ** 30, P + 2 ** 31, M, N, K)
        assert code == 0 and p["tile"] == tile, (M, N, K, p)
    # the small kernel's plan, and where it is not offered: B without 16-byte
    # rows (K % 8), a k-major A without them, 8-bit types, more than 65535
    # column blocks; an m-major A may have any M
    code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 513, 511, 520)
    assert code == 0 and (p["tile"], p["tile_m"], p["tile_n"], p["tile_k"], p["waves"], p["grid"], p["lds_bytes"]) == \
        (20, 32, 32, 32, 4, 17 * 16, 16384)
    # 8 waves once there are at most 256 tiles and K >= 1024
    for (M, N, K), waves in (((512, 512, 1016), 4), ((512, 512, 1024), 8), ((544, 512, 1024), 4),
                             ((256, 256, 32768), 8), ((640, 640, 4096), 4)):
        code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, M, N, K)
        assert code == 0 and (p["tile"], p["waves"], p["lds_bytes"]) == (20, waves, waves * 4096), (M, N, K, p)
    assert binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 512, 512, 516)[1]["tile"] != 20
    assert binding.gemm_plan(1, P + 2, P + 2 ** 30, P + 2 ** 31, 512, 512, 520, a_kmajor=True)[1]["tile"] != 20
    assert binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 512, 512, 516, 20)[0] == -4
    assert binding.gemm_plan(1, P + 2, P + 2 ** 30, P + 2 ** 31, 512, 512, 520, 20, a_kmajor=True)[0] == -4
    assert binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 64, (65536 * 32) + 1, 64, 20)[0] == -6
    assert binding.gemm_plan(2, P, P + 2 ** 30, P + 2 ** 31, 512, 512, 512, 20, a_kmajor=True)[0] == -5
    code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 8192, 8192, 512, 20)
    assert code == 0 and p["grid"] == 256 * 256                   # explicit: any tile count
    # the skinny tile: few columns only, and only with a k-major A
    code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 34816, 8, 5120, 14, a_kmajor=True)
    assert code == 0 and (p["tile"], p["tile_m"], p["tile_n"], p["waves"], p["grid"]) == (14, 32, 8, 4, 1088)
    assert binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 34816, 5, 5120, 14, a_kmajor=True)[1]["tile_n"] == 8
    code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 4096, 4, 5120, a_kmajor=True)
    assert code == 0 and (p["tile"], p["tile_n"]) == (14, 4)          # automatic up to 4 columns (M < 16384)
    assert binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 4096, 5, 5120, a_kmajor=True)[1]["tile"] == 15
    assert L.gemm_tn_ex(0, P, P + 0x100000, P + 0x200000, 64, 9, 64, 14, 0, 1, None) == -5
    assert L.gemm_ex(0, P, P + 0x100000, P + 0x200000, 64, 16, 64, 14, 0, 1, None) == -5
    # the batch tile: 9 .. 128 columns, token blocks of 16 .. 128; 2 waves
    # (32 rows of W) per workgroup for a 16-token block, else 4 (64 rows)
    for n, tn in ((9, 16), (16, 16), (17, 32), (33, 64), (64, 64), (65, 128), (128, 128)):
        code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 34816, n, 5120, 15, a_kmajor=True)
        w = 2 if tn == 16 else 4
        assert code == 0 and (p["tile"], p["tile_m"], p["tile_n"], p["tile_k"], p["waves"]) == (15, 16 * w, tn, 128, w)
        assert p["grid"] == 34816 // (16 * w) and p["lds_bytes"] == 2 * tn * 272 + w * 4096
    assert binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 4096, 32, 5120, a_kmajor=True)[1]["tile"] == 15
    assert binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 34816, 257, 5120, a_kmajor=True)[1]["tile"] == 9
    # the row-balanced tile: W's rows cut into 256 equal parts, rounded up to
    # a multiple of 8 and capped at 144 (9 waves of 16); token blocks of
    # 16 .. 256; automatic for 2 .. 128 columns once M >= 16384, and from 33
    # columns for any M
    for M, R in ((34816, 136), (16384, 64), (2051, 16), (100, 8), (36864, 144), (40000, 144)):
        for n, tn in ((1, 16), (17, 32), (64, 64), (65, 128), (129, 256), (256, 256)):
            code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, M, n, 5120, 18, a_kmajor=True)
            assert code == 0 and (p["tile"], p["tile_m"], p["tile_n"], p["tile_k"], p["waves"]) == (18, R, tn, 64, 9)
            assert p["grid"] == -(-M // R) and p["lds_bytes"] == 2 * tn * 144 + 9 * 2048
    # the wide row-balanced tile: the same rows per workgroup, 8 waves,
    # 128- or 256-column blocks; automatic for 65 .. 256 columns once M > 30720
    for M, R in ((34816, 136), (30721, 128), (16384, 64), (100, 8), (40000, 144)):
        for n, tn, lds in ((1, 128, 4 * 17 * 2048 + 1024), (128, 128, 4 * 17 * 2048 + 1024),
                           (129, 256, 3 * 25 * 2048 + 1024), (256, 256, 3 * 25 * 2048 + 1024)):
            code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, M, n, 5120, 19, a_kmajor=True)
            assert code == 0 and (p["tile"], p["tile_m"], p["tile_n"], p["tile_k"], p["waves"]) == (19, R, tn, 64, 8)
            assert p["grid"] == -(-M // R) and p["lds_bytes"] == lds <= 160 * 1024
    assert L.gemm_tn_ex(0, P, P + 0x100000, P + 0x200000, 64, 257, 64, 19, 0, 1, None) == -5
    assert L.gemm_ex(0, P, P + 0x100000, P + 0x200000, 64, 16, 64, 19, 0, 1, None) == -5
    for M, n, want in ((34816, 1, 14), (34816, 2, 18), (34816, 4, 18), (34816, 64, 18), (34816, 65, 19),
                       (34816, 128, 19), (34816, 256, 19), (34816, 257, 9), (30721, 65, 19), (30720, 65, 18),
                       (30720, 129, 9), (16384, 2, 18), (16383, 2, 14), (4096, 32, 15), (4096, 33, 18),
                       (4096, 128, 18), (64, 33, 18)):
        code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, M, n, 5120, a_kmajor=True)
        assert code == 0 and p["tile"] == want, (M, n, p["tile"])
    assert L.gemm_tn_ex(0, P, P + 0x100000, P + 0x200000, 64, 257, 64, 18, 0, 1, None) == -5
    assert L.gemm_ex(0, P, P + 0x100000, P + 0x200000, 64, 16, 64, 18, 0, 1, None) == -5
    assert L.gemm_tn_ex(0, P, P + 0x100000, P + 0x200000, 64, 129, 64, 15, 0, 1, None) == -5
    assert L.gemm_ex(0, P, P + 0x100000, P + 0x200000, 64, 16, 64, 15, 0, 1, None) == -5
    # only the full-line tiles take a k-major A
    for tile in (1, 2, 3, 4, 5, 6, 16):
        assert L.gemm_tn_ex(0, P, P + 0x100000, P + 0x200000, 64, 64, 64, tile, 0, 1, None) == -5
    # odd K, or an operand only 2-byte aligned: not even 4-byte rows
    assert L.gemm_tn_ex(0, P, P + 0x100000, P + 0x200000, 64, 64, 61, 7, 0, 1, None) == -4
    assert L.gemm_tn_ex(0, P + 2, P + 0x100000, P + 0x200000, 64, 64, 64, 7, 0, 1, None) == -4
    # K = 4 mod 8 (4-byte rows): the full-line tiles only
    code, p = binding.gemm_plan(0, P, P + 2 ** 20, P + 2 ** 21, 64, 64, 60, 7, a_kmajor=True)
    assert code == 0 and p["tile"] == 7 and (p["vec_a"], p["vec_b"]) == (2, 2)
    assert binding.gemm_plan(0, P, P + 2 ** 20, P + 2 ** 21, 64, 8, 60, 14, a_kmajor=True)[0] == -4
    assert binding.gemm_plan(0, P, P + 2 ** 20, P + 2 ** 21, 64, 64, 60, 0, a_kmajor=True)[1]["tile"] == 11     # few tiles: the 64x32 tile
    # the shared checks
    assert L.gemm_tn_f16(P, P + 0x100000, P + 0x200000, -1, 64, 64, None) == -1
    assert L.gemm_tn_bf16(None, P + 0x100000, P + 0x200000, 64, 64, 64, None) == -2
    assert L.gemm_tn_f16(P, P + 0x100000, P + 16, 64, 64, 64, None) == -3
    assert L.gemm_tn_f16(None, None, None, 0, 0, 64, None) == 0


def test_exact_shape_table():
    # measured exact-shape configurations apply when tile and GROUP_M are automatic
    plan = lambda dt, M, N, K, tile=0, gm=0, tn=False: binding.gemm_plan(
        dt, P, P + 2 ** 30, P + 2 ** 31, M, N, K, tile, gm, a_kmajor=tn)[1]
    assert (plan(1, 4096, 34816, 5120)["tile"], plan(1, 4096, 34816, 5120)["group_m"]) == (16, 8)
    assert (plan(1, 34816, 4096, 5120, tn=True)["tile"], plan(1, 34816, 4096, 5120, tn=True)["group_m"]) == (10, 4)
    assert (plan(0, 8192, 8192, 16384)["tile"], plan(0, 8192, 8192, 16384)["group_m"]) == (16, 8)
    assert (plan(1, 5000, 3000, 4100)["tile"], plan(1, 5000, 3000, 4100)["group_m"]) == (16, 16)
    # an explicit GROUP_M or tile, another dtype or shape: the heuristics
    assert plan(1, 4096, 34816, 5120, gm=16)["group_m"] == 16
    assert plan(1, 4096, 34816, 5120, tile=9)["tile"] == 9
    assert plan(0, 4096, 34816, 5120)["group_m"] == 8
    assert plan(1, 4096, 34816, 5128)["group_m"] == 8


def test_splitk_rules_and_errors():
    L = binding.lib()
    # automatic slices: >= 256 workgroups on the 256x256 tile, else 256x128; >= 1024 k each, <= 32
    assert L.migemm_splitk_splits(1, 0, 2048, 2048, 65536) == 4        # 64 tiles x 4
    assert L.migemm_splitk_splits(1, 0, 8192, 1024, 16384) == 2        # 128 tiles x 2
    assert L.migemm_splitk_splits(1, 0, 1024, 1024, 65536) == 16       # 16 tiles x 16
    assert L.migemm_splitk_splits(1, 0, 512, 512, 131072) == 32        # 256x128: 8 tiles x 32
    assert L.migemm_splitk_splits(0, 1, 1024, 1024, 4096) == 4         # 1024 k per slice
    assert L.migemm_splitk_splits(0, 0, 8192, 8192, 16384) == 1
    assert L.migemm_splitk_splits(1, 1, 34816, 16, 5120) == 1      # decode widths stream A once
    assert L.migemm_splitk_splits(2, 1, 1024, 1024, 65536) == 1    # 8-bit types: no split
    assert L.migemm_splitk_workspace_bytes(100, 30, 4) == 4 * 100 * 30 * 4
    assert L.migemm_splitk_workspace_bytes(100, 30, 1) == 0
    W = P + 0x10000000
    call = lambda **k: L.gemm_splitk_ex(*[dict(dt=0, ak=0, A=P, B=P + 0x1000000, C=P + 0x2000000, M=512,
                                                N=512, K=4096, S=4, tile=0, gm=0, xcd=1, ws=W,
                                                wsb=1 << 30, st=None, **{})[x] if x not in k else k[x]
                                          for x in ("dt", "ak", "A", "B", "C", "M", "N", "K", "S",
                                                    "tile", "gm", "xcd", "ws", "wsb", "st")])
    assert call(dt=2) == -5 and call(ak=2) == -5 and call(S=-1) == -5
    assert call(tile=3) == -5 and call(tile=7) == -5 and call(tile=16) == -5   # slices on 9, 10, 13 only
    assert call(ws=None) == -2
    assert call(ws=W + 8) == -4
    assert call(wsb=4 * 512 * 512 * 4 - 1) == -6
    assert call(ws=P + 0x1000000) == -3                           # workspace on B
    assert call(M=-1) == -1
    assert call(M=0) == 0                                         # nothing to do


def test_q8_plan_and_errors():
    L = binding.lib()
    # 8-bit GEMMs: k-major A only, K in elements (multiple of 16), tiles 9, 10, 13 (and 17 for FP8)
    # automatic: FP8 on the double-rate tile 17 once 256x128 tiles fill the chip, INT8 on 10
    code, p = binding.gemm_plan(2, P, P + 2 ** 30, P + 2 ** 31, 8192, 8192, 16384, a_kmajor=True)
    assert code == 0 and (p["tile"], p["tile_m"], p["tile_n"], p["tile_k"]) == (17, 256, 128, 64)
    code, p = binding.gemm_plan(4, P, P + 2 ** 30, P + 2 ** 31, 8192, 8192, 16384, a_kmajor=True)
    assert code == 0 and (p["tile"], p["tile_m"], p["tile_n"], p["tile_k"]) == (10, 256, 256, 64)
    code, p = binding.gemm_plan(4, P, P + 2 ** 30, P + 2 ** 31, 8192, 2048, 4096, a_kmajor=True)
    assert code == 0 and p["tile"] == 9
    code, p = binding.gemm_plan(3, P, P + 2 ** 30, P + 2 ** 31, 512, 512, 512, a_kmajor=True)
    assert code == 0 and p["tile"] == 13
    assert binding.gemm_plan(2, P, P + 2 ** 30, P + 2 ** 31, 512, 512, 512)[0] == -5   # m-major A
    for q in (2, 3, 4):
        assert L.gemm_tn_q_ex(q, P, P + 0x100000, P + 0x200000, 64, 64, 40, 1.0, 0, 0, 1, None) == -4
        assert L.gemm_tn_q_ex(q, P + 8, P + 0x100000, P + 0x200000, 64, 64, 64, 1.0, 0, 0, 1, None) == -4
        for tile in (1, 3, 7, 8, 11, 12, 14, 15, 16):
            assert L.gemm_tn_q_ex(q, P, P + 0x100000, P + 0x200000, 64, 64, 64, 1.0, tile, 0, 1, None) == -5
        assert L.gemm_tn_ex(q, P, P + 0x100000, P + 0x200000, 64, 64, 64, 0, 0, 1, None) == -5
        # tile 17 (the double-rate FP8 MFMA): FP8 only
        assert (L.gemm_tn_q_ex(q, P, P + 0x100000, P + 0x200000, 64, 64, 64, 1.0, 17, 0, 1, None) == -5) == (q == 4)
        assert L.gemm_ex(q, P, P + 0x100000, P + 0x200000, 64, 64, 64, 0, 0, 1, None) == -5
        assert L.gemm_tn_q_ex(q, P, P + 0x100000, P + 0x200000, -1, 64, 64, 1.0, 0, 0, 1, None) == -1
        assert L.gemm_tn_q_ex(q, None, P + 0x100000, P + 0x200000, 64, 64, 64, 1.0, 0, 0, 1, None) == -2
        assert L.gemm_tn_q_ex(q, P, P + 0x100000, P + 16, 64, 64, 64, 1.0, 0, 0, 1, None) == -3
        assert L.gemm_tn_q_ex(q, None, None, None, 0, 0, 64, 1.0, 0, 0, 1, None) == 0
    assert L.gemm_tn_q_ex(0, P, P + 0x100000, P + 0x200000, 64, 64, 64, 1.0, 0, 0, 1, None) == -5
    code, p = binding.gemm_plan(2, P, P + 2 ** 30, P + 2 ** 31, 8192, 8192, 16384, 17, a_kmajor=True)
    assert code == 0 and (p["tile_m"], p["tile_n"], p["waves"], p["lds_bytes"]) == (256, 128, 8, 3 * (256 + 128) * 128)
    assert L.gemm_ex(0, P, P + 0x100000, P + 0x200000, 64, 64, 64, 17, 0, 1, None) == -5     # not for 16-bit
    assert L.gemm_tn_ex(1, P, P + 0x100000, P + 0x200000, 64, 64, 64, 17, 0, 1, None) == -5
    assert L.gemm_tn_q_ex(5, P, P + 0x100000, P + 0x200000, 64, 64, 64, 1.0, 0, 0, 1, None) == -5
    # C = At + 16 overlaps: At spans M*K bytes (one byte per element)
    assert L.gemm_tn_i8(P, P + 0x100000, P + 64 * 64 - 2, 64, 64, 64, 1.0, None) == -3


def test_gemv_argument_errors():
    L = binding.lib()
    assert L.gemv_bf16(P, P + 0x100000, P + 0x200000, -1, 8, 1, None) == -1
    assert L.gemv_bf16(None, P + 0x100000, P + 0x200000, 8, 8, 1, None) == -2
    assert L.gemv_bf16(P, P + 0x100000, P + 0x200001, 8, 8, 1, None) == -4
    assert L.gemv_bf16(P, P + 0x100000, P + 8, 8, 8, 1, None) == -3       # Y inside W
    assert L.gemv_bf16(P, P + 0x100000, P + 0x100000, 8, 8, 1, None) == -3  # Y on X
    assert L.gemv_bf16_ex(P, P + 0x100000, P + 0x200000, 8, 8, 1, 3, None) == -5
    assert L.gemv_bf16(P, P + 0x100000, P + 0x200000, 8, 8, 0, None) == 0    # n == 0
    assert L.gemv_bf16(None, P, None, 0, 8, 4, None) == 0                    # M == 0
    assert L.gemv_bf16(None, None, None, 0, 8, 4, None) == -2                # X has 32 elements


def test_plan_choices():
    # headline square shape: 256x256 tiles, 16-byte loads, 32 x 32 tiles
    code, p = binding.gemm_plan(0, P, P + 2 ** 30, P + 2 ** 31, 8192, 8192, 16384)
    assert code == 0 and (p["tile_m"], p["tile_n"], p["vec_a"], p["vec_b"], p["grid"]) == \
        (256, 256, 8, 8, 1024)
    assert p["tile_k"] == 32 and p["tile"] == 16 and p["waves"] == 8 and p["a_kmajor"] == 0
    assert p["lds_bytes"] <= 160 * 1024
    # ragged: M = 5000 keeps 16-byte A rows, K = 4100 leaves B 4-byte rows,
    # which the full-line tiles take (k loop to 4096, then the last 4 k)
    code, p = binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 5000, 3000, 4100)
    assert code == 0 and (p["tile_m"], p["vec_a"], p["vec_b"]) == (256, 8, 2)
    assert p["grid"] == 20 * 12
    # the 256-row tiles of the older kernel still need 16-byte rows
    assert binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 5000, 3000, 4100, 2)[0] == -5
    assert binding.gemm_plan(1, P, P + 2 ** 30, P + 2 ** 31, 5000, 3000, 4100, 9)[0] == 0
    # odd everything: element loads
    code, p = binding.gemm_plan(1, P + 2, P + 2 ** 30 + 2, P + 2 ** 31, 33, 17, 65)
    assert code == 0 and (p["vec_a"], p["vec_b"]) == (1, 1)
    # explicit grouped width is clamped to the tile rows
    code, p = binding.gemm_plan(0, P, P + 2 ** 30, P + 2 ** 31, 1024, 1024, 64, 3, 16, 0)
    assert code == 0 and p["group_m"] == 8 and p["xcd_remap"] == 0


@pytest.mark.parametrize("group_m", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("num_xcd", [1, 8])
def test_tile_scheduler_bijection(group_m, num_xcd):
    for npm in (1, 2, 5, 8, 13, 32):
        for npn in (1, 3, 7, 16, 33):
            seen = {binding.tile_coord(w, npm, npn, group_m, num_xcd) for w in range(npm * npn)}
            assert len(seen) == npm * npn
            assert all(0 <= a < npm and 0 <= b < npn for a, b in seen)


def test_tile_scheduler_without_remap_is_the_grouped_ordering():
    # the product's mixed-radix map against the oracle's table, which walks
    # the tiles group by group, column by column, row by row
    for npm, npn, gm in ((5, 3, 2), (16, 136, 8), (7, 9, 4), (32, 32, 16), (20, 12, 8), (3, 5, 8),
                         (1, 7, 1), (9, 1, 4)):
        table = oracle.grouped_order(npm, npn, gm)
        assert [binding.tile_coord(w, npm, npn, gm, 1) for w in range(npm * npn)] == table
        assert [oracle.grouped_tile(w, npm, npn, gm) for w in range(0, npm * npn, 7)] == table[::7]


def test_tile_scheduler_xcd_locality():
    # With the renumbering, the ids one XCD receives (x, x+8, x+16, ...) are a
    # contiguous range of the grouped ordering.
    npm, npn, gm = 32, 32, 8
    for x in range(8):
        ids = list(range(x, npm * npn, 8))
        coords = [binding.tile_coord(w, npm, npn, gm, 8) for w in ids]
        logical = [i for i in range(npm * npn)
                   if oracle.grouped_tile(i, npm, npn, gm) in set(coords)]
        assert logical == list(range(logical[0], logical[0] + len(ids)))


def test_tile_coord_rejects_bad_input():
    with pytest.raises(binding.MigemmError):
        binding.tile_coord(15, 5, 3, 2, 1)
    with pytest.raises(binding.MigemmError):
        binding.tile_coord(0, 5, 3, 0, 1)


def test_attention_argument_errors_and_segments():
    L = binding.lib()
    ws = 1 << 20
    args = lambda **k: dict(dict(Q=P, Kc=P + 0x1000000, Vc=P + 0x2000000, bt=P + 0x3000000,
                                 sl=P + 0x3100000, Out=P + 0x3200000, B=1, Hq=16, Hkv=4, D=256,
                                 bs=784, maxb=2, nb=4, scale=0.0625, maxlen=1000, S=16,
                                 ws=P + 0x4000000, wsb=ws), **k)

    def call(a):
        return L.attention_decode_bf16(a["Q"], a["Kc"], a["Vc"], a["bt"], a["sl"], a["Out"], a["B"],
                                       a["Hq"], a["Hkv"], a["D"], a["bs"], a["maxb"], a["nb"],
                                       a["scale"], a["maxlen"], a["S"], a["ws"], a["wsb"], None)
    assert call(args(B=0)) == 0                       # nothing to do, nothing touched
    assert call(args(Hq=-1)) == -1
    assert call(args(Hq=6)) == -1                     # Hq not a multiple of Hkv
    assert call(args(D=96)) == -5                     # head dim not built
    assert call(args(Hq=64)) == -5                    # group of 16 heads not built
    assert call(args(S=2000)) == -5
    assert call(args(Q=None)) == -2
    assert call(args(Kc=P + 0x1000008)) == -4         # caches need 16-byte rows
    assert call(args(wsb=1000)) == -6                 # workspace too small
    assert call(args(Out=P + 8)) == -3                # Out inside Q
    assert call(args(ws=P + 0x3000000 - 64)) == -3    # workspace over the block table
    assert call(args(ws=P + 0x3100000 - 16)) == -3    # workspace over seq_lens
    assert call(args(B=70000, wsb=1 << 40)) == -6     # grid z limit
    assert call(args(maxb=1 << 22, bs=1024)) == -6    # token positions past int
    # workspace: partial max, denominator and D outputs per (b, h, segment)
    assert L.migemm_attention_workspace_bytes(2, 16, 256, 32) == 2 * 16 * 32 * 258 * 4
    # automatic segments: ~1024 workgroups, >= 128 tokens each, <= 256
    assert L.migemm_attention_segments(1, 16, 4, 32768) == 128
    assert L.migemm_attention_segments(1, 16, 4, 16384) == 128
    assert L.migemm_attention_segments(1, 16, 4, 8192) == 64
    assert L.migemm_attention_segments(8, 16, 4, 8192) == 16
    assert L.migemm_attention_segments(32, 16, 4, 4096) == 4
    assert L.migemm_attention_segments(1, 32, 4, 32768) == 64   # groups of 8: 2 workgroups each
    assert L.migemm_attention_segments(1, 16, 4, 100) == 1
    assert L.migemm_attention_segments(1000, 16, 4, 32768) == 1


def test_gemv_route():
    # the automatic route by token count (16-byte rows); non-zero
    # rows_per_block keeps the vector kernel; beyond the GEMM's size limits
    # many tokens stay on the vector kernel instead of failing
    W, X, Y = P, P + (1 << 36), P + (1 << 37)
    for n, want in ((1, 1), (2, 18), (3, 18), (4, 18), (5, 18), (64, 18), (65, 19), (128, 19), (256, 19),
                    (257, 9), (1000, 9)):
        assert binding.gemv_route(W, X, Y, 34816, 5120, n) == (0, want), n
    for n, want in ((1, 1), (2, 1), (3, 14), (4, 14), (5, 15), (32, 15), (33, 18), (128, 18), (129, 9)):
        assert binding.gemv_route(W, X, Y, 4096, 4096, n) == (0, want), n
    assert binding.gemv_route(W, X, Y, 16384, 4096, 2) == (0, 18)
    assert binding.gemv_route(W, X, Y, 16376, 4096, 2) == (0, 1)
    assert binding.gemv_route(W, X, Y, 34816, 5120, 16, rows_per_block=8) == (0, 1)
    assert binding.gemv_route(W, X, Y, 34816, 5122, 16) == (0, 1)          # K % 8: no MFMA route
    assert binding.gemv_route(W, X, Y, (1 << 23) + 64, 8, 257) == (0, 1)    # M past the GEMM limit
    assert binding.gemv_route(W, X, Y, (1 << 23) + 64, 8, 129) == (0, 19)
    assert binding.gemv_route(W, X, Y, 64, (1 << 21) + 8, 129) == (0, 1)    # K past the GEMM limit
    assert binding.gemv_route(W, X, Y, (1 << 23) + 64, 8, 64) == (0, 18)
    assert binding.gemv_route(W, X, Y, 100, 8, 64) == (0, 18)
    assert binding.gemv_route(W, X, Y, 0, 8, 4) == (0, 0)
    assert binding.gemv_route(W, X, Y, 8, 8, -1)[0] == -1
    assert binding.gemv_route(W, X, W + 2, 8, 8, 1)[0] == -3               # Y over W


def test_attention_noalloc_host_errors():
    # the allocation-free attention entry: host-side checks before any HIP
    # call (shape, nulls, alignment, and the scratch limit)
    L = binding.lib()

    def call(B=1, Hq=16, Hkv=4, D=256, S=16, Q=P, Out=P + 0x3200000, maxlen=1000):
        return L.attention_decode_bf16_noalloc(Q, P + 0x1000000, P + 0x2000000, P + 0x3000000,
                                               P + 0x3100000, Out, B, Hq, Hkv, D, 784, 2, 4, 0.0625,
                                               maxlen, S, None)
    assert call(B=0) == 0
    assert call(Hq=-1) == -1
    assert call(D=96) == -5
    assert call(Q=None) == -2
    assert call(Q=P + 8) == -4
    assert call(Out=P + 8) == -3
    # partials of 16 heads x 1024 segments x 258 FP32 = 16.9 MB > the 8 MiB array
    assert L.migemm_attention_workspace_bytes(1, 16, 256, 1024) > (8 << 20)
    assert call(S=1024) == -6
    # 4 sequences x 16 heads x 128 segments x 258 FP32 = 8.45 MB, just past 8 MiB
    assert L.migemm_attention_workspace_bytes(4, 16, 256, 128) == 8454144 > (8 << 20)
    assert call(B=4, S=128) == -6
