// api.hip -- the C ABI declared in include/migemm.h: argument checks,
// configuration choice and launch.  Every argument error is detected here,
// on the host, before any HIP call.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "migemm.h"
#include "tile_map.hpp"

namespace migemm {
int gemv_rows_per_wave(int n_tokens, int rows_per_block);
}

using namespace migemm;

namespace {

bool overlaps(const void *a, size_t abytes, const void *b, size_t bbytes)
{
    if (abytes == 0 || bbytes == 0) return false;
    uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

int vec_width(const void *p, int64_t stride_elems)
{
    uintptr_t a = (uintptr_t)p;
    if (stride_elems % 8 == 0 && a % 16 == 0) return 8;
    if (stride_elems % 2 == 0 && a % 4 == 0) return 2;
    return 1;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shared by gemm_ex and migemm_gemm_plan_for.  Returns 0 and fills L (and
// *launch = true) when a kernel must run, 0 with *launch = false for an empty
// output, or a negative MIGEMM_ERR_* code.
// Exact-shape configurations, measured on one MI355X with the per-workload
// report (GROUP_M x tile sweeps of the prefill shape in both layouts, the
// headline GEMM, the ragged BF16 GEMM).  Consulted when the caller leaves both
// the tile and the grouped width automatic; an entry whose tile the operands
// cannot take (alignment) is skipped.
struct ShapeConfig {
    int dtype, a_kmajor, M, N, K, tile, group_m;
};
constexpr ShapeConfig kShapeTable[] = {
    {DT_F16, 0, 8192, 8192, 16384, TILE_256x256_PP, 8},      // 1.54-1.64 ms vs 1.81-1.93 on tile 10
    {DT_BF16, 0, 4096, 34816, 5120, TILE_256x256_PP, 8},     // 1.029 ms vs 1.034 at 4, 1.049 at 16; tile 10 1.10
    {DT_BF16, 1, 34816, 4096, 5120, TILE_256x256_FL8, 4},    // 1.143 ms vs 1.166 at 8, 1.286 at 16
    {DT_BF16, 0, 5000, 3000, 4100, TILE_256x256_PP, 16},     // 101-124 us vs 131-148 on tile 10
};

const ShapeConfig *find_shape(int dtype, bool a_kmajor, int M, int N, int K)
{
    for (const ShapeConfig &c : kShapeTable)
        if (c.dtype == dtype && c.a_kmajor == (a_kmajor ? 1 : 0) && c.M == M && c.N == N && c.K == K)
            return &c;
    return nullptr;
}

int plan_gemm(int dtype, const uint16_t *A, const uint16_t *B, const uint16_t *C, int M, int N,
              int K, int tile, int group_m, int xcd_remap, GemmLaunch &L, bool &launch,
              bool a_kmajor = false)
{
    launch = false;
    if (dtype < DT_F16 || dtype > DT_I8 || (dt_is_8bit(dtype) && !a_kmajor)) return MIGEMM_ERR_CONFIG;
    const bool q8 = dt_is_8bit(dtype);
    if (q8) {
        // 8-bit elements: the kernels count K in 2-byte units; rows must be
        // whole 16-byte pieces
        if (K < 0) return MIGEMM_ERR_DIM;
        if (K % 16) return MIGEMM_ERR_ALIGN;
        K /= 2;
        if (!(tile == TILE_AUTO || tile == TILE_256x128_FL || tile == TILE_256x256_FL8 ||
              tile == TILE_128x128_SK || (tile == TILE_256x128_F8W && dtype != DT_I8)))
            return MIGEMM_ERR_CONFIG;
    }
    if (tile < TILE_AUTO || tile >= TILE_COUNT || group_m < 0 || xcd_remap < 0 || xcd_remap > 1)
        return MIGEMM_ERR_CONFIG;
    if (tile == TILE_256x128_F8W && !q8) return MIGEMM_ERR_CONFIG;   // FP8 only
    if (M < 0 || N < 0 || K < 0) return MIGEMM_ERR_DIM;
    if (M > MIGEMM_MAX_MN || N > MIGEMM_MAX_MN || K > MIGEMM_MAX_K) return MIGEMM_ERR_SIZE;
    const size_t abytes = (size_t)M * K * 2, bbytes = (size_t)K * N * 2, cbytes = (size_t)M * N * 2;
    if ((abytes && !A) || (bbytes && !B) || (cbytes && !C)) return MIGEMM_ERR_NULL;
    if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 1) return MIGEMM_ERR_ALIGN;
    if (overlaps(C, cbytes, A, abytes) || overlaps(C, cbytes, B, bbytes)) return MIGEMM_ERR_OVERLAP;

    L = GemmLaunch{};
    L.dtype = dtype;
    L.A = A;
    L.B = B;
    L.C = const_cast<uint16_t *>(C);
    L.M = M;
    L.N = N;
    L.K = K;
    L.vec_a = vec_width(A, a_kmajor ? K : M);
    L.vec_b = vec_width(B, K);
    L.c_vec = (M % 4 == 0 && (uintptr_t)C % 8 == 0) ? 1 : 0;
    L.a_kmajor = a_kmajor ? 1 : 0;
    // wide: 16-byte aligned rows of A and B (every tile).  fl: 4-byte
    // aligned rows, enough for the full-line tiles, whose 16-byte loads need
    // dword alignment only; their k loop stops at a multiple of 8 and adds
    // the last K % 8 k after it.
    const bool wide = (L.vec_a == 8 && L.vec_b == 8);
    const bool fl = (L.vec_a >= 2 && L.vec_b >= 2);
    auto is_fl = [](int t) { return (t >= TILE_256x256_FL && t <= TILE_128x128_SK) || t == TILE_256x256_PP; };
    // the small-problem kernel: 16-byte rows of B (and of a k-major A); an
    // m-major A is read 2 bytes at a time; its grid's second dimension is
    // the 32-column blocks
    const bool small_ok = !q8 && L.vec_b == 8 && (!a_kmajor || L.vec_a == 8) && cdiv(N, 32) <= 65535;
    if (tile == TILE_SMALL && !small_ok) return q8 ? MIGEMM_ERR_CONFIG : cdiv(N, 32) > 65535 ? MIGEMM_ERR_SIZE
                                                                                           : MIGEMM_ERR_ALIGN;
    if (tile == TILE_AUTO && group_m == 0 && !q8) {
        const ShapeConfig *c = find_shape(dtype, a_kmajor, M, N, K);
        if (c && (wide || c->tile == TILE_128x128 || (fl && is_fl(c->tile)))) {
            tile = c->tile;
            group_m = c->group_m;
        }
    }
    // Automatic tile for a 16-bit GEMM: the least estimated time, counting
    // rounds of workgroups over the 256 CUs.  Per round at K = 4096 (one
    // MI355X, square and 2:1 shapes from 1024 to 8192): 256x256 with 8 waves
    // 110 us per 256 tiles (the ping-pong variant, m-major A only, 5-10%
    // less: 102); 256x128 80 us per 256; 128x128 56 us for up to 256 tiles,
    // then 85 us per 512 (two workgroups per CU; the full-line 128x128 takes
    // 56 us per 256).
    auto auto_tile = [&]() {
        const int64_t t256 = cdiv(M, 256) * cdiv(N, 256), t2 = cdiv(M, 256) * cdiv(N, 128),
                      t128 = cdiv(M, 128) * cdiv(N, 128);
        // The small-problem kernel up to 768 of its tiles; with 16-byte rows
        // and K a multiple of 64 (the full-line tiles on global loads) only
        // up to 512: above that 64x32 or 128x128 is ahead (BF16, measured:
        // 768x768 at K = 1024 / 4096 / 8192 11.5 / 41.5 / 79.6 us against
        // 12.5 / 44.2 / 86.6, 1024x768x512 7.1 against 8.4; at 512 tiles
        // and below it stays well ahead, 512x1024x4096 32.7 against 41.5)
        const int64_t small_max = wide && K % 64 == 0 ? 512 : kSmallMaxTiles;
        if (small_ok && cdiv(M, 32) * cdiv(N, 32) <= small_max) return (int)TILE_SMALL;
        // Fewer than 128 tiles of 128x128 and a short K: the time per k
        // step (barrier and load latency, not the MFMAs) decides, so the
        // most workgroups win: 64x64 when they fill half the chip, else
        // 64x32 (FP16, measured: 512^3 8.0 us on 64x32 against 11.0 on
        // 128x128, 768^3 11.9 on 64x64 against 14.4, 1024^3 15.2 against
        // 17.7, 512x512x2048 23.1 against 29.7).  Over a long K the
        // 128x128 tile's throughput per CU wins again (512x512x131072: 1586
        // us against 1831 on 64x32).
        // With 16-byte rows and K a multiple of 64 (global-address loads,
        // ragged edges included; BF16, measured): 64x32 ahead of 64x64
        // everywhere (1024^3 11.6 us against 12.1, 1408x1152x256 6.1
        // against 6.7, 1024x1024x2048 20.0 against 20.9), and from K = 4096
        // the 128x128 tile ahead of both (1000x1000x4096 42.9 against 45.0
        // and 51.8, 1024x1024x8192 79.8 against 85.7 and 95.6): the cost
        // model below then picks it.
        if (fl && t128 < 128 && wide && K % 64 == 0) {
            if (K <= 2048) return (int)TILE_64x32_SK;
        } else if (fl && t128 < 128 && K <= 8192) {
            return cdiv(M, 64) * cdiv(N, 64) >= 128 ? (int)TILE_64x64_SK : (int)TILE_64x32_SK;
        }
        int best = TILE_128x128;
        int64_t cost = INT64_MAX;
        auto take = [&](int t, int64_t c) {
            if (c < cost) { cost = c; best = t; }
        };
        // With 16-byte rows and K a multiple of 64 the full-line tiles load
        // through global addresses (in range, or with the lanes past M or N
        // re-reading the tile's first row or column) and their smaller
        // shapes overtake the other kernels (BF16, per round at K = 4096,
        // measured: 256x128 74 us, 128x128 46 with an m-major A, 42
        // k-major; 8192x1024x16384 0.295 ms on 256x128 against 0.34 on the
        // plain 256x128 tile, 2048x2048x16384 0.18 on 128x128 against 0.22;
        // ragged: 8000x1000x16384 0.256 on 256x128 against 0.29 on the
        // plain one, 2000x2000x16384 0.163 on 128x128 against 0.204)
        const bool k64 = K % 64 == 0;
        const bool in2 = wide && k64;
        const bool in1 = wide && k64;
        if (fl) take(a_kmajor ? TILE_256x256_FL8 : TILE_256x256_PP, cdiv(t256, 256) * (a_kmajor ? 110 : 102));
        if (in2) take(TILE_256x128_FL, cdiv(t2, 256) * 74);
        else if (wide && !a_kmajor) take(TILE_256x128, cdiv(t2, 256) * 80);
        else if (fl) take(TILE_256x128_FL, cdiv(t2, 256) * 80);
        if (in1) take(TILE_128x128_SK, cdiv(t128, 256) * (a_kmajor ? 42 : 46));
        else if (!a_kmajor) take(TILE_128x128, t128 <= 256 ? 56 : cdiv(t128, 512) * 85);
        else if (fl) take(TILE_128x128_SK, cdiv(t128, 256) * 56);
        return best;
    };
    if (a_kmajor && q8) {
        if (!wide) return MIGEMM_ERR_ALIGN;
        // FP8: the double-rate MFMA tile (17) once its 256x128 tiles fill
        // the chip (8192x8192x16384: 1.06-1.08 ms against 1.30-1.43 on tile 10)
        if (tile == TILE_AUTO)
            tile = dtype != DT_I8 && cdiv(M, 256) * cdiv(N, 128) >= 256 ? TILE_256x128_F8W
                   : cdiv(M, 256) * cdiv(N, 256) >= 512                  ? TILE_256x256_FL8
                   : cdiv(M, 256) * cdiv(N, 128) >= 256                  ? TILE_256x128_FL
                                                                         : TILE_128x128_SK;
    } else if (a_kmajor) {
        // k-major A: the full-line tiles (4-byte rows) and, with 16-byte
        // rows, the few-token kernels
        if (!fl) return MIGEMM_ERR_ALIGN;
        if (tile == TILE_AUTO) {
            tile = wide && batch_wide_auto(M, N) ? TILE_BATCH_WIDE
                   : wide && batch_rows_auto(M, N) ? TILE_BATCH_ROWS
                   : wide && N <= kSkinnyAutoMax ? TILE_SKINNY
                   : wide && N <= kBatchAutoMax  ? TILE_BATCH
                                                 : auto_tile();
        } else if ((tile < TILE_256x256_FL) || tile == TILE_256x256_PP ||
                   (tile == TILE_SKINNY && N > kSkinnyMaxTokens) ||
                   (tile == TILE_BATCH && N > kBatchMaxTokens) ||
                   (tile == TILE_BATCH_ROWS && N > kBatchRowsMaxTokens) ||
                   (tile == TILE_BATCH_WIDE && N > kBatchWideMaxTokens)) {
            return MIGEMM_ERR_CONFIG;
        } else if (!wide && !is_fl(tile)) {
            return MIGEMM_ERR_ALIGN;
        }
    } else if (tile == TILE_AUTO) {
        tile = auto_tile();
    } else if (is_decode_tile(tile)) {
        return MIGEMM_ERR_CONFIG;   // only with a k-major A (gemm_tn_ex)
    } else if (tile != TILE_128x128 && tile != TILE_SMALL && !(wide || (fl && is_fl(tile)))) {
        return MIGEMM_ERR_CONFIG;   // the other tiles load 16-byte (full-line: 4-byte aligned) rows
    }
    L.tile = tile;
    int bm = kTileShapes[tile].bm, bn = kTileShapes[tile].bn;
    if (tile == TILE_SKINNY) bn = N <= 4 ? 4 : 8;
    if (tile == TILE_BATCH) {
        bm = batch_tile_m(N);
        bn = batch_tile_n(N);
    }
    if (tile == TILE_BATCH_ROWS) {
        bm = batch_rows_per_workgroup(M);
        bn = batch_rows_tile_n(N);
    }
    if (tile == TILE_BATCH_WIDE) {
        bm = batch_rows_per_workgroup(M);
        bn = batch_wide_tile_n(N);
    }
    const int64_t pm = cdiv(M, bm), pn = cdiv(N, bn);
    if (pm * pn > 0x7fffffff) return MIGEMM_ERR_SIZE;
    L.num_pid_m = (int)(pm ? pm : 1);
    L.num_pid_n = (int)(pn ? pn : 1);
    int gm = group_m ? group_m : 8;
    if (gm > L.num_pid_m) gm = L.num_pid_m;
    L.group_m = gm;
    L.num_xcd = xcd_remap ? 8 : 1;
    L.grid = pm * pn;
    L.in_range = (L.vec_a == 8 && L.vec_b == 8 && M % bm == 0 && N % bn == 0 && K % 64 == 0) ? 1 : 0;
    L.edge_gl = (!L.in_range && L.vec_a == 8 && L.vec_b == 8 && (K & ~7) % 64 == 0) ? 1 : 0;
    launch = (M > 0 && N > 0);
    return MIGEMM_OK;
}

// Y = X W^T on one of the decode kernels: W = At, X = B, Y = C (all
// row-major), the product gemm_tn computes
hipError_t decode_launch(int tile, int dtype, const uint16_t *At, const uint16_t *B, uint16_t *C,
                         int M, int N, int K, int c_vec, hipStream_t stream)
{
    SkinnyLaunch S{dtype, At, B, C, M, K, N, c_vec};
    return tile == TILE_SKINNY       ? skinny_launch(S, stream)
           : tile == TILE_BATCH      ? batch_launch(S, stream)
           : tile == TILE_BATCH_ROWS ? batch_rows_launch(S, stream)
                                     : batch_wide_launch(S, stream);
}

// gemm_launch, or the small-problem kernel for its tile
hipError_t launch_gemm_or_small(const GemmLaunch &L, hipStream_t stream)
{
    return L.tile == TILE_SMALL ? small_launch(L, stream) : gemm_launch(L, stream);
}

int finish(hipError_t e, void *stream)
{
    if (e != hipSuccess) return (int)e;
    if (stream == nullptr) {
        e = hipStreamSynchronize(nullptr);
        if (e != hipSuccess) return (int)e;
    }
    return MIGEMM_OK;
}

}  // namespace

extern "C" {

int gemm_ex(int dtype, const uint16_t *A, const uint16_t *B, uint16_t *C, int M, int N, int K,
            int tile, int group_m, int xcd_remap, void *stream)
{
    GemmLaunch L;
    bool launch;
    int rc = plan_gemm(dtype, A, B, C, M, N, K, tile, group_m, xcd_remap, L, launch);
    if (rc != MIGEMM_OK || !launch) return rc;
    return finish(launch_gemm_or_small(L, (hipStream_t)stream), stream);
}

int migemm_gemm_clocked(int dtype, const uint16_t *A, const uint16_t *B, uint16_t *C, int M, int N,
                        int K, int tile, int group_m, int xcd_remap, uint64_t *clocks, void *stream)
{
    GemmLaunch L;
    bool launch;
    int rc = plan_gemm(dtype, A, B, C, M, N, K, tile, group_m, xcd_remap, L, launch);
    if (rc != MIGEMM_OK || !launch) return rc;
    // the record is written by the full-line kernels only
    if (!((L.tile >= TILE_256x256_FL && L.tile <= TILE_128x128_SK) || L.tile == TILE_256x256_PP))
        return MIGEMM_ERR_CONFIG;
    if (!clocks) return MIGEMM_ERR_NULL;
    if ((uintptr_t)clocks % 8) return MIGEMM_ERR_ALIGN;
    const size_t cbytes = (size_t)M * N * 2, rbytes = (size_t)L.grid * 16;
    if (overlaps(clocks, rbytes, A, (size_t)M * K * 2) || overlaps(clocks, rbytes, B, (size_t)K * N * 2) ||
        overlaps(clocks, rbytes, C, cbytes))
        return MIGEMM_ERR_OVERLAP;
    L.clocks = clocks;
    return finish(gemm_launch(L, (hipStream_t)stream), stream);
}

int gemm_f16(const uint16_t *A, const uint16_t *B, uint16_t *C, int M, int N, int K, void *stream)
{
    return gemm_ex(DT_F16, A, B, C, M, N, K, TILE_AUTO, 0, 1, stream);
}

int gemm_bf16(const uint16_t *A, const uint16_t *B, uint16_t *C, int M, int N, int K, void *stream)
{
    return gemm_ex(DT_BF16, A, B, C, M, N, K, TILE_AUTO, 0, 1, stream);
}

int gemm_tn_ex(int dtype, const uint16_t *At, const uint16_t *B, uint16_t *C, int M, int N, int K,
               int tile, int group_m, int xcd_remap, void *stream)
{
    if (dt_is_8bit(dtype)) return MIGEMM_ERR_CONFIG;   // gemm_tn_q_ex takes the scale
    GemmLaunch L;
    bool launch;
    int rc = plan_gemm(dtype, At, B, C, M, N, K, tile, group_m, xcd_remap, L, launch, true);
    if (rc != MIGEMM_OK || !launch) return rc;
    if (is_decode_tile(L.tile))
        // C(m,n) = sum_k At[k + m*K] B[k + n*K] is Y = X W^T with W = At,
        // X = B, Y = C, all row-major: the decode kernels' contract
        return finish(decode_launch(L.tile, dtype, At, B, C, M, N, K, L.c_vec, (hipStream_t)stream), stream);
    return finish(launch_gemm_or_small(L, (hipStream_t)stream), stream);
}

// The automatic split: the 256x256 tile (10) with the smallest power-of-two
// slice count that gives it >= 256 workgroups, else the 256x128 tile (9)
// likewise, else tile 9 with as many slices as allowed; slices keep >= 1024
// k and number at most 32 (measured on 1024^2 .. 8192x1024 outputs with K
// of 16K .. 128K).  Returns the slice count, *tile the tile.
static int splitk_choice(int M, int N, int K, int a_kmajor, int *tile)
{
    *tile = TILE_256x128_FL;
    if (M <= 0 || N <= 0 || K <= 0 || (a_kmajor && N <= kBatchAutoMax)) return 1;
    const int64_t t10 = cdiv(M, 256) * cdiv(N, 256), t9 = cdiv(M, 256) * cdiv(N, 128);
    if (t10 >= 256) return 1;                               // fills the chip unsplit
    auto slices = [&](int64_t tiles) {
        int S = 1;
        while (S < 32 && tiles * S < 256 && K / (2 * S) >= 1024) S <<= 1;
        return S;
    };
    const int s10 = slices(t10);
    if (t10 * s10 >= 256) {
        *tile = TILE_256x256_FL8;
        return s10;
    }
    return t9 >= 256 ? 1 : slices(t9);
}

int migemm_splitk_splits(int dtype, int a_kmajor, int M, int N, int K)
{
    if (dtype != DT_F16 && dtype != DT_BF16) return 1;
    int tile;
    return splitk_choice(M, N, K, a_kmajor, &tile);
}

size_t migemm_splitk_workspace_bytes(int M, int N, int splits)
{
    if (M <= 0 || N <= 0 || splits <= 1) return 0;
    return (size_t)splits * M * N * sizeof(float);
}

int gemm_splitk_ex(int dtype, int a_kmajor, const uint16_t *A, const uint16_t *B, uint16_t *C,
                   int M, int N, int K, int splits, int tile, int group_m, int xcd_remap,
                   void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != DT_F16 && dtype != DT_BF16) return MIGEMM_ERR_CONFIG;
    if (splits < 0 || a_kmajor < 0 || a_kmajor > 1) return MIGEMM_ERR_CONFIG;
    int auto_tile;
    const int auto_S = splitk_choice(M, N, K, a_kmajor, &auto_tile);
    int S = splits ? splits : auto_S;
    // slices run on tiles 9, 10, 13; the automatic tile with a split is the
    // rule's (9 when the caller fixed the slice count and the rule splits not)
    const bool split_tile = tile == TILE_256x128_FL || tile == TILE_256x256_FL8 || tile == TILE_128x128_SK;
    if (S > 1 && tile != TILE_AUTO && !split_tile) return MIGEMM_ERR_CONFIG;
    GemmLaunch L;
    bool launch;
    int rc = plan_gemm(dtype, A, B, C, M, N, K, S > 1 && tile == TILE_AUTO ? (auto_S > 1 ? auto_tile : TILE_256x128_FL) : tile,
                       group_m, xcd_remap, L, launch, a_kmajor != 0);
    // slices need 16-byte rows of A and B (a slice's last 16-byte piece of a
    // row must not reach into the next row); without them: no split
    const bool wide = vec_width(A, a_kmajor ? K : M) == 8 && vec_width(B, K) == 8;
    if (S > 1 && (!wide || (tile == TILE_AUTO && rc == MIGEMM_ERR_CONFIG))) {
        S = 1;
        rc = plan_gemm(dtype, A, B, C, M, N, K, tile, group_m, xcd_remap, L, launch, a_kmajor != 0);
    }
    if (rc != MIGEMM_OK || !launch) return rc;
    const int ks = S > 1 ? (int)(((int64_t)K + S - 1) / S + 63) / 64 * 64 : K;
    const int S_eff = S > 1 ? (int)(((int64_t)K + ks - 1) / ks) : 1;
    if (S_eff > 1) {
        const size_t need = (size_t)S_eff * M * N * sizeof(float);
        if (!workspace) return MIGEMM_ERR_NULL;
        if ((uintptr_t)workspace % 16) return MIGEMM_ERR_ALIGN;
        if (workspace_bytes < need) return MIGEMM_ERR_SIZE;
        const size_t ab = (size_t)M * K * 2, bb = (size_t)K * N * 2, cb = (size_t)M * N * 2;
        if (overlaps(workspace, need, A, ab) || overlaps(workspace, need, B, bb) ||
            overlaps(workspace, need, C, cb))
            return MIGEMM_ERR_OVERLAP;
        L.splits = S_eff;
        L.ks = ks;
        L.part = (float *)workspace;
        hipError_t e = gemm_launch(L, (hipStream_t)stream);
        if (e == hipSuccess)
            e = splitk_reduce_launch(dtype, L.part, C, (int64_t)M * N, S_eff, (hipStream_t)stream);
        return finish(e, stream);
    }
    if (is_decode_tile(L.tile))
        return finish(decode_launch(L.tile, dtype, A, B, C, M, N, K, L.c_vec, (hipStream_t)stream), stream);
    return finish(launch_gemm_or_small(L, (hipStream_t)stream), stream);
}

int gemm_tn_q_ex(int qtype, const void *At, const void *B, uint16_t *C, int M, int N, int K,
                 float scale, int tile, int group_m, int xcd_remap, void *stream)
{
    if (!dt_is_8bit(qtype) || qtype > DT_I8) return MIGEMM_ERR_CONFIG;
    GemmLaunch L;
    bool launch;
    int rc = plan_gemm(qtype, (const uint16_t *)At, (const uint16_t *)B, C, M, N, K, tile, group_m,
                       xcd_remap, L, launch, true);
    if (rc != MIGEMM_OK || !launch) return rc;
    L.scale = scale;
    return finish(gemm_launch(L, (hipStream_t)stream), stream);
}

int gemm_tn_fp8_e4m3(const uint8_t *At, const uint8_t *B, uint16_t *C, int M, int N, int K,
                     float scale, void *stream)
{
    return gemm_tn_q_ex(DT_F8E4M3, At, B, C, M, N, K, scale, TILE_AUTO, 0, 1, stream);
}

int gemm_tn_fp8_e5m2(const uint8_t *At, const uint8_t *B, uint16_t *C, int M, int N, int K,
                     float scale, void *stream)
{
    return gemm_tn_q_ex(DT_F8E5M2, At, B, C, M, N, K, scale, TILE_AUTO, 0, 1, stream);
}

int gemm_tn_i8(const int8_t *At, const int8_t *B, uint16_t *C, int M, int N, int K, float scale,
               void *stream)
{
    return gemm_tn_q_ex(DT_I8, At, B, C, M, N, K, scale, TILE_AUTO, 0, 1, stream);
}

int gemm_tn_f16(const uint16_t *At, const uint16_t *B, uint16_t *C, int M, int N, int K, void *stream)
{
    return gemm_tn_ex(DT_F16, At, B, C, M, N, K, TILE_AUTO, 0, 1, stream);
}

int gemm_tn_bf16(const uint16_t *At, const uint16_t *B, uint16_t *C, int M, int N, int K, void *stream)
{
    return gemm_tn_ex(DT_BF16, At, B, C, M, N, K, TILE_AUTO, 0, 1, stream);
}

static int plan_for(int dtype, const uint16_t *A, const uint16_t *B, const uint16_t *C,
                    int M, int N, int K, int tile, int group_m, int xcd_remap,
                    migemm_gemm_plan *plan, bool a_kmajor)
{
    GemmLaunch L;
    bool launch;
    int rc = plan_gemm(dtype, A, B, C, M, N, K, tile, group_m, xcd_remap, L, launch, a_kmajor);
    if (rc != MIGEMM_OK || !plan) return rc;
    memset(plan, 0, sizeof(*plan));
    const TileShape &t = a_kmajor ? kTileShapesKmajorA[L.tile] : kTileShapes[L.tile];
    if (L.tile == TILE_SKINNY) {
        plan->tile_m = 32;                      // 4 waves x 2 groups of 4 rows
        plan->tile_n = N <= 4 ? 4 : 8;
        plan->tile_k = 128;
        plan->waves = 4;
        plan->group_m = 1;
        plan->xcd_remap = 0;
        plan->vec_a = L.vec_a;
        plan->vec_b = L.vec_b;
        plan->grid = launch ? L.grid : 0;
        plan->lds_bytes = 0;
        plan->tile = L.tile;
        plan->a_kmajor = 1;
        return rc;
    }
    if (L.tile == TILE_SMALL) {
        plan->tile_m = 32;
        plan->tile_n = 32;
        plan->tile_k = 32;
        plan->waves = small_waves(cdiv(M, 32) * cdiv(N, 32), K);   // splitting K between them
        plan->group_m = 1;
        plan->xcd_remap = 0;
        plan->vec_a = L.vec_a;
        plan->vec_b = L.vec_b;
        plan->grid = launch ? L.grid : 0;
        plan->lds_bytes = small_lds_bytes(cdiv(M, 32) * cdiv(N, 32), K);
        plan->tile = L.tile;
        plan->a_kmajor = a_kmajor ? 1 : 0;
        return rc;
    }
    if (L.tile == TILE_BATCH_ROWS || L.tile == TILE_BATCH_WIDE) {
        const bool wide = L.tile == TILE_BATCH_WIDE;
        plan->tile_m = batch_rows_per_workgroup(M);   // rows per workgroup
        plan->tile_n = wide ? batch_wide_tile_n(N) : batch_rows_tile_n(N);
        plan->tile_k = 64;
        plan->waves = wide ? 8 : 9;
        plan->group_m = 1;
        plan->xcd_remap = 0;
        plan->vec_a = L.vec_a;
        plan->vec_b = L.vec_b;
        plan->grid = launch ? L.grid : 0;
        plan->lds_bytes = wide ? batch_wide_lds_bytes(N) : batch_rows_lds_bytes(N);
        plan->tile = L.tile;
        plan->a_kmajor = 1;
        return rc;
    }
    if (L.tile == TILE_BATCH) {
        plan->tile_m = batch_tile_m(N);         // waves x 16 rows
        plan->tile_n = batch_tile_n(N);
        plan->tile_k = 128;
        plan->waves = batch_waves(N);
        plan->group_m = 1;
        plan->xcd_remap = 0;
        plan->vec_a = L.vec_a;
        plan->vec_b = L.vec_b;
        plan->grid = launch ? L.grid : 0;
        plan->lds_bytes = batch_lds_bytes(N);
        plan->tile = L.tile;
        plan->a_kmajor = 1;
        return rc;
    }
    plan->tile_m = t.bm;
    plan->tile_n = t.bn;
    plan->tile_k = dt_is_8bit(dtype) ? 2 * t.bk : t.bk;   // in elements
    plan->waves = t.waves;
    plan->group_m = L.group_m;
    plan->xcd_remap = L.num_xcd > 1;
    plan->vec_a = L.vec_a;
    plan->vec_b = L.vec_b;
    plan->grid = launch ? L.grid : 0;
    plan->lds_bytes = tile_lds_bytes(t, a_kmajor);
    plan->tile = L.tile;
    plan->a_kmajor = a_kmajor ? 1 : 0;
    return rc;
}

int migemm_gemm_plan_for(int dtype, const uint16_t *A, const uint16_t *B, const uint16_t *C,
                         int M, int N, int K, int tile, int group_m, int xcd_remap,
                         migemm_gemm_plan *plan)
{
    return plan_for(dtype, A, B, C, M, N, K, tile, group_m, xcd_remap, plan, false);
}

int migemm_gemm_tn_plan_for(int dtype, const uint16_t *At, const uint16_t *B, const uint16_t *C,
                            int M, int N, int K, int tile, int group_m, int xcd_remap,
                            migemm_gemm_plan *plan)
{
    return plan_for(dtype, At, B, C, M, N, K, tile, group_m, xcd_remap, plan, true);
}

// gemv_bf16_ex's argument checks and kernel choice (route codes as in
// migemm_gemv_plan_for).
static int plan_gemv(const uint16_t *W, const uint16_t *X, const uint16_t *Y, int M, int K, int n,
                     int rows_per_block, int &route)
{
    route = 0;
    if (!(rows_per_block == 0 || rows_per_block == 2 || rows_per_block == 4 ||
          rows_per_block == 8 || rows_per_block == 16 || rows_per_block == 32))
        return MIGEMM_ERR_CONFIG;
    if (M < 0 || K < 0 || n < 0) return MIGEMM_ERR_DIM;
    const size_t wbytes = (size_t)M * K * 2, xbytes = (size_t)n * K * 2, ybytes = (size_t)n * M * 2;
    if ((wbytes && !W) || (xbytes && !X) || (ybytes && !Y)) return MIGEMM_ERR_NULL;
    if (((uintptr_t)W | (uintptr_t)X | (uintptr_t)Y) & 1) return MIGEMM_ERR_ALIGN;
    if (overlaps(Y, ybytes, W, wbytes) || overlaps(Y, ybytes, X, xbytes)) return MIGEMM_ERR_OVERLAP;
    if (M == 0 || n == 0) return MIGEMM_OK;
    const bool vec = (K % 8 == 0 && (uintptr_t)W % 16 == 0 && (uintptr_t)X % 16 == 0);
    // Y = X W^T is gemm_tn with At = W, B = X, C = Y (all row-major): the
    // wide row-balanced kernel where batch_wide_auto says so, the
    // row-balanced kernel where batch_rows_auto does, else up to
    // kSkinnyAutoMax tokens on the 4x4x4 MFMA kernel, up to kBatchAutoMax on
    // the 16x16x32 batch kernel, more on the full-line 256x128 tile within
    // the GEMM's own size limits; everything else on the vector kernel
    const bool gemm_fits = M <= MIGEMM_MAX_MN && K <= MIGEMM_MAX_K;
    route = 1;
    if (rows_per_block == 0 && vec && batch_wide_auto(M, n))
        route = TILE_BATCH_WIDE;
    else if (rows_per_block == 0 && vec && batch_rows_auto(M, n))
        route = TILE_BATCH_ROWS;
    else if (rows_per_block == 0 && vec && n >= kSkinnyMinTokens)
        route = n <= kSkinnyAutoMax ? TILE_SKINNY
                : n <= kBatchAutoMax ? TILE_BATCH
                : gemm_fits ? TILE_256x128_FL : 1;
    return MIGEMM_OK;
}

int migemm_gemv_plan_for(const uint16_t *W, const uint16_t *X, const uint16_t *Y, int M, int K,
                         int n, int rows_per_block, int *route)
{
    int r;
    const int rc = plan_gemv(W, X, Y, M, K, n, rows_per_block, r);
    if (route) *route = r;
    return rc;
}

int gemv_bf16_ex(const uint16_t *W, const uint16_t *X, uint16_t *Y, int M, int K, int n,
                 int rows_per_block, void *stream)
{
    int route;
    const int rc = plan_gemv(W, X, Y, M, K, n, rows_per_block, route);
    if (rc != MIGEMM_OK || route == 0) return rc;
    if (route == TILE_256x128_FL)
        return gemm_tn_ex(DT_BF16, W, X, Y, M, n, K, TILE_256x128_FL, 0, 1, stream);
    if (is_decode_tile(route))
        return finish(decode_launch(route, DT_BF16, W, X, Y, M, n, K,
                                    (M % 4 == 0 && (uintptr_t)Y % 8 == 0) ? 1 : 0, (hipStream_t)stream),
                      stream);
    const bool vec = (K % 8 == 0 && (uintptr_t)W % 16 == 0 && (uintptr_t)X % 16 == 0);

    GemvLaunch L{};
    L.W = W;
    L.M = M;
    L.K = K;
    L.rows_per_block = rows_per_block ? rows_per_block : 2;
    L.vec = vec ? 8 : 1;
    L.grid = cdiv(M, L.rows_per_block);
    // Token blocks of 16, 8, 4, 2, 1: each launch streams W once.
    int done = 0;
    hipError_t e = hipSuccess;
    while (done < n && e == hipSuccess) {
        int left = n - done;
        int nt = left >= 16 ? 16 : left >= 8 ? 8 : left >= 4 ? 4 : left >= 2 ? 2 : 1;
        L.n = nt;
        L.X = X + (size_t)done * K;
        L.Y = Y + (size_t)done * M;
        e = gemv_launch(L, (hipStream_t)stream);
        done += nt;
    }
    return finish(e, stream);
}

int gemv_bf16(const uint16_t *W, const uint16_t *X, uint16_t *Y, int M, int K, int n, void *stream)
{
    return gemv_bf16_ex(W, X, Y, M, K, n, 0, stream);
}

int migemm_attention_segments(int B, int Hq, int Hkv, int max_seq_len)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return 1;
    // Double S while the segment workgroups still fit in one round of
    // residency (2 per CU at the segment kernel's register use) and every
    // segment keeps at least 128 tokens; measured best on the
    // 16 Q / 4 KV / head-dim-256 shape for 1 x 8K .. 32K and 8 x 8K,
    // 32 x 4K tokens.
    const int64_t per_s = (int64_t)B * Hkv * ((Hq / Hkv + 3) / 4);   // workgroups per segment
    const int64_t resident = 2 * 256;
    int S = 1;
    while (S < 1024 && per_s * 2 * S <= resident && (max_seq_len + 2 * S - 1) / (2 * S) >= 128)
        S <<= 1;
    return S;
}

size_t migemm_attention_workspace_bytes(int B, int Hq, int D, int num_segments)
{
    if (B < 0 || Hq < 0 || D < 0 || num_segments < 1) return 0;
    return attention_workspace_bytes(B, Hq, D, num_segments);
}

}  // extern "C"

namespace {

// attention_decode_bf16's checks of everything but the workspace, before any
// HIP call.  On MIGEMM_OK with *run set, S is the segment count and need the
// workspace bytes the call uses.
int attention_plan(const uint16_t *Q, const uint16_t *Kc, const uint16_t *Vc,
                   const int32_t *block_table, const int32_t *seq_lens, const uint16_t *Out,
                   int B, int Hq, int Hkv, int D, int block_size, int max_blocks, int num_blocks,
                   int max_seq_len, int num_segments, bool &run, int &S, size_t &need)
{
    run = false;
    if (B < 0 || Hq < 0 || Hkv < 0 || D < 0 || block_size < 0 || max_blocks < 0 ||
        num_blocks < 0 || max_seq_len < 0 || num_segments < 0)
        return MIGEMM_ERR_DIM;
    if (B == 0 || Hq == 0) return MIGEMM_OK;
    if (Hkv == 0 || Hq % Hkv != 0 || block_size == 0 || max_blocks == 0 || num_blocks == 0)
        return MIGEMM_ERR_DIM;
    const int G = Hq / Hkv;
    if (!(D == 64 || D == 128 || D == 256) || !(G == 1 || G == 2 || G == 4 || G == 8) ||
        num_segments > 1024)
        return MIGEMM_ERR_CONFIG;
    // grid (kv heads, segments, sequences); token positions (plus a few
    // steps of look-ahead) held in int
    if (B > 65535 || Hkv > 65535 || (int64_t)max_blocks * block_size > (1 << 30))
        return MIGEMM_ERR_SIZE;
    if (!Q || !Kc || !Vc || !block_table || !seq_lens || !Out) return MIGEMM_ERR_NULL;
    if (((uintptr_t)Q | (uintptr_t)Kc | (uintptr_t)Vc) % 16 ||
        ((uintptr_t)block_table | (uintptr_t)seq_lens) % 4 || (uintptr_t)Out % 2)
        return MIGEMM_ERR_ALIGN;
    S = num_segments ? num_segments : migemm_attention_segments(B, Hq, Hkv, max_seq_len);
    need = attention_workspace_bytes(B, Hq, D, S);
    const size_t qb = (size_t)B * Hq * D * 2;
    const size_t cb = (size_t)num_blocks * block_size * Hkv * D * 2;
    if (overlaps(Out, qb, Q, qb) || overlaps(Out, qb, Kc, cb) || overlaps(Out, qb, Vc, cb) ||
        overlaps(Out, qb, block_table, (size_t)B * max_blocks * 4) ||
        overlaps(Out, qb, seq_lens, (size_t)B * 4))
        return MIGEMM_ERR_OVERLAP;
    run = true;
    return MIGEMM_OK;
}

// The segment partials of attention_decode_bf16_noalloc: a file-scope device
// array in place of a caller workspace.  In host code its name is only a
// stand-in; the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[MIGEMM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (a HIP error code, or
// MIGEMM_ERR_CONFIG past kMaxDevices devices).
int scratch_address(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return MIGEMM_ERR_CONFIG;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        if (!p) return (int)hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MIGEMM_OK;
}

}  // namespace

extern "C" {

int attention_decode_bf16(const uint16_t *Q, const uint16_t *Kc, const uint16_t *Vc,
                          const int32_t *block_table, const int32_t *seq_lens, uint16_t *Out,
                          int B, int Hq, int Hkv, int D, int block_size, int max_blocks,
                          int num_blocks, float scale, int max_seq_len, int num_segments,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    bool run;
    int S = 0;
    size_t need = 0;
    int rc = attention_plan(Q, Kc, Vc, block_table, seq_lens, Out, B, Hq, Hkv, D, block_size,
                            max_blocks, num_blocks, max_seq_len, num_segments, run, S, need);
    if (rc != MIGEMM_OK || !run) return rc;
    if (!workspace) return MIGEMM_ERR_NULL;
    if ((uintptr_t)workspace % 16) return MIGEMM_ERR_ALIGN;
    if (workspace_bytes < need) return MIGEMM_ERR_SIZE;
    const size_t qb = (size_t)B * Hq * D * 2;
    const size_t cb = (size_t)num_blocks * block_size * Hkv * D * 2;
    if (overlaps(Out, qb, workspace, need) || overlaps(workspace, need, Q, qb) ||
        overlaps(workspace, need, Kc, cb) || overlaps(workspace, need, Vc, cb) ||
        overlaps(workspace, need, block_table, (size_t)B * max_blocks * 4) ||
        overlaps(workspace, need, seq_lens, (size_t)B * 4))
        return MIGEMM_ERR_OVERLAP;
    AttentionLaunch A{Q, Kc, Vc, block_table, seq_lens, Out, B, Hq, Hkv, D, block_size,
                      max_blocks, num_blocks, scale, S, workspace};
    return finish(attention_launch(A, (hipStream_t)stream), stream);
}

int attention_decode_bf16_noalloc(const uint16_t *Q, const uint16_t *Kc, const uint16_t *Vc,
                                  const int32_t *block_table, const int32_t *seq_lens,
                                  uint16_t *Out, int B, int Hq, int Hkv, int D, int block_size,
                                  int max_blocks, int num_blocks, float scale, int max_seq_len,
                                  int num_segments, void *stream)
{
    bool run;
    int S = 0;
    size_t need = 0;
    int rc = attention_plan(Q, Kc, Vc, block_table, seq_lens, Out, B, Hq, Hkv, D, block_size,
                            max_blocks, num_blocks, max_seq_len, num_segments, run, S, need);
    if (rc != MIGEMM_OK || !run) return rc;
    if (need > (size_t)MIGEMM_NOALLOC_SCRATCH_BYTES) return MIGEMM_ERR_SIZE;
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != MIGEMM_OK) return rc;
    // every segment row of the partials is written before the merge reads
    // it, so nothing left by an earlier call is read and nothing is cleared
    AttentionLaunch A{Q, Kc, Vc, block_table, seq_lens, Out, B, Hq, Hkv, D, block_size,
                      max_blocks, num_blocks, scale, S, ws};
    return finish(attention_launch(A, (hipStream_t)stream), stream);
}

int migemm_tile_coord(int64_t wg, int64_t num_pid_m, int64_t num_pid_n, int64_t group_m,
                      int64_t num_xcd, int64_t *pid_m, int64_t *pid_n)
{
    if (num_pid_m <= 0 || num_pid_n <= 0 || group_m <= 0 || num_xcd <= 0 || wg < 0 ||
        wg >= num_pid_m * num_pid_n || !pid_m || !pid_n)
        return MIGEMM_ERR_DIM;
    tile_coord<int64_t>(wg, num_pid_m, num_pid_n, group_m, num_xcd, *pid_m, *pid_n);
    return MIGEMM_OK;
}

const char *migemm_strerror(int code)
{
    switch (code) {
    case MIGEMM_OK: return "ok";
    case MIGEMM_ERR_DIM: return "negative dimension";
    case MIGEMM_ERR_NULL: return "null pointer with a non-zero extent";
    case MIGEMM_ERR_OVERLAP: return "output overlaps an input";
    case MIGEMM_ERR_ALIGN: return "pointer or size not aligned as the entry point requires";
    case MIGEMM_ERR_CONFIG: return "configuration not offered";
    case MIGEMM_ERR_SIZE: return "dimension beyond the supported range";
    }
    return code > 0 ? "HIP runtime error (code is a hipError_t)" : "unknown error";
}

int migemm_abi_version(void) { return 3; }

int migemm_hbm_read(const void *buf, size_t bytes, uint32_t *sink, void *stream)
{
    if ((bytes && !buf) || !sink) return MIGEMM_ERR_NULL;
    if ((uintptr_t)buf % 16 || bytes % 16) return MIGEMM_ERR_ALIGN;
    return finish(hbm_read_launch(buf, bytes, sink, (hipStream_t)stream), stream);
}

int migemm_hbm_read_sink_words(void) { return hbm_read_sink_words(); }

int migemm_clock_probe(uint64_t *out, int blocks, int iters, void *stream)
{
    if (blocks < 0 || iters < 0) return MIGEMM_ERR_DIM;
    if (blocks == 0) return MIGEMM_OK;
    if (blocks > 65535) return MIGEMM_ERR_SIZE;
    if (!out) return MIGEMM_ERR_NULL;
    if ((uintptr_t)out % 8) return MIGEMM_ERR_ALIGN;
    return finish(clock_probe_launch(out, blocks, iters, (hipStream_t)stream), stream);
}

}  // extern "C"
