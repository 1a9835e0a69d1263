// kernels.hpp -- launch descriptors shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace migemm {

enum GemmTile {
    TILE_AUTO = 0,
    TILE_256x256 = 1,           // 256x256, 4 waves as 2x2 (128x128 per wave), 4 stages
    TILE_256x128 = 2,           // 256x128, 4 waves as 2x2, 5 stages
    TILE_128x128 = 3,           // 128x128, 4 waves as 2x2, 4 stages, 2 workgroups per CU
    TILE_256x256_S5 = 4,        // tile 1 with 5 stages (all 160 KiB of LDS)
    TILE_256x256_W41 = 5,       // 256x256, 4 waves stacked along M (64x256 per wave), 4 stages
    TILE_256x256_S3 = 6,        // tile 1 with 3 stages
    TILE_256x256_FL = 7,        // 256x256, waves along M, full-line B ring (A 4 x 32 k, B 3 x 64 k)
    TILE_256x256_FL22 = 8,      // as 7 with 4 waves as 2x2
    TILE_256x128_FL = 9,        // 256x128, waves along M, full-line B ring (A 4 x 32 k, B 4 x 64 k)
    TILE_256x256_FL8 = 10,      // as 7 with 8 waves (4 x 2, two per SIMD), 64x128 per wave
    TILE_64x32_SK = 11,         // skinny: 64x32, 2 waves along M, full-line rings, 4 WG per CU
    TILE_64x64_SK = 12,         // skinny: 64x64, 2 waves along M, 3 WG per CU
    TILE_128x128_SK = 13,       // 128x128, 4 waves as 2x2, full-line rings
    TILE_SKINNY = 14,           // few columns: W straight into 4x4x4 MFMA registers (skinny.hip)
    TILE_BATCH = 15,            // 9..128 columns: W into 16x16x32 MFMA registers, X in LDS (batch.hip)
    TILE_256x256_PP = 16,       // as 10, m-major A, ping-pong: the two waves of a SIMD alternate MFMA and memory phases
    TILE_256x128_F8W = 17,      // FP8 only, k-major A: 256x128, 8 waves of 64x64, whole 64-unit steps on the 16x16x128 MFMA
    TILE_BATCH_ROWS = 18,       // up to 256 columns: W's rows spread evenly, 9 waves of 16 rows per workgroup (batch.hip)
    TILE_BATCH_WIDE = 19,       // up to 256 columns: W's rows spread evenly, 8 waves of 7 or 2 row tiles x a quarter of the columns (wide.hip)
    TILE_SMALL = 20,            // few output tiles: 32x32 per workgroup, 4 waves splitting K, no LDS staging (small.hip)
    TILE_COUNT
};

// stages: ring stages of 32 k (A and B together, or A alone when b_stages
// > 0); b_stages: B ring stages of 64 k in the full-line variants.
struct TileShape {
    int bm, bn, bk, stages, waves, b_stages;
};

// Indexed by GemmTile (entry 0 unused).  Every tile steps K by 32.
constexpr TileShape kTileShapes[TILE_COUNT] = {
    {0, 0, 0, 0, 0, 0},
    {256, 256, 32, 4, 4, 0},
    {256, 128, 32, 5, 4, 0},
    {128, 128, 32, 4, 4, 0},
    {256, 256, 32, 5, 4, 0},
    {256, 256, 32, 4, 4, 0},
    {256, 256, 32, 3, 4, 0},
    {256, 256, 32, 4, 4, 3},
    {256, 256, 32, 4, 4, 3},
    {256, 128, 32, 4, 4, 4},
    {256, 256, 32, 4, 8, 3},
    {64, 32, 32, 4, 2, 2},
    {64, 64, 32, 4, 2, 2},
    {128, 128, 32, 4, 4, 3},
    {32, 64, 32, 0, 4, 0},
    {64, 128, 128, 0, 4, 0},
    {256, 256, 32, 4, 8, 3},
    {256, 128, 32, 3, 8, 3},
    {144, 256, 64, 0, 9, 0},
    {144, 256, 64, 0, 8, 0},
    {32, 32, 32, 0, 4, 0},
};

// The full-line tiles with A k-major: stages = A ring stages of 64 k.
constexpr TileShape kTileShapesKmajorA[TILE_COUNT] = {
    {0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0},
    {0, 0, 0, 0, 0, 0},
    {256, 256, 32, 2, 4, 3},
    {256, 256, 32, 2, 4, 3},
    {256, 128, 32, 3, 4, 4},
    {256, 256, 32, 2, 8, 3},
    {64, 32, 32, 4, 2, 2},
    {64, 64, 32, 4, 2, 2},
    {128, 128, 32, 4, 4, 3},
    {32, 64, 32, 0, 4, 0},
    {64, 128, 128, 0, 4, 0},
    {0, 0, 0, 0, 0, 0},
    {256, 128, 32, 3, 8, 3},
    {144, 256, 64, 0, 9, 0},
    {144, 256, 64, 0, 8, 0},
    {32, 32, 32, 0, 4, 0},
};

constexpr int tile_lds_bytes(const TileShape &t, bool a_kmajor = false)
{
    return a_kmajor ? (t.stages * t.bm + t.b_stages * t.bn) * 2 * t.bk * 2
           : t.b_stages ? t.stages * t.bk * t.bm * 2 + t.b_stages * 2 * t.bk * t.bn * 2
                        : t.stages * t.bk * (t.bm + t.bn) * 2;
}

struct GemmLaunch {
    int dtype;                    // DT_F16 or DT_BF16
    int tile;                     // GemmTile (never TILE_AUTO here)
    const uint16_t *A, *B;
    uint16_t *C;
    int M, N, K;
    int num_pid_m, num_pid_n;
    int group_m, num_xcd;
    int vec_a, vec_b;             // elements per global->LDS load (8, 2 or 1)
    int c_vec;                    // 1: 8-byte stores of 4 rows are aligned
    int a_kmajor;                 // 1: A(m,k) = A[k + m*K] (full-line tiles only)
    int64_t grid;
    float scale;                  // 8-bit types: C = BF16(scale x accumulator)
    int splits;                   // > 1: split-K over `splits` k slices of ks (full-line tiles)
    int ks;                       // slice length, a multiple of 64 (2-byte units)
    float *part;                  // split-K FP32 partials [splits][N][M]
    uint64_t *clocks;             // measurement (full-line tiles, unsplit): per workgroup, shader
                                  // clocks and 10 ns real-time ticks it ran for; nullptr = off
    int in_range;                 // 1: every tile load lies inside A and B (16-byte rows, M and N
                                  // multiples of the tile, K of 64): the full-line tiles (9-13, 16,
                                  // 17) then load through global addresses (no range check)
    int edge_gl;                  // 1: not in range, but 16-byte rows and (K & ~7) a multiple of
                                  // 64: the full-line tiles (9-13, 16, 17) load through global
                                  // addresses, lanes past M or N re-reading the tile's first row
                                  // or column
};

// Sum of split-K partials: C = round(sum_z part[z][n][m]) (gemm.hip).
hipError_t splitk_reduce_launch(int dtype, const float *part, uint16_t *C, int64_t count,
                                int splits, hipStream_t stream);

hipError_t gemm_launch(const GemmLaunch &L, hipStream_t stream);
// The small-problem kernel (small.hip): automatic while the 32x32 output
// tiles number at most kSmallMaxTiles (measured, FP16: 512^3 4.2 us against
// 7.9 on the 64x32 tile, 512x512x4096 21.5 against 54.6, 2048x256x512 6.2
// against 8.2, 768^3 (576 tiles) 10.3 against 12.0 on 64x64; at 1024 tiles
// (1024^3) it loses, 17.1 against 15.3).
constexpr int kSmallMaxTiles = 768;
// Waves per tile, splitting K: 8 for at most 256 tiles with K >= 1024, else 4
// (measured, FP16: 512x512xK 5.9 / 9.4 / 19.0 / 66.7 us at K = 1024 / 2048 /
// 4096 / 16384 against 6.3 / 10.2 / 21.7 / 79.8 with 4; 16 waves no better;
// with more tiles the extra waves only wait: 768x768x4096 47.5 against 45.2).
constexpr int small_waves(int64_t tiles, int K) { return tiles <= 256 && K >= 1024 ? 8 : 4; }
constexpr int small_lds_bytes(int64_t tiles, int K) { return small_waves(tiles, K) * 4 * 64 * 16; }
hipError_t small_launch(const GemmLaunch &L, hipStream_t stream);

struct GemvLaunch {
    const uint16_t *W, *X;
    uint16_t *Y;
    int M, K, n;                  // n: tokens in this launch (1, 2, 4, 8 or 16)
    int rows_per_block;           // 2, 4, 8, 16 or 32
    int vec;                      // 8: 16-byte loads; 1: element loads
    int64_t grid;
};

hipError_t gemv_launch(const GemvLaunch &L, hipStream_t stream);

// Y = X W^T on MFMA for n <= kSkinnyMaxTokens token rows (skinny.hip).
constexpr int kSkinnyMaxTokens = 8;
constexpr int kSkinnyMinTokens = 3;    // the automatic GEMV switches to MFMA from here
// Y = X W^T on the 16x16x32 MFMA with X staged in LDS (batch.hip), for up
// to kBatchMaxTokens tokens.
constexpr int kBatchMaxTokens = 128;
// Automatic choice (measured on W 34816 x 5120): the 4x4x4 kernel up to 4
// tokens, the batch kernel up to 64 (its 128-token block holds 86 KB of LDS
// per workgroup, too little residency to keep W streaming), then the GEMM's
// 256x128 tile.
constexpr int kSkinnyAutoMax = 4;
constexpr int kBatchAutoMax = 64;
struct SkinnyLaunch {
    int dtype;
    const uint16_t *W, *X;        // W row-major [M, K], X row-major [n, K]
    uint16_t *Y;                  // Y row-major [n, M]
    int M, K, n;
    int y_vec;                    // 1: 8-byte stores of 4 consecutive rows are aligned
};

hipError_t skinny_launch(const SkinnyLaunch &L, hipStream_t stream);
hipError_t batch_launch(const SkinnyLaunch &L, hipStream_t stream);
// Row-balanced batch kernel (batch.hip): W's rows spread evenly over the
// workgroups, 9 waves of 16 rows each, up to kBatchRowsMaxTokens tokens.
constexpr int kBatchRowsMaxTokens = 256;
// Automatic choice for 2 .. 128 tokens (measured on W 34816 x 5120, 16384 x
// 4096 and 4096 x 4096): the row-balanced kernel once its workgroups hold
// 64 rows or more (M >= 16384; 54 us against 58-65 us for 2-16 tokens and 64
// against 92 us for 64 tokens on 34816 x 5120), and from 33 tokens on for any
// M (4096 x 4096, 64 tokens: 20 against 28 us).  Above 128 tokens the GEMM's
// tiles do as well or better.
constexpr int kBatchRowsAutoMax = 128;
constexpr int kBatchRowsAutoMinM = 16384;
constexpr int kBatchRowsAutoAnyM = 33;
constexpr bool batch_rows_auto(int M, int n)
{
    return n >= 2 && n <= kBatchRowsAutoMax && (M >= kBatchRowsAutoMinM || n >= kBatchRowsAutoAnyM);
}
hipError_t batch_rows_launch(const SkinnyLaunch &L, hipStream_t stream);
int batch_rows_per_workgroup(int M);
// token columns of one row-balanced workgroup (16, 32, 64, 128, 256) and its
// LDS: two staged 64-k chunks of X (token rows of 144 bytes) and the 9
// waves' 2 KB areas that re-lay W out
constexpr int batch_rows_tile_n(int n) { return n <= 16 ? 16 : n <= 32 ? 32 : n <= 64 ? 64 : n <= 128 ? 128 : 256; }
constexpr int batch_rows_lds_bytes(int n) { return 2 * batch_rows_tile_n(n) * 144 + 9 * 2048; }
// Row-balanced wide kernel (wide.hip): the same rows per workgroup, 8 waves
// in two row groups (5 and 4 tiles of 16) times four column groups, both
// operands staged in LDS by direct loads; 128- or 256-column blocks.
constexpr int kBatchWideMaxTokens = 256;
hipError_t batch_wide_launch(const SkinnyLaunch &L, hipStream_t stream);
constexpr int batch_wide_tile_n(int n) { return n <= 128 ? 128 : 256; }
// Automatic choice for 65 .. 256 tokens once the workgroups hold more than
// 120 rows (M > 30720): on W 34816 x 5120, 73 us for 128 tokens (the
// row-balanced kernel 113-122 us, the GEMM's 256x128 tile 115 us) and
// 118-136 us for 256 (the GEMM tiles 158-203 us).  With fewer rows its
// fixed 9 row tiles waste work (16384 x 4096, 128 tokens: 47 us against 40
// for the row-balanced kernel).
constexpr int kBatchWideAutoMinM = 30721;
constexpr bool batch_wide_auto(int M, int n) { return n >= 65 && n <= kBatchWideMaxTokens && M >= kBatchWideAutoMinM; }
// its LDS: 4 ring stages of 9 + 8 tiles of 2 KiB (128 columns) or 3 of
// 9 + 16, and a 1 KiB sink
constexpr int batch_wide_lds_bytes(int n)
{
    return n <= 128 ? 4 * (9 + 8) * 2048 + 1024 : 3 * (9 + 16) * 2048 + 1024;
}
// the kernels above that take Y = X W^T directly (gemm_tn with At = W, B = X)
constexpr bool is_decode_tile(int t)
{
    return t == TILE_SKINNY || t == TILE_BATCH || t == TILE_BATCH_ROWS || t == TILE_BATCH_WIDE;
}
// token columns of one batch-kernel workgroup for n tokens (16, 32, 64, 128)
constexpr int batch_tile_n(int n) { return n <= 16 ? 16 : n <= 32 ? 32 : n <= 64 ? 64 : 128; }
// its waves (16 rows of W each): 2 for one 16-token block (finer workgroups
// balance the CUs better; measured 65 against 68 us at 16 tokens), else 4
constexpr int batch_waves(int n) { return batch_tile_n(n) == 16 ? 2 : 4; }
constexpr int batch_tile_m(int n) { return 16 * batch_waves(n); }
// its LDS bytes: two staged chunks of tile_n token rows of 272 bytes, and
// the waves' 4 KB areas that re-lay W out
constexpr int batch_lds_bytes(int n) { return 2 * batch_tile_n(n) * (128 * 2 + 16) + batch_waves(n) * 4096; }

// Decode attention over a paged KV cache, split into S segments (attention.hip).
struct AttentionLaunch {
    const uint16_t *Q, *Kc, *Vc;          // Q [B][Hq][D]; caches [block][token][Hkv][D]
    const int32_t *block_table, *seq_lens; // [B][max_blocks], [B]
    uint16_t *Out;                        // [B][Hq][D]
    int B, Hq, Hkv, D, block_size, max_blocks, num_blocks;
    float scale;
    int S;                                // segments per (sequence, kv head)
    void *workspace;                      // attention_workspace_bytes(B, Hq, D, S)
};

size_t attention_workspace_bytes(int B, int Hq, int D, int S);
hipError_t attention_launch(const AttentionLaunch &A, hipStream_t stream);

hipError_t hbm_read_launch(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream);
int hbm_read_sink_words();
hipError_t clock_probe_launch(uint64_t *out, int blocks, int iters, hipStream_t stream);

}  // namespace migemm
