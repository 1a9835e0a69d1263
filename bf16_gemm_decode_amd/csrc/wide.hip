// wide.hip -- Y = X W^T for a decode batch of 65 .. 256 token rows on the
// 16x16x32 MFMA, W streamed from HBM once and both operands staged in LDS.
//
// The product of the DCU decode page (forum.sourcefind.cn db785961), section
// 6.1: W row-major [M, K], X row-major [n, K], Y row-major [n, M], FP32
// accumulation, one rounding.  At a few hundred tokens the MFMA work per W
// byte is no longer small (256 tokens: 256 FLOP per byte of W), so the
// operands must be reused from registers: a kernel that reads one LDS
// operand per MFMA (one wave per 16 rows of W, every token) runs at the LDS
// port's rate, not the matrix cores'.
//
//  * W's rows are cut evenly over the workgroups as in the row-balanced
//    kernel (R = ceil(M / 256) rounded up to 8, at most 144: 136 rows of
//    34816), so every CU streams the same share of W once.
//  * A workgroup is 8 waves, two per SIMD, in two row groups (waves 0-3 the
//    first 7 row tiles of 16, waves 4-7 the other 2) and four token groups
//    (TW = NT/4 tiles of 16 each); the two waves of a SIMD are one of each
//    row group, so every SIMD multiplies all 9 row tiles.  Waves 4-7 also
//    issue every load of the ring: a load waits at issue while the memory
//    pipe is backed up, and that stall then holds up only the wave with the
//    smaller share of MFMAs while the other keeps the SIMD's matrix core
//    busy (measured 99-109 against 111-127 us at 256 tokens with 5 + 4 row
//    tiles and every wave loading).  Per 32-k step a wave reads its 7 (2) A
//    operands and TW B operands from LDS for 7 TW (2 TW) MFMAs: 144 KiB of
//    LDS reads per 64-k chunk at 256 tokens, against 288 KiB when every
//    wave reads one operand per MFMA (one wave per 16 rows, every token).
//    The accumulators stay in AGPRs over all of K.
//  * K goes in chunks of 64 (one 128-byte line per row).  Both W's rows and
//    X's token rows reach LDS by direct buffer loads (buffer_load ... lds),
//    each instruction one 1 KiB half of a 16-row tile: 8 whole 128-byte
//    lines (loads of 64 bytes per row stream W at little more than half
//    the rate), with the lanes permuted so that the 64 16-byte pieces land
//    in the order the operand reads want (below).  W's loads carry the
//    non-temporal hint (each line is read once), which leaves L2 to the
//    token rows every workgroup re-reads.  The 2 * (RT + NT) loads of a
//    chunk go round-robin over the four loading waves, padded to a multiple
//    of 4 with loads of nothing, so every loading wave issues the same count
//    and one counter wait plus one barrier per chunk order the ring.
//  * ST ring stages.  The wait and barrier for chunk c + 1 sit between the
//    two 32-k steps of chunk c; the barrier also closes every wave's reads
//    of chunk c, so chunk c + ST is loaded into that stage right after it.
//    Step 1's operand reads overlap step 0's MFMAs and the next chunk's
//    step-0 reads overlap step 1's.
//
// LDS layout of one 16-row tile (2 KiB; the same for W rows and token rows):
// tile row r = 8b + q (b the half, q < 8) sits in LDS row P = 8b + (q ^ b)
// with its 16-byte piece p (k 8p .. 8p+7 of the chunk) at slot p ^ q, i.e.
// at byte 128 P + 16 (p ^ q).  An operand read of step j has lane (g, r)
// (g = lane / 16, r = lane % 16) fetch piece 4j + g of tile row r; the 16
// lanes of one g then hit 16 distinct 16-byte bank groups (the q ^ b
// exchange makes the two halves use complementary groups), so the read runs
// without bank conflicts.  The direct load of half b has lane s write slot
// s, so lane s fetches tile row 8b + ((s / 8) ^ b), piece (s % 8) ^ that
// row's q.  A and B operands pair the same piece of the same lane, so both
// sides agree on which k each lane holds.
//
// Rows past the workgroup's range (or past M) and tokens past n read as zero
// through the buffer descriptors' range and are never stored; pieces past K
// are given an out-of-range offset and read as zero.
#include <type_traits>

#include "common.hpp"
#include "dma.hpp"
#include "kernels.hpp"

namespace migemm {

namespace {

constexpr int kWideWaves = 8;
constexpr int kWideRT = 9;             // row tiles per workgroup (144 rows at most)
constexpr int kWideRT0 = 7;            // row tiles of waves 0-3; waves 4-7 take the other 2
constexpr int kWideLoaders = 4;        // waves 4-7 issue the ring's loads
constexpr int kWideKC = 64;            // k per chunk
constexpr int kTileBytes = 16 * kWideKC * 2;

// acc += a * b on one 16x16x32 block, the accumulator pinned to AGPRs (as
// inline assembly: with the builtin the compiler rotates the accumulator
// blocks through VGPR copies).  The compiler does not see the result
// latency, so nothing but another MFMA reads an accumulator before
// mfma_settle().
template <int DT>
__device__ inline void mfma_acc(f32x4 &acc, u32x4 a, u32x4 b)
{
    if constexpr (DT == DT_F16)
        asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// More wait states than the longest MFMA write-to-read requirement.
__device__ inline void mfma_settle()
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Byte offset of tile row r's piece p inside its 2 KiB tile.
__device__ inline int tile_slot(int r, int p)
{
    const int b = r >> 3, q = r & 7;
    return 128 * (8 * b + (q ^ b)) + 16 * (p ^ q);
}

}  // namespace

template <int DT, int NT, int ST, int RT0, int LW>
__global__ void __launch_bounds__(64 * kWideWaves)
batch_wide_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ X,
                  uint16_t *__restrict__ Y, int M, int K, int n, int R, int y_vec)
{
    constexpr int TW = NT / 4;                            // token tiles per wave
    constexpr int NLOAD = 2 * (kWideRT + NT);             // 1 KiB loads per chunk
    constexpr int Q = (NLOAD + LW - 1) / LW;              // per loading wave, padded
    static_assert(LW == 4 || LW == 8, "loads by all waves or by waves 4-7");
    static_assert(RT0 >= 1 && RT0 < kWideRT, "two row groups");
    constexpr int STAGE = (kWideRT + NT) * kTileBytes;
    constexpr int B_OFF = kWideRT * kTileBytes;           // B tiles after the A tiles
    static_assert(NT % 4 == 0 && ST >= 3, "token tiles per wave, ring depth");
    static_assert(Q * (ST - 2) < 64, "vmcnt range");
    // ST stages and a 1 KiB sink for the padding loads (they write zeros)
    __shared__ __attribute__((aligned(1024))) unsigned char smem[ST * STAGE + 1024];

    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int g = lane >> 4, r16 = lane & 15;
    const int rbeg = blockIdx.x * R;
    const int rows = min(R, M - rbeg);
    const int tok0 = blockIdx.y * (NT * 16);
    const int toks = min(NT * 16, n - tok0);
    const int chunks = (K + kWideKC - 1) / kWideKC;
    const size_t row_bytes = (size_t)K * 2;

    // descriptors over this workgroup's rows of W and its tokens of X:
    // anything past them reads as zero
    const u32x4 dw = make_desc(W + (size_t)rbeg * K, clamp_records((int64_t)rows * K * 2));
    const u32x4 dx = make_desc(X + (size_t)tok0 * K, clamp_records((int64_t)toks * K * 2));
    const uint32_t lds0 = (uint32_t)(uintptr_t)(MIGEMM_LDS unsigned char *)smem;

    // this lane's part of each of the wave's Q loads per chunk: the source
    // row's byte offset plus the piece's, and the piece's first k
    uint32_t src[Q];
    int pk[Q];
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        const int id = (wave - (kWideWaves - LW)) + LW * i;  // load id within the chunk
        const int tile = (id >> 1) < kWideRT ? (id >> 1) : (id >> 1) - kWideRT;
        const int b = id & 1;
        const int q = (lane >> 3) ^ b;                    // tile row 8b + q
        const int p = (lane & 7) ^ q;
        src[i] = (uint32_t)((tile * 16 + 8 * b + q) * row_bytes) + 16 * p;
        pk[i] = 8 * p;
        if (id >= NLOAD) pk[i] = K;                       // padding: never in range
    }
    auto issue = [&](int c) {
        if (wave < kWideWaves - LW) return;               // not a loading wave
        const uint32_t base = lds0 + (uint32_t)((c % ST) * STAGE);
#pragma unroll
        for (int i = 0; i < Q; ++i) {
            const int id = (wave - (kWideWaves - LW)) + LW * i;  // wave-uniform
            const bool is_a = (id >> 1) < kWideRT;
            const uint32_t dst = id >= NLOAD ? lds0 + ST * STAGE
                                 : base + (is_a ? 0 : B_OFF) +
                                       (uint32_t)(((is_a ? (id >> 1) : (id >> 1) - kWideRT) * 2 + (id & 1)) * 1024);
            const int k = c * kWideKC + pk[i];
            const uint32_t off = k < K ? src[i] + (uint32_t)(c * kWideKC * 2) : kOutOfRange;
            if (is_a)
                dma16_to_lds_nt(dw, uniform((int)dst), off);    // W: read once
            else
                dma_to_lds<16>(dx, uniform((int)dst), off);
        }
    };

    // operand read offsets inside a tile for the two 32-k steps
    const int rd0 = tile_slot(r16, g), rd1 = tile_slot(r16, 4 + g);
    const int tg = wave & 3;                              // token group

#pragma unroll
    for (int s = 0; s < ST - 1; ++s) issue(s);

    // the wave's row tiles: R0 .. R0 + RTW - 1 (one copy of the loop per
    // row group, so both keep exact operand counts)
    auto run = [&](auto r0_c, auto rtw_c) {
        constexpr int R0 = decltype(r0_c)::value, RTW = decltype(rtw_c)::value;
        f32x4 acc[RTW][TW];
#pragma unroll
        for (int r = 0; r < RTW; ++r)
#pragma unroll
            for (int t = 0; t < TW; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

        // step j's operands of chunk c from its stage, and their MFMAs
        auto operands = [&](int c, int j, u32x4 (&a)[RTW], u32x4 (&b)[TW]) {
            const MIGEMM_LDS unsigned char *st = (const MIGEMM_LDS unsigned char *)smem + (c % ST) * STAGE;
            const int rd = j ? rd1 : rd0;
#pragma unroll
            for (int t = 0; t < TW; ++t)
                b[t] = *(const MIGEMM_LDS u32x4 *)(st + B_OFF + (tg * TW + t) * kTileBytes + rd);
#pragma unroll
            for (int r = 0; r < RTW; ++r) a[r] = *(const MIGEMM_LDS u32x4 *)(st + (R0 + r) * kTileBytes + rd);
        };
        auto multiply = [&](const u32x4 (&a)[RTW], const u32x4 (&b)[TW]) {
#pragma unroll
            for (int r = 0; r < RTW; ++r)
#pragma unroll
                for (int t = 0; t < TW; ++t) mfma_acc<DT>(acc[r][t], a[r], b[t]);
        };

        // chunk c's loads are waited for (own count, then the barrier for
        // everyone's) between the two steps of chunk c - 1; that barrier
        // also ends every wave's reads of chunk c - 1, so its stage takes
        // chunk c - 1 + ST right after.  Step 1's reads overlap step 0's
        // MFMAs, the next chunk's step-0 reads overlap step 1's.
        u32x4 a0[RTW], b0[TW], a1[RTW], b1[TW];
        wait_vmcnt<Q * (ST - 2)>();
        __syncthreads();
        issue(ST - 1);
        operands(0, 0, a0, b0);
        for (int c = 0; c < chunks; ++c) {
            operands(c, 1, a1, b1);
            multiply(a0, b0);
            // at most the loads of chunks c + 2 .. c + ST - 1 outstanding
            wait_vmcnt<Q * (ST - 2)>();
            __syncthreads();
            issue(c + ST);
            if (c + 1 < chunks) operands(c + 1, 0, a0, b0);
            multiply(a1, b1);
        }
        // the last ring loads (past K, all zero) may still be landing
        wait_vmcnt<0>();
        mfma_settle();

        // lane (g, r16) holds rows 4g .. 4g+3 of each row tile for token r16
        // of each of the wave's token tiles
#pragma unroll
        for (int r = 0; r < RTW; ++r) {
            const int m = (R0 + r) * 16 + 4 * g;          // row within the workgroup
            if (m >= rows) break;
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const int tok = (tg * TW + t) * 16 + r16;
                if (tok >= toks) continue;
                uint16_t *dst = Y + (size_t)(tok0 + tok) * M + rbeg + m;
                if (y_vec && m + 3 < rows) {
                    u16x4 v = {to_out<DT>(acc[r][t][0]), to_out<DT>(acc[r][t][1]), to_out<DT>(acc[r][t][2]),
                               to_out<DT>(acc[r][t][3])};
                    *(u16x4 *)dst = v;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (m + i < rows) dst[i] = to_out<DT>(acc[r][t][i]);
                }
            }
        }
    };
    // waves w and w + 4 share a SIMD: one of each row group on every SIMD
    if (wave < 4)
        run(std::integral_constant<int, 0>{}, std::integral_constant<int, RT0>{});
    else
        run(std::integral_constant<int, RT0>{}, std::integral_constant<int, kWideRT - RT0>{});
}

namespace {

template <int DT, int NT, int ST, int RT0 = kWideRT0, int LW = kWideLoaders>
hipError_t launch_wide(const SkinnyLaunch &L, hipStream_t s)
{
    const int R = batch_rows_per_workgroup(L.M);
    const dim3 grid((unsigned)((L.M + R - 1) / R), (unsigned)((L.n + NT * 16 - 1) / (NT * 16)));
    hipLaunchKernelGGL((batch_wide_kernel<DT, NT, ST, RT0, LW>), grid, dim3(64 * kWideWaves), 0, s, L.W, L.X, L.Y,
                       L.M, L.K, L.n, R, L.y_vec && R % 4 == 0);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_wide_dt(const SkinnyLaunch &L, hipStream_t s)
{
    // 128-token blocks: 4 stages of 34 KiB; 256-token blocks: 3 of 50 KiB
    if (L.n <= 128) return launch_wide<DT, 8, 4>(L, s);
    return launch_wide<DT, 16, 3>(L, s);
}

}  // namespace

hipError_t batch_wide_launch(const SkinnyLaunch &L, hipStream_t s)
{
    if (L.n < 1 || L.n > kBatchWideMaxTokens) return hipErrorInvalidValue;
    return L.dtype == DT_F16 ? launch_wide_dt<DT_F16>(L, s) : launch_wide_dt<DT_BF16>(L, s);
}

}  // namespace migemm
