// batch.hip -- Y = X W^T for a decode batch of 9 .. 128 token rows on the
// 16x16x32 MFMA, streaming W from HBM once.
//
// The product of the DCU decode page (forum.sourcefind.cn db785961), section
// 6.1: W row-major [M, K], X row-major [n, K], Y row-major [n, M], FP32
// accumulation, one rounding.  With a few dozen tokens the work per W element
// is still small (2n FLOP per 2 bytes), so the kernel is built to stream W at
// HBM speed with enough MFMA throughput to spare:
//
//  * A workgroup of NWV waves (2 for a 16-token block, else 4) owns 16*NWV
//    rows of W (16 per wave) and a block of up to 16*NTT tokens; K is walked
//    in chunks of 128.
//  * W is read as whole 128-byte lines: each load instruction covers 8 rows x
//    128 bytes (lane l: row l/8, bytes 16*(l%8)); a wave's 16 rows x 128 k of
//    a chunk are 4 such loads, non-temporal, U chunks in flight in
//    registers.  (Loads of 64 bytes per row, the A operand's own shape,
//    stream W at two thirds of this rate.)  Each chunk goes through a
//    wave-private 4 KB LDS area -- row r's 16-byte piece x at
//    r*256 + 16*(x ^ r), so the line writes and the operand reads both spread
//    over all banks -- and comes back as A operands of v_mfma_f32_16x16x32
//    (lane l: row l%16, k 32*j + 8*(l/16) .. +7).
//  * The chunk of X (the block's tokens x 128 k) is staged once per
//    workgroup in LDS, double-buffered, token rows padded to 272 bytes so the
//    16 rows a B-operand read touches fall in distinct banks; each wave reads
//    its B operands (token l%16, k 32*j + 8*(l/16)) with ds_read_b128.
//  * One barrier per chunk; X is fetched from L2 two chunks ahead, into
//    alternating staging registers, ahead of the W loads issued with it.
//  * The chunk count is rounded up to a multiple of U; chunks past K (and k
//    past K inside the last real chunk) read as zero (from a zero block), rows past M are
//    clamped on load and never stored, tokens past n read as zero and are
//    never stored.
#include <type_traits>
#include "common.hpp"
#include "kernels.hpp"

namespace migemm {

namespace {

constexpr int kKC = 128;                  // k per chunk
constexpr int kXRow = kKC * 2 + 16;       // LDS bytes per staged token row

// 16 zero bytes in device memory.  A masked lane loads from here instead of
// selecting zero after its load: a select placed on the loaded value makes
// the compiler wait for that load wherever it puts the select.
__device__ const uint16_t kZeros[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// 16-byte loads through a global-address-space pointer (a select between a
// kernel argument and kZeros would otherwise leave a generic pointer and a
// flat load, which also counts against the LDS counter)
typedef const __attribute__((address_space(1))) u32x4 *gptr16;
__device__ inline u32x4 load16(const void *p) { return *(gptr16)p; }
__device__ inline u32x4 load16_nt(const void *p) { return __builtin_nontemporal_load((gptr16)p); }

template <int DT>
__device__ inline void mfma_16x16x32(f32x4 &acc, u32x4 a, u32x4 b)
{
    if constexpr (DT == DT_F16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

}  // namespace

template <int DT, int NTT, int U, int NWV>
__global__ void __launch_bounds__(64 * NWV)
batch_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ X,
             uint16_t *__restrict__ Y, int M, int K, int n, int y_vec)
{
    constexpr int XP = NTT * 4 / NWV;             // 16-byte X pieces per thread and chunk
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][NTT * 16][kXRow];
    __shared__ __attribute__((aligned(16))) uint8_t ws[NWV][16 * 256];   // per wave

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int row0 = blockIdx.x * (16 * NWV) + wave * 16;
    const int tok0 = blockIdx.y * (NTT * 16);
    const int chunks = (K + kKC - 1) / kKC;
    const int padded = (chunks + U - 1) / U * U;

    // W loads: instruction 2h + q reads rows 8h + l/8 (clamped) at k
    // 64q + 8*(l%8) of the chunk; piece x = 8q + l%8 of row rw
    const int lr = lane >> 3, lc = lane & 7;
    const uint16_t *wrow0 = W + (size_t)min(row0 + lr, M - 1) * K;
    const uint16_t *wrow1 = W + (size_t)min(row0 + 8 + lr, M - 1) * K;
    auto load_w = [&](int c, u32x4 (&w)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = c * kKC + 64 * (i & 1) + 8 * lc;
            w[i] = load16_nt(k < K ? (i < 2 ? wrow0 : wrow1) + k : kZeros);
        }
    };
    uint8_t *wsw = ws[wave];
    // write a chunk's 4 loads into the wave's area, read back the 4 A operands
    auto relayout_w = [&](const u32x4 (&w)[4], u32x4 (&a)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rw = 8 * (i >> 1) + lr, x = 8 * (i & 1) + lc;
            *(u32x4 *)(wsw + rw * 256 + 16 * (x ^ rw)) = w[i];
        }
        // the area is private to the wave and LDS runs a wave's accesses in
        // order; the wait only keeps the compiler from reordering
        __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int x = 4 * j + g;
            a[j] = *(const u32x4 *)(wsw + r16 * 256 + 16 * (x ^ r16));
        }
    };
    auto load_x = [&](int c, u32x4 (&xr)[XP]) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int e = p * (64 * NWV) + tid;
            const int t = e >> 4, ch = e & 15;
            const int k = c * kKC + ch * 8;
            const bool ok = tok0 + t < n && k < K;
            xr[p] = load16(ok ? X + (size_t)(tok0 + t) * K + k : kZeros);
        }
    };
    auto store_x = [&](int buf, const u32x4 (&xr)[XP]) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int e = p * (64 * NWV) + tid;
            *(u32x4 *)&xs[buf][e >> 4][(e & 15) * 16] = xr[p];
        }
    };

    f32x4 acc[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Chunk c's X sits in LDS buffer c & 1 and, before that, in staging
    // registers xr[c & 1] (U is even, so c & 1 == u & 1 is static).  Per
    // chunk: W from w[u] through the wave's LDS area into A operands; the X
    // loads of chunk c + 2 and the W loads of chunk c + U (into the freed
    // w[u]); the MFMAs; the store of chunk c + 1's X (fetched a chunk ago,
    // ahead of the previous W loads, so waiting for it leaves the W loads in
    // flight); one barrier.
    static_assert(U % 2 == 0, "U even");
    u32x4 w[U][4];
    u32x4 xr[2][XP];
    load_x(0, xr[0]);
    load_x(1, xr[1]);
#pragma unroll
    for (int u = 0; u < U; ++u) load_w(u, w[u]);
    store_x(0, xr[0]);
    __syncthreads();

    for (int c0 = 0; c0 < padded; c0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u, buf = u & 1;
            u32x4 a[4];
            relayout_w(w[u], a);
            load_x(c + 2, xr[buf]);
            load_w(c + U, w[u]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < NTT; ++t) {
                    const u32x4 b = *(const u32x4 *)&xs[buf][t * 16 + r16][(32 * j + 8 * g) * 2];
                    mfma_16x16x32<DT>(acc[t], a[j], b);
                }
            store_x(buf ^ 1, xr[buf ^ 1]);
            __syncthreads();
        }
    }

    // lane (g, r16) holds rows 4g .. 4g+3 of the wave's 16 for token r16 of
    // each 16-token tile
    const int m = row0 + 4 * g;
    if (m >= M) return;
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
        const int tok = tok0 + t * 16 + r16;
        if (tok >= n) continue;
        uint16_t *dst = Y + (size_t)tok * M + m;
        if (y_vec && m + 3 < M) {
            u16x4 v = {to_out<DT>(acc[t][0]), to_out<DT>(acc[t][1]), to_out<DT>(acc[t][2]),
                       to_out<DT>(acc[t][3])};
            *(u16x4 *)dst = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (m + i < M) dst[i] = to_out<DT>(acc[t][i]);
        }
    }
}

// ---------------------------------------------------------------------------
// Row-balanced variant: the same product for up to 256 tokens, with the rows
// of W cut evenly over the workgroups instead of in tiles of a power of two.
// W's 34816 rows (2^11 x 17) over 256 CUs are 136 rows each: power-of-two
// tiles leave half the CUs idle (256 rows) or give 16 CUs a second tile
// (128), and small workgroups re-read X for every few rows.  Here workgroup b
// owns rows [b*R, b*R + R) (R a multiple of 8, at most 144) with 9 waves of
// 16 rows (the last one holding only R - 128 live rows), so that every CU
// streams the same share of W once, and all 9 waves share each staged chunk
// of X.  K goes in chunks of 64 (one 128-byte line per row):
//  * W: per wave and chunk two loads of 8 rows x 128 bytes (lane l: row
//    8h + l/8, bytes 16*(l%8)), non-temporal, U chunks in flight; through a
//    wave-private 2 KB LDS area (row r's piece x at r*128 + 16*(x ^ (r&7)):
//    the operand reads of 16 rows touch 16 distinct 16-byte bank groups) into
//    the A operands of the chunk's two 32-k steps;
//  * X: the chunk for the block's 16*NTT tokens staged in LDS, double
//    buffered, token rows padded to 144 bytes (16 rows of an operand read fall
//    in distinct banks), fetched from L2 two chunks ahead;
//  * one barrier per chunk.
// Rows outside the workgroup's range or past M load zeros and are not
// stored; so are tokens past n and k past K.
constexpr int kRowWaves = 9;
constexpr int kRKC = 64;                   // k per chunk
constexpr int kRXRow = kRKC * 2 + 16;      // LDS bytes per staged token row

template <int DT, int NTT, int U, int XD>
__global__ void __launch_bounds__(64 * kRowWaves)
batch_rows_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ X,
                  uint16_t *__restrict__ Y, int M, int K, int n, int R, int y_vec)
{
    constexpr int NT = 64 * kRowWaves;
    constexpr int XPIECES = NTT * 16 * (kRKC / 8);       // 16-byte X pieces per chunk
    constexpr int XP = (XPIECES + NT - 1) / NT;          // per thread
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][NTT * 16][kRXRow];
    __shared__ __attribute__((aligned(16))) uint8_t ws[kRowWaves][16 * kRKC * 2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int rbeg = blockIdx.x * R;
    const int rend = min(rbeg + R, M);
    const int row0 = rbeg + wave * 16;
    // waves past the workgroup's rows (R < 144) only help stage X
    const bool live = row0 < rend;
    const int tok0 = blockIdx.y * (NTT * 16);
    const int chunks = (K + kRKC - 1) / kRKC;
    const int padded = (chunks + U - 1) / U * U;

    // W loads: instruction h reads row 8h + l/8 of the wave's 16 at k 8*(l%8)
    const int lr = lane >> 3, lc = lane & 7;
    const int wr0 = row0 + lr, wr1 = row0 + 8 + lr;
    const uint16_t *wrow0 = wr0 < rend ? W + (size_t)wr0 * K : nullptr;
    const uint16_t *wrow1 = wr1 < rend ? W + (size_t)wr1 * K : nullptr;
    auto load_w = [&](int c, u32x4 (&w)[2]) {
        const int k = c * kRKC + 8 * lc;
        w[0] = load16_nt(wrow0 && k < K ? wrow0 + k : kZeros);
        w[1] = load16_nt(wrow1 && k < K ? wrow1 + k : kZeros);
    };
    uint8_t *wsw = ws[wave];
    auto relayout_w = [&](const u32x4 (&w)[2], u32x4 (&a)[2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rw = 8 * h + lr;
            *(u32x4 *)(wsw + rw * (kRKC * 2) + 16 * (lc ^ (rw & 7))) = w[h];
        }
        // the area is private to the wave and LDS runs a wave's accesses in
        // order; the wait only keeps the compiler from reordering
        __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int x = 4 * j + g;
            a[j] = *(const u32x4 *)(wsw + r16 * (kRKC * 2) + 16 * (x ^ (r16 & 7)));
        }
    };
    auto load_x = [&](int c, u32x4 (&xr)[XP]) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int e = p * NT + tid;
            const int t = e >> 3, ch = e & 7;
            const int k = c * kRKC + ch * 8;
            const bool ok = e < XPIECES && tok0 + t < n && k < K;
            xr[p] = load16(ok ? X + (size_t)(tok0 + t) * K + k : kZeros);
        }
    };
    auto store_x = [&](int buf, const u32x4 (&xr)[XP]) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int e = p * NT + tid;
            if (XPIECES % NT == 0 || e < XPIECES) *(u32x4 *)&xs[buf][e >> 3][(e & 7) * 16] = xr[p];
        }
    };

    f32x4 acc[NTT];
#pragma unroll
    for (int t = 0; t < NTT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // chunk c's X sits in LDS buffer c & 1 and, before that, in staging
    // registers (XD sets: fetched XD chunks ahead); per chunk: W through the
    // wave's area into A operands, the X loads of chunk c + XD and the W
    // loads of chunk c + U, the MFMAs, the store of chunk c + 1's X, one
    // barrier
    static_assert(U % 2 == 0 && (XD == 1 || XD == 2), "U even, one or two X staging sets");
    // one copy of the pipeline for waves with rows and one, without the W
    // loads and MFMAs, for waves that only stage X: the branch is uniform
    // and each copy keeps its exact count of loads in flight
    auto pipeline = [&](auto live_c) {
        constexpr bool LV = decltype(live_c)::value;
        u32x4 w[U][2];
        u32x4 xr[XD][XP];
        load_x(0, xr[0]);
        if constexpr (XD == 2) load_x(1, xr[1]);
        if constexpr (LV) {
#pragma unroll
            for (int u = 0; u < U; ++u) load_w(u, w[u]);
        }
        store_x(0, xr[0]);
        if constexpr (XD == 1) load_x(1, xr[0]);
        __syncthreads();

        for (int c0 = 0; c0 < padded; c0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u, buf = u & 1;
                u32x4 a[2];
                if constexpr (LV) relayout_w(w[u], a);
                if constexpr (XD == 2) load_x(c + 2, xr[buf]);
                if constexpr (LV) {
                    load_w(c + U, w[u]);
                    // the chunk's 2 * NTT MFMAs, B operand i read PB MFMAs
                    // ahead of its use from a rolling window (the compiler
                    // would otherwise fetch all of them first and run out
                    // of registers)
                    constexpr int NI = 2 * NTT, PB = NTT >= 16 ? 2 : (NTT == 8 ? 8 : (NI < 4 ? NI : 4));
                    auto bread = [&](int i) {
                        const int j = i / NTT, t = i % NTT;
                        return *(const u32x4 *)&xs[buf][t * 16 + r16][(32 * j + 8 * g) * 2];
                    };
                    u32x4 bw[PB];
#pragma unroll
                    for (int i = 0; i < PB; ++i) bw[i] = bread(i);
#pragma unroll
                    for (int i = 0; i < NI; ++i) {
                        mfma_16x16x32<DT>(acc[i % NTT], a[i / NTT], bw[i % PB]);
                        if (i + PB < NI) bw[i % PB] = bread(i + PB);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                if constexpr (XD == 2) {
                    store_x(buf ^ 1, xr[buf ^ 1]);
                } else {
                    store_x(buf ^ 1, xr[0]);
                    load_x(c + 2, xr[0]);
                }
                __syncthreads();
            }
        }
    };
    if (live)
        pipeline(std::true_type{});
    else
        pipeline(std::false_type{});

    // lane (g, r16) holds rows 4g .. 4g+3 of the wave's 16 for token r16 of
    // each 16-token tile
    const int m = row0 + 4 * g;
    if (!live || m >= rend) return;
#pragma unroll
    for (int t = 0; t < NTT; ++t) {
        const int tok = tok0 + t * 16 + r16;
        if (tok >= n) continue;
        uint16_t *dst = Y + (size_t)tok * M + m;
        if (y_vec && m + 3 < rend) {
            u16x4 v = {to_out<DT>(acc[t][0]), to_out<DT>(acc[t][1]), to_out<DT>(acc[t][2]),
                       to_out<DT>(acc[t][3])};
            *(u16x4 *)dst = v;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (m + i < rend) dst[i] = to_out<DT>(acc[t][i]);
        }
    }
}

// Rows per workgroup: W's rows spread evenly over 256 workgroups (one per
// CU), rounded up to a multiple of 8, at most 144 (9 waves of 16).
int batch_rows_per_workgroup(int M)
{
    int R = (M + 255) / 256;
    R = (R + 7) / 8 * 8;
    return R < 8 ? 8 : (R > 16 * kRowWaves ? 16 * kRowWaves : R);
}

template <int DT, int NTT, int U>
static hipError_t launch_rows_ntt_u(const SkinnyLaunch &L, int R, hipStream_t s)
{
    // X staged one chunk ahead for 256 tokens (the second staging set would
    // not fit the 168 registers of 9 waves)
    constexpr int XD = NTT >= 16 ? 1 : 2;
    const dim3 grid((unsigned)((L.M + R - 1) / R), (unsigned)((L.n + NTT * 16 - 1) / (NTT * 16)));
    hipLaunchKernelGGL((batch_rows_kernel<DT, NTT, U, XD>), grid, dim3(64 * kRowWaves), 0, s, L.W, L.X, L.Y, L.M,
                       L.K, L.n, R, L.y_vec && R % 4 == 0);
    return hipGetLastError();
}

template <int DT, int NTT>
static hipError_t launch_rows_ntt(const SkinnyLaunch &L, hipStream_t s)
{
    // W chunks in flight per wave: 2 for 256 tokens, else 4 -- measured 1-4%
    // faster than 8 from 64 to 136 rows per workgroup (4 to 9 waves with
    // rows; 2 chunks lose 7-35%) -- and 8 when a workgroup has fewer rows,
    // whose few waves carry all of the CU's loads
    const int R = batch_rows_per_workgroup(L.M);
    if constexpr (NTT >= 16)
        return launch_rows_ntt_u<DT, NTT, 2>(L, R, s);
    else if constexpr (NTT >= 4)
        return launch_rows_ntt_u<DT, NTT, 4>(L, R, s);
    else
        return R >= 64 ? launch_rows_ntt_u<DT, NTT, 4>(L, R, s) : launch_rows_ntt_u<DT, NTT, 8>(L, R, s);
}

template <int DT>
static hipError_t launch_rows_dt(const SkinnyLaunch &L, hipStream_t s)
{
    if (L.n <= 16) return launch_rows_ntt<DT, 1>(L, s);
    if (L.n <= 32) return launch_rows_ntt<DT, 2>(L, s);
    if (L.n <= 64) return launch_rows_ntt<DT, 4>(L, s);
    if (L.n <= 128) return launch_rows_ntt<DT, 8>(L, s);
    return launch_rows_ntt<DT, 16>(L, s);
}

hipError_t batch_rows_launch(const SkinnyLaunch &L, hipStream_t s)
{
    if (L.n < 1 || L.n > kBatchRowsMaxTokens) return hipErrorInvalidValue;
    return L.dtype == DT_F16 ? launch_rows_dt<DT_F16>(L, s) : launch_rows_dt<DT_BF16>(L, s);
}

template <int DT, int NTT>
static hipError_t launch_ntt(const SkinnyLaunch &L, hipStream_t s)
{
    constexpr int NWV = batch_waves(NTT * 16);
    // 4 chunks of W in flight; 2 for the 64- and 128-token blocks, whose X
    // staging already takes the registers (measured faster there)
    constexpr int U = NTT >= 4 ? 2 : 4;
    const dim3 grid((unsigned)((L.M + 16 * NWV - 1) / (16 * NWV)), (unsigned)((L.n + NTT * 16 - 1) / (NTT * 16)));
    hipLaunchKernelGGL((batch_kernel<DT, NTT, U, NWV>), grid, dim3(64 * NWV), 0, s, L.W, L.X, L.Y, L.M, L.K,
                       L.n, L.y_vec);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(const SkinnyLaunch &L, hipStream_t s)
{
    if (L.n <= 16) return launch_ntt<DT, 1>(L, s);
    if (L.n <= 32) return launch_ntt<DT, 2>(L, s);
    if (L.n <= 64) return launch_ntt<DT, 4>(L, s);
    return launch_ntt<DT, 8>(L, s);
}

hipError_t batch_launch(const SkinnyLaunch &L, hipStream_t s)
{
    if (L.n < 1 || L.n > kBatchMaxTokens) return hipErrorInvalidValue;
    return L.dtype == DT_F16 ? launch_dt<DT_F16>(L, s) : launch_dt<DT_BF16>(L, s);
}

}  // namespace migemm
