// skinny.hip -- Y = X W^T for a batch of a few token rows on MFMA, streaming W
// from HBM once.
//
// The product of the DCU decode page (forum.sourcefind.cn db785961), section
// 6.1: W row-major [M, K], X row-major [n, K], Y row-major [n, M], FP32
// accumulation.  The page computes it with a row-blocked vector kernel
// (section 6.2); with a handful of tokens that kernel turns from
// bandwidth-bound into ALU-bound, since every W element then feeds n
// multiply-adds.  Here the multiply-adds run on the 4x4x4 MFMA with 16
// independent blocks per instruction (v_mfma_f32_4x4x4_16b_{f16,bf16}):
// lane 4b+i supplies row i of block b's A (4 k values), lane 4b+j column j
// of its B, and block b's 4x4 result lands in lane 4b+j, register i.
//
//  * A wave owns RW groups of 4 rows of W and TG groups of 4 token slots,
//    over all of K, in 128-wide k chunks.  Block b of a chunk takes k
//    offsets 8b .. 8b+7 (two MFMAs: the low and the high four).
//  * W is read with one 16-byte non-temporal load per lane per row group
//    and chunk, lane l taking row l/16 at offset 8*(l%16): 16 lanes read
//    256 contiguous bytes of one row, so every group of 4 lanes asks for 64
//    contiguous bytes (the address unit's fast case) and a wave reads whole
//    cache lines, straight into registers (no LDS), U chunks in flight in a
//    ring (each chunk's X requested before its W, so a wait for one chunk
//    never covers a younger request).  A
//    cross-lane permute (ds_bpermute, lane 4b+i <- lane 16i+b) then puts
//    row i's chunk b where block b's A operand expects it.
//  * X is loaded and permuted the same way (token j in place of row i),
//    from L1/L2.
//  * The 16 blocks hold partial sums over disjoint k; they are added with
//    four cross-lane butterflies at the end, and lane j of the wave stores
//    4 consecutive rows of token j.
//  * Rows past M are clamped on load and never stored; token slots past n
//    and k past K read as zero.  Each output is summed in FP32 and rounded
//    once to the output format.
#include "common.hpp"
#include "kernels.hpp"

namespace migemm {

typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

// 16 zero bytes in device memory: masked lanes load from here
__device__ const uint16_t kSkZeros[8] = {0, 0, 0, 0, 0, 0, 0, 0};
typedef const __attribute__((address_space(1))) u32x4 *sk_gptr16;
__device__ inline u32x4 sk_load16(const void *p) { return *(sk_gptr16)p; }
__device__ inline u32x4 sk_load16_nt(const void *p) { return __builtin_nontemporal_load((sk_gptr16)p); }

// acc += (low or high four halves of a) x (the same of b) on 16 4x4x4 blocks
template <int DT, int HI>
__device__ inline void mfma4(f32x4 &acc, u32x4 a, u32x4 b)
{
    const uint32_t a0 = a[2 * HI], a1 = a[2 * HI + 1], b0 = b[2 * HI], b1 = b[2 * HI + 1];
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    const u32x2 av = {a0, a1}, bv = {b0, b1};
    if constexpr (DT == DT_F16)
        acc = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(f16x4, av),
                                                 __builtin_bit_cast(f16x4, bv), acc, 0, 0, 0);
    else
        acc = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(i16x4, av),
                                                     __builtin_bit_cast(i16x4, bv), acc, 0, 0, 0);
}

// 16 bytes per lane, moved from lane 16*(L%4) + L/4 to lane L
__device__ inline u32x4 to_mfma4_layout(u32x4 v, int addr)
{
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 4; ++d) r[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v[d]);
    return r;
}

template <int DT, int RW, int TG, int U>
__global__ void __launch_bounds__(256)
skinny_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ X,
              uint16_t *__restrict__ Y, int M, int K, int n, int y_vec)
{
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int b = lane >> 2, q = lane & 3;          // MFMA block, row / column within it
    const int lr = lane >> 4, lc = lane & 15;       // load layout: row / 16-byte chunk
    const int perm = (16 * q + b) * 4;              // ds_bpermute source of this lane
    const int row0 = (blockIdx.x * 4 + wave) * (4 * RW);
    if (row0 >= M) return;                          // whole wave idle; no barrier follows

    const uint16_t *wr[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) wr[r] = W + (size_t)min(row0 + 4 * r + lr, M - 1) * K + 8 * lc;
    const uint16_t *xr[TG];
    bool xok[TG];
#pragma unroll
    for (int t = 0; t < TG; ++t) {
        xok[t] = 4 * t + lr < n;
        xr[t] = X + (size_t)(xok[t] ? 4 * t + lr : 0) * K + 8 * lc;
    }

    f32x4 acc[RW][TG];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < TG; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Ring of U chunks in flight: chunk c + U is requested into the slot
    // chunk c has just been read from, X before W, so that waiting for a
    // chunk never waits for a younger request.  Lanes past K (and chunks
    // past the end) load from a zero block instead of selecting zero after
    // the load.
    const int chunks = (K + 127) / 128;
    const int padded = (chunks + U - 1) / U * U;
    auto load_chunk = [&](int c, u32x4 (&wv)[RW], u32x4 (&xv)[TG]) {
        const bool kok = c * 128 + 8 * lc < K;
#pragma unroll
        for (int t = 0; t < TG; ++t) xv[t] = sk_load16((xok[t] && kok) ? (const void *)(xr[t] + c * 128) : kSkZeros);
#pragma unroll
        for (int r = 0; r < RW; ++r) wv[r] = sk_load16_nt(kok ? (const void *)(wr[r] + c * 128) : kSkZeros);
    };
    u32x4 w[U][RW], xs[U][TG];
#pragma unroll
    for (int u = 0; u < U; ++u) load_chunk(u, w[u], xs[u]);
    for (int c0 = 0; c0 < padded; c0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4 x[TG], wv[RW];
#pragma unroll
            for (int t = 0; t < TG; ++t) x[t] = to_mfma4_layout(xs[u][t], perm);
#pragma unroll
            for (int r = 0; r < RW; ++r) wv[r] = to_mfma4_layout(w[u][r], perm);
            load_chunk(c0 + u + U, w[u], xs[u]);
            // all low halves, then all high halves: consecutive MFMAs
            // never feed each other
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int t = 0; t < TG; ++t) mfma4<DT, 0>(acc[r][t], wv[r], x[t]);
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int t = 0; t < TG; ++t) mfma4<DT, 1>(acc[r][t], wv[r], x[t]);
        }
    }

    // add the 16 blocks (lanes q, q+4, ..., q+60), then lane q of the wave
    // (block 0) stores rows row0 + 4r .. +3 of token 4t + q
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int t = 0; t < TG; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = acc[r][t][e];
#pragma unroll
                for (int m = 4; m <= 32; m <<= 1) v += __shfl_xor(v, m, 64);
                acc[r][t][e] = v;
            }
    if (b != 0) return;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int rr = row0 + 4 * r;
#pragma unroll
        for (int t = 0; t < TG; ++t) {
            const int tok = 4 * t + q;
            if (tok >= n) continue;
            uint16_t *dst = Y + (size_t)tok * M + rr;
            if (y_vec && rr + 3 < M) {
                u16x4 v = {to_out<DT>(acc[r][t][0]), to_out<DT>(acc[r][t][1]),
                           to_out<DT>(acc[r][t][2]), to_out<DT>(acc[r][t][3])};
                *(u16x4 *)dst = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (rr + e < M) dst[e] = to_out<DT>(acc[r][t][e]);
            }
        }
    }
}

template <int DT, int TG>
static hipError_t launch_tg(const SkinnyLaunch &L, hipStream_t s)
{
    // chunks in flight: 8 with one token group (84 + 48 registers), 4 with
    // two (measured best of 4 / 6 / 8)
    constexpr int RW = 2, U = TG == 1 ? 8 : 4;
    const unsigned grid = (unsigned)((L.M + 16 * RW - 1) / (16 * RW));   // 4 waves x 4*RW rows
    hipLaunchKernelGGL((skinny_kernel<DT, RW, TG, U>), dim3(grid), dim3(256), 0, s,
                       L.W, L.X, L.Y, L.M, L.K, L.n, L.y_vec);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(const SkinnyLaunch &L, hipStream_t s)
{
    if (L.n <= 4) return launch_tg<DT, 1>(L, s);
    return launch_tg<DT, 2>(L, s);
}

hipError_t skinny_launch(const SkinnyLaunch &L, hipStream_t s)
{
    if (L.n < 1 || L.n > kSkinnyMaxTokens) return hipErrorInvalidValue;
    return L.dtype == DT_F16 ? launch_dt<DT_F16>(L, s) : launch_dt<DT_BF16>(L, s);
}

}  // namespace migemm
