// small.hip -- C = A x B for shapes whose 32x32 output tiles number at most
// a few hundred: FP16/BF16 inputs, FP32 accumulation, one rounding.
//
// The product of the S4000 GEMM write-up (section 1's rules, section 2's
// column-major addressing): C(m,n) = C[m + n*M] = sum_k A(m,k) B(k,n) with
// B(k,n) = B[k + n*K] and A(m,k) = A[m + k*M] (m-major) or At[k + m*K]
// (k-major, the gemm_tn form).
//
// At these sizes the tiled kernels wait on one chain per k step (a barrier,
// the operand reads, the MFMAs) over all of K, with most CUs idle.  Here a
// workgroup of NW waves (4, or 8 when K is long) owns one 32x32 tile of
// C and the waves split K between them (wave w takes the 32-k steps w,
// w + NW, ...), so each wave walks 1/NW of the steps:
//  * no LDS staging: a wave loads its operands straight into the 16x16x32
//    MFMA layout (lane (g, r): row or column r of a 16-wide block, k 8g ..
//    8g+7 of the step).  B's column and a k-major A's row are 16 contiguous
//    bytes; an m-major A gives each lane 8 values one row of A apart (2-byte
//    loads, 16 lanes reading 32 contiguous bytes per k);
//  * two steps' loads in flight per wave before their MFMAs;
//  * the NW waves' 32x32 FP32 partials meet in LDS (4 KiB per wave), one
//    thread sums the NW of each output element and rounds it once to
//    FP16/BF16.
// Elements past M, N or K read as zero (from a zero block) and are never
// stored.  B (and a k-major A) must have 16-byte rows: K a multiple of 8 and
// 16-byte aligned base pointers; an m-major A may have any M.
#include "common.hpp"
#include "kernels.hpp"

namespace migemm {

namespace {

constexpr int kSmallSteps = 2;            // 32-k steps a wave loads before multiplying

// 16 zero bytes in device memory: masked lanes load from here.
__device__ const uint16_t kSmallZeros[8] = {0, 0, 0, 0, 0, 0, 0, 0};

typedef const __attribute__((address_space(1))) u32x4 *sg16;
typedef const __attribute__((address_space(1))) uint16_t *sg2;

template <int DT>
__device__ inline void small_mfma(f32x4 &acc, u32x4 a, u32x4 b)
{
    if constexpr (DT == DT_F16)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

}  // namespace

template <int DT, bool AK, int NW>
__global__ void __launch_bounds__(64 * NW)
small_gemm_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
                  uint16_t *__restrict__ C, int M, int N, int K)
{
    static_assert(NW == 4 || NW == 8, "waves per tile");
    __shared__ f32x4 part[NW][4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
    const int steps = (K + 31) / 32;

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s0 = w; s0 < steps; s0 += NW * kSmallSteps) {
        u32x4 a[kSmallSteps][2], b[kSmallSteps][2];
#pragma unroll
        for (int q = 0; q < kSmallSteps; ++q) {
            const int s = s0 + NW * q;
            const int k0 = 32 * s + 8 * g;                     // this lane's 8 k of step s
            const bool kin = s < steps && k0 < K;              // K % 8 == 0: all 8 in or out
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + 16 * j + r16;
                b[q][j] = *(sg16)(kin && n < N ? B + (size_t)n * K + k0 : kSmallZeros);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int m = m0 + 16 * i + r16;
                if constexpr (AK) {
                    a[q][i] = *(sg16)(kin && m < M ? A + (size_t)m * K + k0 : kSmallZeros);
                } else {
                    uint16_t v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[e] = *(sg2)(kin && m < M ? A + (size_t)(k0 + e) * M + m : kSmallZeros);
                    a[q][i] = u32x4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
                                    (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
                }
            }
        }
#pragma unroll
        for (int q = 0; q < kSmallSteps; ++q)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) small_mfma<DT>(acc[i][j], a[q][i], b[q][j]);
    }

    // the waves' partial tiles: block (i, j) of wave w at part[w][2i + j]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) part[w][2 * i + j][lane] = acc[i][j];
    __syncthreads();
    // thread (w, lane), w < 4, sums block w's lane over the NW waves: rows
    // 4g .. 4g+3 of the block, column r16
    if (w >= 4) return;
    f32x4 t = part[0][w][lane];
#pragma unroll
    for (int v = 1; v < NW; ++v) {
        const f32x4 u = part[v][w][lane];
        t = f32x4{t[0] + u[0], t[1] + u[1], t[2] + u[2], t[3] + u[3]};
    }
    const int n = n0 + 16 * (w & 1) + r16;
    if (n >= N) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * (w >> 1) + 4 * g + e;
        if (m < M) C[(size_t)n * M + m] = to_out<DT>(t[e]);
    }
}

template <int DT, int NW>
static hipError_t small_launch_nw(const GemmLaunch &L, hipStream_t s)
{
    const dim3 grid((unsigned)((L.M + 31) / 32), (unsigned)((L.N + 31) / 32));
    if (L.a_kmajor)
        hipLaunchKernelGGL((small_gemm_kernel<DT, true, NW>), grid, dim3(64 * NW), 0, s, L.A, L.B, L.C,
                           L.M, L.N, L.K);
    else
        hipLaunchKernelGGL((small_gemm_kernel<DT, false, NW>), grid, dim3(64 * NW), 0, s, L.A, L.B, L.C,
                           L.M, L.N, L.K);
    return hipGetLastError();
}

template <int DT>
static hipError_t small_launch_dt(const GemmLaunch &L, hipStream_t s)
{
    const int64_t tiles = (int64_t)((L.M + 31) / 32) * ((L.N + 31) / 32);
    return small_waves(tiles, L.K) == 8 ? small_launch_nw<DT, 8>(L, s) : small_launch_nw<DT, 4>(L, s);
}

hipError_t small_launch(const GemmLaunch &L, hipStream_t s)
{
    if (L.K % 8 || L.splits > 1) return hipErrorInvalidValue;
    return L.dtype == DT_F16 ? small_launch_dt<DT_F16>(L, s) : small_launch_dt<DT_BF16>(L, s);
}

}  // namespace migemm
