// gemv.hip -- bandwidth-bound decode GEMV  Y = X W^T  (bfloat16), no MFMA.
//
// Defined by the DCU decode page (forum.sourcefind.cn db785961): section 6.1
// fixes Y = X W^T with X:[n,k], W:[m,k], Y:[n,m]; section 6.2 splits the
// work along W's output rows, every Y[i,j] being an independent full-K dot
// product; section 5 observes that the plain kernel already runs at the
// HBM ceiling when enough waves are resident, so there is no explicit double
// buffer here -- many resident waves, each with several 16-byte loads in
// flight, hide the latency.
//
// Mapping: a wave owns RW consecutive rows of W.  Each lane covers 8
// consecutive k of every 512-wide chunk of K (one 16-byte load per row per
// chunk, one wave instruction = 1 KiB of a row, fully coalesced), and U chunks
// are loaded before any is consumed.  W is read once, with non-temporal loads
// (measured: they keep W from displacing other lines and raise the streaming
// rate); X is small and read through the caches.
// Products are exact in FP32 (BF16 widens by a shift) and accumulate with FP32
// fused multiply-adds; the 64 per-lane partial sums of each output
// are then added across the wave with cross-lane shuffles, and the result is
// rounded once to BF16 (nearest even).
#include "common.hpp"
#include "kernels.hpp"

namespace migemm {

// Eight BF16 products added into an FP32 accumulator.  A BF16 value widens
// to FP32 exactly by a 16-bit shift, so each product is exact in FP32 and
// only the additions round.
__device__ inline float dot8_bf16(u32x4 w, u32x4 x, float acc)
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        acc = fmaf(__builtin_bit_cast(float, w[c] << 16), __builtin_bit_cast(float, x[c] << 16), acc);
        acc = fmaf(__builtin_bit_cast(float, w[c] & 0xffff0000u),
                   __builtin_bit_cast(float, x[c] & 0xffff0000u), acc);
    }
    return acc;
}

__device__ inline float bf16_to_f32(uint16_t h)
{
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
    return v;
}

template <int NT, int RW, int VEC, int U>
__global__ void __launch_bounds__(1024)
gemv_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ X,
            uint16_t *__restrict__ Y, int M, int K)
{
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int row0 = (blockIdx.x * waves + wave) * RW;
    if (row0 >= M) return;   // whole wave idle; no block-wide barrier follows

    const uint16_t *wr[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) wr[r] = W + (size_t)min(row0 + r, M - 1) * K;

    float acc[RW][NT];
#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[r][i] = 0.f;

    if constexpr (VEC == 8) {
        constexpr int CH = 512;          // elements of K per wave-wide 16-byte load
        const int nfull = K / CH;
        const int lk = lane * 8;
        int t = 0;
        for (; t + U <= nfull; t += U) {
            u32x4 w[U][RW];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int r = 0; r < RW; ++r)
                    w[u][r] = __builtin_nontemporal_load((const u32x4 *)(wr[r] + (t + u) * CH + lk));
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    u32x4 x = *(const u32x4 *)(X + (size_t)i * K + (t + u) * CH + lk);
#pragma unroll
                    for (int r = 0; r < RW; ++r) acc[r][i] = dot8_bf16(w[u][r], x, acc[r][i]);
                }
        }
        for (; t < nfull; ++t) {
            u32x4 w[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r) w[r] = __builtin_nontemporal_load((const u32x4 *)(wr[r] + t * CH + lk));
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                u32x4 x = *(const u32x4 *)(X + (size_t)i * K + t * CH + lk);
#pragma unroll
                for (int r = 0; r < RW; ++r) acc[r][i] = dot8_bf16(w[r], x, acc[r][i]);
            }
        }
        const int k = nfull * CH + lk;   // last partial chunk: K % 8 == 0
        if (k < K) {
            u32x4 w[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r) w[r] = *(const u32x4 *)(wr[r] + k);
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                u32x4 x = *(const u32x4 *)(X + (size_t)i * K + k);
#pragma unroll
                for (int r = 0; r < RW; ++r) acc[r][i] = dot8_bf16(w[r], x, acc[r][i]);
            }
        }
    } else {
        for (int k = lane; k < K; k += 64) {
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                float x = bf16_to_f32(X[(size_t)i * K + k]);
#pragma unroll
                for (int r = 0; r < RW; ++r) acc[r][i] = fmaf(bf16_to_f32(wr[r][k]), x, acc[r][i]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            float s = wave_sum(acc[r][i]);
            if (lane == r * NT + i && row0 + r < M) Y[(size_t)i * M + row0 + r] = to_out<DT_BF16>(s);
        }
}

template <int NT, int RW, int VEC>
static hipError_t launch_t(const GemvLaunch &L, hipStream_t s)
{
    constexpr int U = (RW == 2) ? 5 : 2;
    const int waves = L.rows_per_block / RW;
    hipLaunchKernelGGL((gemv_kernel<NT, RW, VEC, U>), dim3((unsigned)L.grid), dim3(waves * 64), 0, s,
                       L.W, L.X, L.Y, L.M, L.K);
    return hipGetLastError();
}

// Rows per wave: 2, or 4 for the 8/16-token kernels (more rows share each
// X load); rows_per_block must be a multiple of it.
int gemv_rows_per_wave(int n_tokens, int rows_per_block)
{
    int rw = (n_tokens >= 8) ? 4 : 2;
    return rows_per_block < rw ? rows_per_block : rw;
}

template <int NT>
static hipError_t launch_nt(const GemvLaunch &L, hipStream_t s)
{
    int rw = gemv_rows_per_wave(NT, L.rows_per_block);
    if (L.vec == 8) return rw == 4 ? launch_t<NT, 4, 8>(L, s) : launch_t<NT, 2, 8>(L, s);
    return rw == 4 ? launch_t<NT, 4, 1>(L, s) : launch_t<NT, 2, 1>(L, s);
}

hipError_t gemv_launch(const GemvLaunch &L, hipStream_t s)
{
    switch (L.n) {
    case 1: return launch_nt<1>(L, s);
    case 2: return launch_nt<2>(L, s);
    case 4: return launch_nt<4>(L, s);
    case 8: return launch_nt<8>(L, s);
    case 16: return launch_nt<16>(L, s);
    }
    return hipErrorInvalidValue;
}

// ---- streaming-read probe ------------------------------------------------

constexpr int kProbeWaves = 768;         // one-wave workgroups, 3 per CU
constexpr int kProbeChunk = 8 * 64;      // 16-byte words per wave per step (8 KiB)

// Wave w reads the 8 KiB chunks w, w + kProbeWaves, ...: each lane keeps
// eight 16-byte non-temporal loads in flight, a wave's loads of one chunk
// cover it contiguously.  The grid size was swept (512 .. 8192 waves, 4 or
// 16 loads per lane): 3 waves per CU (6 MiB in flight over the chip) read
// fastest at 4 GiB and at 356 MB; more waves keep more requests in flight
// and read a few percent slower, fewer cannot cover the latency.  The words past the last whole chunk are read
// grid-stride.  sink[w] receives the XOR of every 32-bit word wave w read,
// so the XOR of all sink words equals the XOR of the buffer.
__global__ void __launch_bounds__(64) hbm_read_kernel(const u32x4 *__restrict__ buf, size_t n16,
                                                      uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t chunks = n16 / kProbeChunk;
    for (size_t c = blockIdx.x; c < chunks; c += kProbeWaves) {
        const u32x4 *p = buf + c * kProbeChunk + lane;
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + u * 64);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u];
    }
    for (size_t i = chunks * kProbeChunk + (size_t)blockIdx.x * 64 + lane; i < n16;
         i += (size_t)kProbeWaves * 64)
        acc ^= buf[i];
    uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v ^= __shfl_xor(v, s, 64);
    if (lane == 0) sink[blockIdx.x] = v;
}

int hbm_read_sink_words() { return kProbeWaves; }

hipError_t hbm_read_launch(const void *buf, size_t bytes, uint32_t *sink, hipStream_t s)
{
    hipLaunchKernelGGL(hbm_read_kernel, dim3(kProbeWaves), dim3(64), 0, s,
                       (const u32x4 *)buf, bytes / 16, sink);
    return hipGetLastError();
}

// Shader clock probe: each single-wave workgroup reads the shader-clock
// counter (s_memtime) and the 100 MHz real-time counter (s_memrealtime)
// around a dependent chain of `iters` FMAs and writes both elapsed counts;
// their ratio is the clock the wave ran at.
__global__ void __launch_bounds__(64) clock_probe_kernel(uint64_t *__restrict__ out, int iters)
{
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    float x = (float)threadIdx.x;
    for (int i = 0; i < iters; ++i) x = __builtin_fmaf(x, 0.999f, 1.0f);
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = t1 - t0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
    if (x == -1.0f) out[0] = 0;   // keeps the chain (x stays positive)
}

hipError_t clock_probe_launch(uint64_t *out, int blocks, int iters, hipStream_t s)
{
    hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)blocks), dim3(64), 0, s, out, iters);
    return hipGetLastError();
}

}  // namespace migemm
