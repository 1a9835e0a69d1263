// attention.hip -- decode attention over a paged KV cache, split along the
// cached sequence into segments, merged with a log-sum-exp reduction.
//
// What it computes is the DCU decode page's (forum.sourcefind.cn db785961)
// section 6.1: for each query head, scores = q K^T over the L cached tokens
// (here times `scale`), prob = softmax(scores), out = prob V, with the KV
// cache kept in pages [block][token_in_block][kv_head][head_dim].  How it is
// split is the same page's section 6.3: the L tokens are cut into S
// contiguous segments; each segment produces its local maximum, local
// softmax denominator and local prob V; a second pass merges them with the
// global maximum.  Section 7 tunes S (16 or 32) for its chip; here S is a
// parameter, chosen automatically for 256 CUs (enough workgroups to keep the
// HBM stream busy, enough tokens per segment to amortise the merge).
//
// Segment kernel: one workgroup (4 waves) per (segment, kv head, sequence).
// A K or V row of D BF16 values is D/8 lanes x 16 bytes, so one wave load
// reads 64/(D/8) whole rows (2 rows of 512 B at D = 256): full cache lines,
// every 4 lanes contiguous.  The G = Hq / Hkv query heads of the kv head
// share every K and V load.  Each lane keeps its 8 elements of q (for G
// heads, pre-multiplied by scale * log2 e so that exponentials are powers of
// two) and its 8 elements of the running output; a token's score is the
// dot product summed across its D/8 lanes with cross-lane butterflies.
// Scores are taken a batch at a time: one rescale of the running state per
// batch, then exp2 and the accumulation of prob * V.  At the end the token
// slots of a wave and then the 4 waves are merged, and the segment's
// (max, denominator, unnormalised output) go to the workspace in FP32.
//
// Merge kernel: one workgroup per (query head, sequence), one thread per
// output element: global max over segments, the weighted sums, one division
// and one rounding to BF16.  Empty segments (max = -inf, denominator 0) add
// nothing; a sequence with no token gives zeros.  Tokens whose page id is
// outside [0, num_blocks) are skipped instead of read.
#include "common.hpp"
#include "kernels.hpp"

namespace migemm {

namespace {

constexpr int kAttnWaves = 4;
constexpr float kNegInf = -__builtin_inff();

__device__ inline float exp2_guarded(float x)
{
    return x == kNegInf ? 0.f : __builtin_amdgcn_exp2f(x);
}

// (m, l, o) <- merge of itself and (m2, l2, o2), maxima in log2 units
template <int G>
__device__ inline void merge_state(float (&m)[G], float (&l)[G], float (&o)[G][8],
                                   const float (&m2)[G], const float (&l2)[G],
                                   const float (&o2)[G][8])
{
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], m2[h]);
        const float a = (mn == kNegInf) ? 0.f : exp2_guarded(m[h] - mn);
        const float b = (mn == kNegInf) ? 0.f : exp2_guarded(m2[h] - mn);
        l[h] = l[h] * a + l2[h] * b;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = o[h][e] * a + o2[h][e] * b;
        m[h] = mn;
    }
}

}  // namespace

template <int D, int G>
__global__ void __launch_bounds__(kAttnWaves * 64)
attn_segment_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kc,
                    const uint16_t *__restrict__ Vc, const int32_t *__restrict__ block_table,
                    const int32_t *__restrict__ seq_lens, float *__restrict__ part_o,
                    float *__restrict__ part_ml, int Hq, int Hkv, int block_size, int max_blocks,
                    int num_blocks, float qscale, int S)
{
    constexpr int CPL = D / 8;          // lanes per cached row (16 bytes each)
    constexpr int TPI = 64 / CPL;       // rows per wave load
    constexpr int U = 4;                // wave loads of K (and of V) per batch
    static_assert(D % 64 == 0 && D <= 512 && TPI >= 1, "head dim");
    __shared__ float xs[kAttnWaves][G][2 + D];

    const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int slot = lane / CPL, c = lane % CPL;

    int L = seq_lens[b];
    L = L < 0 ? 0 : (L > max_blocks * block_size ? max_blocks * block_size : L);
    const int seg = (L + S - 1) / S;
    const int l0 = min(L, s * seg), l1 = min(L, l0 + seg);
    const int per = (l1 - l0 + kAttnWaves - 1) / kAttnWaves;
    const int w0 = min(l1, l0 + wave * per), w1 = min(l1, w0 + per);

    // this lane's 8 elements of q for the G heads, in log2 units
    float q[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const u32x4 v = *(const u32x4 *)(Q + ((size_t)b * Hq + kvh * G + h) * D + c * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            q[h][2 * e] = __builtin_bit_cast(float, v[e] << 16) * qscale;
            q[h][2 * e + 1] = __builtin_bit_cast(float, v[e] & 0xffff0000u) * qscale;
        }
    }

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    const int32_t *bt = block_table + (size_t)b * max_blocks;
    const size_t row_stride = (size_t)Hkv * D;          // elements between tokens in a page
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int t0 = w0; t0 < w1; t0 += TPI * U) {
        u32x4 kv[U], vv[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tok = t0 + TPI * u + slot;
            ok[u] = tok < w1;
            size_t off = 0;
            if (ok[u]) {
                const int blk = bt[tok / block_size];
                ok[u] = blk >= 0 && blk < num_blocks;
                off = ((size_t)blk * block_size + tok % block_size) * row_stride + (size_t)kvh * D + c * 8;
            }
            kv[u] = ok[u] ? *(const u32x4 *)(Kc + off) : zero;
            vv[u] = ok[u] ? *(const u32x4 *)(Vc + off) : zero;
        }
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = __builtin_bit_cast(float, kv[u][e] << 16);
                kf[2 * e + 1] = __builtin_bit_cast(float, kv[u][e] & 0xffff0000u);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) p = fmaf(q[h][e], kf[e], p);
#pragma unroll
                for (int x = 1; x < CPL; x <<= 1) p += __shfl_xor(p, x, 64);
                sc[u][h] = ok[u] ? p : kNegInf;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mb = sc[0][h];
#pragma unroll
            for (int u = 1; u < U; ++u) mb = fmaxf(mb, sc[u][h]);
            const float mn = fmaxf(m[h], mb);
            if (mn == kNegInf) continue;                 // nothing seen yet
            const float corr = exp2_guarded(m[h] - mn);
            l[h] *= corr;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= corr;
            m[h] = mn;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = exp2_guarded(sc[u][h] - mn);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[h][2 * e] = fmaf(p, __builtin_bit_cast(float, vv[u][e] << 16), o[h][2 * e]);
                    o[h][2 * e + 1] = fmaf(p, __builtin_bit_cast(float, vv[u][e] & 0xffff0000u), o[h][2 * e + 1]);
                }
            }
        }
    }

    // merge the token slots of the wave (lanes c, c + CPL, ...)
#pragma unroll
    for (int x = CPL; x < 64; x <<= 1) {
        float m2[G], l2[G], o2[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m2[h] = __shfl_xor(m[h], x, 64);
            l2[h] = __shfl_xor(l[h], x, 64);
#pragma unroll
            for (int e = 0; e < 8; ++e) o2[h][e] = __shfl_xor(o[h][e], x, 64);
        }
        merge_state<G>(m, l, o, m2, l2, o2);
    }
    // then the waves, through LDS; wave 0 writes the segment's state
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (c == 0) {
                xs[wave][h][0] = m[h];
                xs[wave][h][1] = l[h];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[wave][h][2 + c * 8 + e] = o[h][e];
        }
    }
    __syncthreads();
    if (wave != 0 || slot != 0) return;
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) {
        float m2[G], l2[G], o2[G][8];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m2[h] = xs[w][h][0];
            l2[h] = xs[w][h][1];
#pragma unroll
            for (int e = 0; e < 8; ++e) o2[h][e] = xs[w][h][2 + c * 8 + e];
        }
        merge_state<G>(m, l, o, m2, l2, o2);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const size_t row = ((size_t)b * Hq + kvh * G + h) * S + s;
        if (c == 0) {
            part_ml[row * 2] = m[h];
            part_ml[row * 2 + 1] = l[h];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) part_o[row * D + c * 8 + e] = o[h][e];
    }
}

__global__ void __launch_bounds__(512)
attn_merge_kernel(const float *__restrict__ part_o, const float *__restrict__ part_ml,
                  uint16_t *__restrict__ Out, int Hq, int D, int S)
{
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    if (d >= D) return;
    const size_t base = ((size_t)b * Hq + h) * S;
    float M = kNegInf;
    for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[(base + s) * 2]);
    float z = 0.f, acc = 0.f;
    if (M != kNegInf) {
        for (int s = 0; s < S; ++s) {
            const float ls = part_ml[(base + s) * 2 + 1];
            if (ls > 0.f) {
                const float a = exp2_guarded(part_ml[(base + s) * 2] - M);
                z = fmaf(ls, a, z);
                acc = fmaf(part_o[(base + s) * D + d], a, acc);
            }
        }
    }
    Out[((size_t)b * Hq + h) * D + d] = to_out<DT_BF16>(z > 0.f ? acc / z : 0.f);
}

template <int D, int G>
static hipError_t launch_segments(const AttentionLaunch &A, float *po, float *pml, hipStream_t st)
{
    const float log2e = 1.4426950408889634f;
    dim3 grid((unsigned)A.S, (unsigned)A.Hkv, (unsigned)A.B);
    hipLaunchKernelGGL((attn_segment_kernel<D, G>), grid, dim3(kAttnWaves * 64), 0, st, A.Q, A.Kc,
                       A.Vc, A.block_table, A.seq_lens, po, pml, A.Hq, A.Hkv, A.block_size,
                       A.max_blocks, A.num_blocks, A.scale * log2e, A.S);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttentionLaunch &A, float *po, float *pml, hipStream_t st)
{
    switch (A.Hq / A.Hkv) {
    case 1: return launch_segments<D, 1>(A, po, pml, st);
    case 2: return launch_segments<D, 2>(A, po, pml, st);
    case 4: return launch_segments<D, 4>(A, po, pml, st);
    case 8: return launch_segments<D, 8>(A, po, pml, st);
    }
    return hipErrorInvalidValue;
}

size_t attention_workspace_bytes(int B, int Hq, int D, int S)
{
    return (size_t)B * Hq * S * ((size_t)D + 2) * sizeof(float);
}

hipError_t attention_launch(const AttentionLaunch &A, hipStream_t st)
{
    float *po = (float *)A.workspace;
    float *pml = po + (size_t)A.B * A.Hq * A.S * A.D;
    hipError_t e = hipErrorInvalidValue;
    switch (A.D) {
    case 64: e = launch_d<64>(A, po, pml, st); break;
    case 128: e = launch_d<128>(A, po, pml, st); break;
    case 256: e = launch_d<256>(A, po, pml, st); break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)A.Hq, (unsigned)A.B), dim3(A.D), 0, st,
                       po, pml, A.Out, A.Hq, A.D, A.S);
    return hipGetLastError();
}

}  // namespace migemm
