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
// Segment kernel: one workgroup (4 waves) per (kv head, segment, sequence),
// kv heads fastest so the workgroups reading the same token rows run
// together.  A K or V row of D BF16 values is D/8 lanes x 16 bytes, so one
// wave load reads 64/(D/8) whole rows (2 rows of 512 B at D = 256): full
// cache lines, every 4 lanes contiguous.  Up to 4 query heads of the kv head
// share every K and V load.  Each lane keeps its 8 elements of q (per head,
// pre-multiplied by scale * log2 e so that exponentials are powers of two)
// and its 8 elements of the running output; a token's score is the dot
// product summed across its D/8 lanes with DPP row operations (and one
// swizzle at D = 256).  The 4 waves split the segment's tokens and walk
// them in steps of 4 wave loads of K and of V, triple-buffered in
// registers: while a step is computed the next two steps' rows are in
// flight, and the page ids of the step after those (each lane reads the
// block-table entry of its own row) are on their way.
// Per step and head: one rescale of the running state, then exp2 and
// prob * V, branch-free.  At the end the token slots of a wave and then
// the 4 waves are merged, and the segment's (max, denominator,
// unnormalised output) go to the workspace in FP32.
//
// Merge kernel: one workgroup per (query head, sequence, 64 output
// columns); each thread merges a quarter of the segments of its column
// online (log-sum-exp), the quarters are merged through LDS, then one
// division and one rounding to BF16.  Empty segments (max = -inf, denominator 0) add
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

// (m, l, o) <- merge of itself and (m2, l2, o2) for one head, maxima in
// log2 units
__device__ inline void merge_state(float &m, float &l, float (&o)[8], float m2, float l2,
                                   const float (&o2)[8])
{
    const float mn = fmaxf(m, m2);
    const float a = (mn == kNegInf) ? 0.f : exp2_guarded(m - mn);
    const float b = (mn == kNegInf) ? 0.f : exp2_guarded(m2 - mn);
    l = l * a + l2 * b;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * a + o2[e] * b;
    m = mn;
}

}  // namespace

// Sum over aligned groups of CPL lanes (8, 16 or 32), the total in every
// lane of the group: DPP row rotations and quad permutes within a row of 16
// lanes, one swizzle across the two rows of a 32-lane group.
template <int CTRL>
__device__ inline float dpp_f(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xf, 0xf, true));
}

template <int CPL>
__device__ inline float group_sum(float x)
{
    if constexpr (CPL >= 16) {
        x += dpp_f<0x128>(x);                        // row_ror:8
        x += dpp_f<0x124>(x);                        // row_ror:4
    }
    x += dpp_f<0x4e>(x);                             // quad_perm [2,3,0,1]
    x += dpp_f<0xb1>(x);                             // quad_perm [1,0,3,2]
    if constexpr (CPL == 8) x += dpp_f<0x141>(x);    // row_half_mirror: the other quad
    if constexpr (CPL == 32)                         // lane ^ 16 within 32 lanes
        x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401f));
    return x;
}

// G query heads per workgroup: all of a kv head's group when it has up to
// 4 heads, else 4 of them (the workgroups of one kv head then read the same
// K and V rows; the second read is served by the caches).
template <int D, int G>
__global__ void __launch_bounds__(kAttnWaves * 64)
attn_segment_kernel(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kc,
                    const uint16_t *__restrict__ Vc, const int32_t *__restrict__ block_table,
                    const int32_t *__restrict__ seq_lens, float *__restrict__ part_o,
                    float *__restrict__ part_ml, int Hq, int Hkv, int group, int block_size,
                    int max_blocks, int num_blocks, float qscale, int S)
{
    constexpr int CPL = D / 8;          // lanes per cached row (16 bytes each)
    constexpr int TPI = 64 / CPL;       // rows per wave load
    constexpr int U = 4;                // wave loads of K (and of V) per step
    constexpr int T = TPI * U;          // tokens per wave step (<= 64)
    static_assert(D % 64 == 0 && D <= 256 && T <= 64, "head dim");
    __shared__ float xs[kAttnWaves][G][2 + D];

    const int parts = group / G;                        // workgroups per kv head
    const int kvh = blockIdx.x / parts, s = blockIdx.y, b = blockIdx.z;
    const int h0 = kvh * group + (blockIdx.x % parts) * G;  // first query head
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
        const u32x4 v = *(const u32x4 *)(Q + ((size_t)b * Hq + h0 + h) * D + c * 8);
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
    const size_t lane_off = (size_t)kvh * D + c * 8;
    const float inv_bs = 1.0f / (float)block_size;

    // Page id and slot of every row this lane loads in the step starting
    // at token t (id -1 past the range).  Each lane reads the block-table
    // entry of its own token (lanes on one page share the address); the
    // read itself is unconditional, from a clamped index.
    auto page_ids = [&](int t, int (&pg)[U], int (&in)[U]) {
        const int pf = t / block_size;
        const int r0 = t - pf * block_size;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int rel = r0 + TPI * u + slot;                 // < block_size + T
            int idx = (int)((float)rel * inv_bs);
            int i = rel - idx * block_size;
            if (i < 0) { --idx; i += block_size; }
            else if (i >= block_size) { ++idx; i -= block_size; }
            in[u] = i;
            const int v = bt[min(pf + idx, max_blocks - 1)];
            pg[u] = t + TPI * u + slot < w1 ? v : -1;
        }
    };
    // K and V loads (non-temporal: every row is read once) of one step.  A
    // row past the range or on an invalid page loads row 0 of the cache
    // (always in bounds) and is masked out by ok.
    auto issue = [&](const int (&pg)[U], const int (&in)[U], u32x4 (&kr)[U], u32x4 (&vr)[U],
                     bool (&ok)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ok[u] = pg[u] >= 0 && pg[u] < num_blocks;
            const size_t off = ok[u] ? ((size_t)pg[u] * block_size + in[u]) * row_stride + lane_off : 0;
            kr[u] = __builtin_nontemporal_load((const u32x4 *)(Kc + off));
            vr[u] = __builtin_nontemporal_load((const u32x4 *)(Vc + off));
        }
    };

    // One step: scores of the U x TPI tokens for the G heads (dot product
    // over the CPL lanes of a row), one rescale of the running state per
    // head, then prob * V.
    auto step = [&](const u32x4 (&kr)[U], const u32x4 (&vr)[U], const bool (&ok)[U]) {
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[2 * e] = __builtin_bit_cast(float, kr[u][e] << 16);
                kf[2 * e + 1] = __builtin_bit_cast(float, kr[u][e] & 0xffff0000u);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) p = fmaf(q[h][e], kf[e], p);
                p = group_sum<CPL>(p);
                sc[u][h] = ok[u] ? p : kNegInf;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mb = sc[0][h];
#pragma unroll
            for (int u = 1; u < U; ++u) mb = fmaxf(mb, sc[u][h]);
            const float mn = fmaxf(m[h], mb);
            // branch-free: while nothing has been seen, any finite reference
            // gives exp2(-inf - ref) = 0 (v_exp_f32 maps -inf to +0)
            const float ref = mn == kNegInf ? 0.f : mn;
            const float corr = __builtin_amdgcn_exp2f(m[h] - ref);
            l[h] *= corr;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= corr;
            m[h] = mn;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = __builtin_amdgcn_exp2f(sc[u][h] - ref);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[h][2 * e] = fmaf(p, __builtin_bit_cast(float, vr[u][e] << 16), o[h][2 * e]);
                    o[h][2 * e + 1] = fmaf(p, __builtin_bit_cast(float, vr[u][e] & 0xffff0000u), o[h][2 * e + 1]);
                }
            }
        }
    };

    // Three register buffers rotate: while one step is computed, the next
    // two steps' K and V are in flight.  The page ids of the step after
    // those are requested before the K and V loads issued alongside, so
    // waiting for the ids never waits for the newest loads.
    u32x4 ka[U], va[U], kb[U], vb[U], kx[U], vx[U];
    bool oka[U], okb[U], okx[U];
    int pa[U], ia[U], pb[U], ib[U], px[U], ix[U];
    page_ids(w0, pa, ia);
    page_ids(w0 + T, pb, ib);
    page_ids(w0 + 2 * T, px, ix);
    issue(pa, ia, ka, va, oka);
    issue(pb, ib, kb, vb, okb);
    for (int t0 = w0; t0 < w1; t0 += 3 * T) {
        page_ids(t0 + 3 * T, pa, ia);
        issue(px, ix, kx, vx, okx);
        step(ka, va, oka);
        if (t0 + T >= w1) break;
        page_ids(t0 + 4 * T, pb, ib);
        issue(pa, ia, ka, va, oka);
        step(kb, vb, okb);
        if (t0 + 2 * T >= w1) break;
        page_ids(t0 + 5 * T, px, ix);
        issue(pb, ib, kb, vb, okb);
        step(kx, vx, okx);
    }

    // merge the token slots of the wave (lanes c, c + CPL, ...), one head
    // at a time
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int x = CPL; x < 64; x <<= 1) {
            float o2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[h][e], x, 64);
            merge_state(m[h], l[h], o[h], __shfl_xor(m[h], x, 64), __shfl_xor(l[h], x, 64), o2);
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
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int w = 1; w < kAttnWaves; ++w) {
            float o2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o2[e] = xs[w][h][2 + c * 8 + e];
            merge_state(m[h], l[h], o[h], xs[w][h][0], xs[w][h][1], o2);
        }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const size_t row = ((size_t)b * Hq + h0 + h) * S + s;
        if (c == 0) {
            part_ml[row * 2] = m[h];
            part_ml[row * 2 + 1] = l[h];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) part_o[row * D + c * 8 + e] = o[h][e];
    }
}

constexpr int kMaxSegments = 1024;
constexpr int kMergeRows = 4;            // segment rows per merge workgroup

// grid (query head, sequence, 64-column chunk), 256 threads: thread
// (r, col) merges segments r, r + 4, ... of its column online (all loads
// independent of each other), then the 4 rows are merged through LDS.
__global__ void __launch_bounds__(64 * kMergeRows)
attn_merge_kernel(const float *__restrict__ part_o, const float *__restrict__ part_ml,
                  uint16_t *__restrict__ Out, int Hq, int D, int S)
{
    __shared__ float sm[kMergeRows][64], sz[kMergeRows][64], so[kMergeRows][64];
    const int h = blockIdx.x, b = blockIdx.y;
    const int col = blockIdx.z * 64 + (threadIdx.x & 63), r = threadIdx.x >> 6;
    const size_t base = ((size_t)b * Hq + h) * S;

    float m = kNegInf, z = 0.f, acc = 0.f;
#pragma unroll 8
    for (int s = r; s < S; s += kMergeRows) {
        const float ms = part_ml[(base + s) * 2], ls = part_ml[(base + s) * 2 + 1];
        const float os = part_o[(base + s) * D + col];
        const float mn = fmaxf(m, ms);
        const float a = mn == kNegInf ? 0.f : exp2_guarded(m - mn);
        const float w = mn == kNegInf ? 0.f : exp2_guarded(ms - mn);
        z = z * a + ls * w;
        acc = acc * a + os * w;
        m = mn;
    }
    sm[r][threadIdx.x & 63] = m;
    sz[r][threadIdx.x & 63] = z;
    so[r][threadIdx.x & 63] = acc;
    __syncthreads();
    if (r != 0) return;
    const int c = threadIdx.x;
#pragma unroll
    for (int rr = 1; rr < kMergeRows; ++rr) {
        const float ms = sm[rr][c];
        const float mn = fmaxf(m, ms);
        const float a = mn == kNegInf ? 0.f : exp2_guarded(m - mn);
        const float w = mn == kNegInf ? 0.f : exp2_guarded(ms - mn);
        z = z * a + sz[rr][c] * w;
        acc = acc * a + so[rr][c] * w;
        m = mn;
    }
    Out[((size_t)b * Hq + h) * D + col] = to_out<DT_BF16>(z > 0.f ? acc / z : 0.f);
}

template <int D, int G>
static hipError_t launch_segments(const AttentionLaunch &A, float *po, float *pml, hipStream_t st)
{
    const float log2e = 1.4426950408889634f;
    const int group = A.Hq / A.Hkv;
    dim3 grid((unsigned)(A.Hkv * (group / G)), (unsigned)A.S, (unsigned)A.B);
    hipLaunchKernelGGL((attn_segment_kernel<D, G>), grid, dim3(kAttnWaves * 64), 0, st, A.Q, A.Kc,
                       A.Vc, A.block_table, A.seq_lens, po, pml, A.Hq, A.Hkv, group,
                       A.block_size, A.max_blocks, A.num_blocks, A.scale * log2e, A.S);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttentionLaunch &A, float *po, float *pml, hipStream_t st)
{
    switch (A.Hq / A.Hkv) {
    case 1: return launch_segments<D, 1>(A, po, pml, st);
    case 2: return launch_segments<D, 2>(A, po, pml, st);
    case 4: return launch_segments<D, 4>(A, po, pml, st);
    case 8: return launch_segments<D, 4>(A, po, pml, st);
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
    if (A.S > kMaxSegments) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)A.Hq, (unsigned)A.B, (unsigned)(A.D / 64)),
                       dim3(64 * kMergeRows), 0, st, po, pml, A.Out, A.Hq, A.D, A.S);
    return hipGetLastError();
}

}  // namespace migemm
