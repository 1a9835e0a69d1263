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
// together; up to 4 query heads of the kv head share every K and V load (a
// larger group is split over workgroups, whose second read of the rows the
// caches serve).  A K or V row of D BF16 values is D/8 lanes x 16 bytes, so
// one wave load reads 64/(D/8) whole rows (2 rows of 512 B at D = 256): full
// cache lines.  The 4 waves split the segment's tokens and walk them in
// steps of 16 tokens, double-buffered in registers: the next step's K rows
// are requested before a step and its V rows half way through it (before
// prob V), the page ids of the step after that on their way (each lane
// reads the block-table entry of its own row).  Per
// step, q K^T is one 16-token x 16-head tile on the matrix cores, the
// online softmax runs once per (token, head), and prob V runs on the vector
// ALUs; the details are at the kernel.  At the end the token slots of a
// wave and then the 4 waves are merged, and the segment's (max,
// denominator, unnormalised output) go to the workspace in FP32.
//
// Merge kernel: one workgroup per (query head, sequence, 64 output
// columns); each thread merges a sixteenth of the segments of its column
// online (log-sum-exp), the sixteen are merged through LDS, then one
// division and one rounding to BF16.  Empty segments (max = -inf, denominator 0) add
// nothing; a sequence with no token gives zeros.  Tokens whose page id is
// outside [0, num_blocks) add nothing: their rows are read from a block of
// zeros and their scores are -inf.
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

// 16 zero bytes in device memory: masked K and V rows load from here, so a
// token past the range or on an invalid page contributes exact zeros (row 0
// of a cache page could hold anything).
__device__ const uint16_t kAttnZeros[8] = {0, 0, 0, 0, 0, 0, 0, 0};

typedef const __attribute__((address_space(1))) u32x4 *attn_gptr16;

// One step of 16 tokens:
//  * scores: the step's K rows (loaded in the row layout) are written to a
//    wave-private LDS tile, row t's 16-byte piece x at t*2D + 16*(x ^ f(t)),
//    and read back as A operands of v_mfma_f32_16x16x32_bf16 (token l%16,
//    d 32*kk + 8*(l/16)); Q^T of the G query heads is the B operand (head
//    l%16, zero past G), read from a copy staged once in LDS;
//  * softmax once per (token, head) in the MFMA result layout (lane l:
//    head l%16, tokens 4*(l/16) .. +3): step max over the 16 tokens, one
//    rescale of the running state per head (kept per lane, the same in the
//    4 lanes of a head), exp2, the running denominator;
//  * prob x V on the VALU in the row layout, each lane reading its token's
//    probabilities and the step's per-head rescale from LDS.  All token
//    slots of a wave share one running maximum, so the slots add up at the
//    end without rescaling; the 4 waves then merge through LDS.
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
    constexpr int T = 16;               // tokens per step: one MFMA tile
    constexpr int U = T / TPI;          // wave loads of K (and of V) per step
    constexpr int KS = D / 32;          // MFMA k-steps over the head dim
    constexpr int KROW = 2 * D;         // bytes of one staged K row
    static_assert(D % 64 == 0 && D <= 256 && G <= 4, "shape");
    __shared__ __attribute__((aligned(16))) uint8_t kt[kAttnWaves][T * KROW];
    __shared__ __attribute__((aligned(16))) float pt[kAttnWaves][T][4];    // probabilities [token][head]
    __shared__ __attribute__((aligned(16))) float ct[kAttnWaves][4];       // per-head rescale of a step
    __shared__ __attribute__((aligned(16))) float vt[kAttnWaves][T];       // 0 or -inf per token
    __shared__ __attribute__((aligned(16))) uint16_t qt[16][D + 8];        // Q^T operand rows
    __shared__ float xs[kAttnWaves][G][2 + D];

    const int parts = group / G;
    const int kvh = blockIdx.x / parts, s = blockIdx.y, b = blockIdx.z;
    const int h0 = kvh * group + (blockIdx.x % parts) * G;
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int slot = lane / CPL, c = lane % CPL;
    const int g = lane >> 4, r16 = lane & 15;

    int L = seq_lens[b];
    L = L < 0 ? 0 : (L > max_blocks * block_size ? max_blocks * block_size : L);
    const int seg = (L + S - 1) / S;
    const int l0 = min(L, s * seg), l1 = min(L, l0 + seg);
    const int per = (l1 - l0 + kAttnWaves - 1) / kAttnWaves;
    const int w0 = min(l1, l0 + wave * per), w1 = min(l1, w0 + per);

    // Q^T as B operands, staged once in LDS: row h < G holds query head
    // h0 + h, rows G .. 15 are zero; lane (g, h) reads Q[h0 + h][32 kk + 8 g .. +7].
    // Requested first, stored after the first K/V requests, so that its
    // latency overlaps the block-table lookups instead of preceding them.
    constexpr int QP = (16 * (D / 8) + kAttnWaves * 64 - 1) / (kAttnWaves * 64);
    u32x4 qv[QP];
#pragma unroll
    for (int p = 0; p < QP; ++p) {
        const int i = threadIdx.x + p * kAttnWaves * 64;
        const int h = i / (D / 8), x = i % (D / 8);
        qv[p] = *(attn_gptr16)(i < 16 * (D / 8) && h < G ? Q + ((size_t)b * Hq + h0 + h) * D + 8 * x
                                                         : kAttnZeros);
    }
    auto store_q = [&]() {
#pragma unroll
        for (int p = 0; p < QP; ++p) {
            const int i = threadIdx.x + p * kAttnWaves * 64;
            if (i < 16 * (D / 8)) *(u32x4 *)&qt[i / (D / 8)][8 * (i % (D / 8))] = qv[p];
        }
        __syncthreads();
    };

    float mrun = kNegInf, lrun = 0.f;      // head r16's running max (log2 units) and denominator
    float o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;

    const int32_t *bt = block_table + (size_t)b * max_blocks;
    const size_t row_stride = (size_t)Hkv * D;
    const size_t lane_off = (size_t)kvh * D + c * 8;
    const float inv_bs = 1.0f / (float)block_size;
    uint8_t *ktw = kt[wave];
    // swizzle of a staged K row: keeps the 16 rows of an operand read in
    // distinct banks
    auto swz = [](int t) { return D == 64 ? (t >> 1) & 7 : t & 15; };

    // Page id of every row this lane loads in the step starting at t (-1
    // past the range); each lane reads its own token's block-table entry.
    auto page_ids = [&](int t, int (&pg)[U]) {
        const int pf = t / block_size;
        const int r0 = t - pf * block_size;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int rel = r0 + TPI * u + slot;
            int idx = (int)((float)rel * inv_bs);
            const int i = rel - idx * block_size;
            idx += i < 0 ? -1 : (i >= block_size ? 1 : 0);
            const int v = bt[min(pf + idx, max_blocks - 1)];
            pg[u] = t + TPI * u + slot < w1 ? v : -1;
        }
    };
    // K loads of a step (non-temporal), keeping each row's validity and
    // offset for the V loads; masked rows read zeros
    auto issue_k = [&](int t, const int (&pg)[U], u32x4 (&kr)[U], bool (&ok)[U], size_t (&of)[U]) {
        const int pf = t / block_size;
        const int r0 = t - pf * block_size;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int rel = r0 + TPI * u + slot;
            int idx = (int)((float)rel * inv_bs);
            int in = rel - idx * block_size;
            if (in < 0) in += block_size;
            else if (in >= block_size) in -= block_size;
            ok[u] = pg[u] >= 0 && pg[u] < num_blocks;
            of[u] = ((size_t)pg[u] * block_size + in) * row_stride + lane_off;
            kr[u] = __builtin_nontemporal_load((attn_gptr16)(ok[u] ? Kc + of[u] : kAttnZeros));
        }
    };
    auto issue_v = [&](u32x4 (&vr)[U], const bool (&ok)[U], const size_t (&of)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            vr[u] = __builtin_nontemporal_load((attn_gptr16)(ok[u] ? Vc + of[u] : kAttnZeros));
    };

    // `mid` runs between the softmax and prob x V: it requests the next
    // step's V rows, so about one and a half steps of K and V are in flight
    // (measured: faster than two whole steps, and than one)
    auto step = [&](const u32x4 (&kr)[U], const u32x4 (&vr)[U], const bool (&ok)[U], auto &&mid) {
        // K rows into the tile, token validity beside them
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = TPI * u + slot;
            *(u32x4 *)(ktw + t * KROW + 16 * (c ^ swz(t))) = kr[u];
            if (c == 0) vt[wave][t] = ok[u] ? 0.f : kNegInf;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);             // lgkmcnt(0): wave-private tile
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const u32x4 a = *(const u32x4 *)(ktw + r16 * KROW + 16 * ((4 * kk + g) ^ swz(r16)));
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, *(const u32x4 *)&qt[r16][32 * kk + 8 * g]),
                                                          sacc, 0, 0, 0);
        }
        // softmax bookkeeping for head r16 over tokens 4g .. 4g+3 of the tile
        const f32x4 valid = *(const f32x4 *)&vt[wave][4 * g];
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[r] = fmaf(sacc[r], qscale, valid[r]);
        float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mn = fmaxf(mrun, mt);
        const float ref = mn == kNegInf ? 0.f : mn;     // exp2(-inf - ref) = 0 while nothing is seen
        const float corr = __builtin_amdgcn_exp2f(mrun - ref);
        float p[4], psum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = __builtin_amdgcn_exp2f(sv[r] - ref);
            psum += p[r];
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        lrun = lrun * corr + psum;
        mrun = mn;
        if (r16 < G) {
#pragma unroll
            for (int r = 0; r < 4; ++r) pt[wave][4 * g + r][r16] = p[r];
            if (g == 0) ct[wave][r16] = corr;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        mid();
        // prob x V for this lane's tokens
        const f32x4 cr = *(const f32x4 *)ct[wave];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] *= cr[h];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const f32x4 pp = *(const f32x4 *)pt[wave][TPI * u + slot];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v0 = __builtin_bit_cast(float, vr[u][e] << 16);
                const float v1 = __builtin_bit_cast(float, vr[u][e] & 0xffff0000u);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    o[h][2 * e] = fmaf(pp[h], v0, o[h][2 * e]);
                    o[h][2 * e + 1] = fmaf(pp[h], v1, o[h][2 * e + 1]);
                }
            }
        }
    };

    // two register buffers: while one step is computed the next one's K is
    // in flight and its V is requested half way; each step's page ids are
    // requested two steps ahead
    u32x4 ka[U], va[U], kb2[U], vb2[U];
    bool oka[U], okb[U];
    size_t oa[U], ob[U];
    int pa[U], pb[U];
    page_ids(w0, pa);
    page_ids(w0 + T, pb);
    issue_k(w0, pa, ka, oka, oa);
    issue_v(va, oka, oa);
    store_q();
    for (int t0 = w0; t0 < w1; t0 += 2 * T) {
        page_ids(t0 + 2 * T, pa);
        issue_k(t0 + T, pb, kb2, okb, ob);
        step(ka, va, oka, [&] { issue_v(vb2, okb, ob); });
        if (t0 + T >= w1) break;
        page_ids(t0 + 3 * T, pb);
        issue_k(t0 + 2 * T, pa, ka, oka, oa);
        step(kb2, vb2, okb, [&] { issue_v(va, oka, oa); });
    }

    // the token slots of a wave share the running max: add their outputs
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int x = CPL; x < 64; x <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][e] += __shfl_xor(o[h][e], x, 64);
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[wave][h][2 + c * 8 + e] = o[h][e];
    }
    if (g == 0 && r16 < G) {
        xs[wave][r16][0] = mrun;
        xs[wave][r16][1] = lrun;
    }
    __syncthreads();
    if (wave != 0 || slot != 0) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float m = xs[0][h][0], l = xs[0][h][1], acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = xs[0][h][2 + c * 8 + e];
#pragma unroll
        for (int w = 1; w < kAttnWaves; ++w) {
            float o2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o2[e] = xs[w][h][2 + c * 8 + e];
            merge_state(m, l, acc, xs[w][h][0], xs[w][h][1], o2);
        }
        const size_t row = ((size_t)b * Hq + h0 + h) * S + s;
        if (c == 0) {
            part_ml[row * 2] = m;
            part_ml[row * 2 + 1] = l;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) part_o[row * D + c * 8 + e] = acc[e];
    }
}

constexpr int kMaxSegments = 1024;
constexpr int kMergeRows = 16;           // segment rows per merge workgroup
constexpr int kMergeBatch = 8;           // rows a thread loads before merging them

// grid (query head, sequence, 64-column chunk), 1024 threads: thread
// (r, col) merges segments r, r + 16, ... of its column online, loading 8
// rows at a time before using any (the partials come from other XCDs'
// writes: one trip to memory per batch, not per row), then the 16 rows are
// merged through LDS.
__global__ void __launch_bounds__(64 * kMergeRows)
attn_merge_kernel(const float *__restrict__ part_o, const float *__restrict__ part_ml,
                  uint16_t *__restrict__ Out, int Hq, int D, int S)
{
    __shared__ float sm[kMergeRows][64], sz[kMergeRows][64], so[kMergeRows][64];
    const int h = blockIdx.x, b = blockIdx.y;
    const int col = blockIdx.z * 64 + (threadIdx.x & 63), r = threadIdx.x >> 6;
    const size_t base = ((size_t)b * Hq + h) * S;

    float m = kNegInf, z = 0.f, acc = 0.f;
    for (int s0 = r; s0 < S; s0 += kMergeRows * kMergeBatch) {
        float ms[kMergeBatch], ls[kMergeBatch], os[kMergeBatch];
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
            const int s = s0 + i * kMergeRows;
            const size_t row = base + (s < S ? s : r);            // past S: row r again, ignored
            ms[i] = part_ml[row * 2];
            ls[i] = part_ml[row * 2 + 1];
            os[i] = part_o[row * D + col];
            if (s >= S) ms[i] = kNegInf;
        }
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
            const float mn = fmaxf(m, ms[i]);
            const float a = mn == kNegInf ? 0.f : exp2_guarded(m - mn);
            const float w = mn == kNegInf ? 0.f : exp2_guarded(ms[i] - mn);
            z = z * a + ls[i] * w;
            acc = acc * a + os[i] * w;
            m = mn;
        }
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
