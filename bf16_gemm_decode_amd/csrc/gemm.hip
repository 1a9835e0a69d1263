// gemm.hip -- dense column-major C = A x B on gfx950 MFMA.
//
// Defined by the MTT S4000 GEMM write-up (blog.mthreads.com GEMM03):
// section 1 (16-bit inputs, FP32 accumulation, 16-bit output, column-major),
// section 2 (C(m,n) = sum_k A(m,k) B(k,n), A(m,k) = A[m + k*M],
// B(k,n) = B[k + n*K], C(m,n) = C[m + n*M]).  The kernel design is ours:
//
//  * one workgroup owns a BM x BN tile of C, picked by tile_coord() (XCD
//    renumbering + the grouped ordering of the FlagGems Hygon page);
//  * K advances in BK-wide steps through a ring of S LDS stages.  Each step's
//    A tile (BK rows of BM m-contiguous elements) and B tile (BN rows of BK
//    k-contiguous elements) go straight from HBM into LDS with buffer loads
//    that write LDS directly (no VGPR staging), S-2 steps ahead of the step
//    being computed;
//  * A is m-contiguous, but an MFMA operand needs 8 consecutive k of one row
//    per lane, so A is read out of LDS with the transposing ds_read_b64_tr_b16
//    (lane i of each 16-lane group receives row i of a 16 x 4 block); B is
//    already k-contiguous and is read with ds_read_b128;
//  * operand fragments are double-buffered in registers: the LDS reads of the
//    next 32-wide k slice (including the first slice of the next step, right
//    after the step's barrier) are issued before the MFMAs of the current one;
//  * v_mfma_f32_16x16x32_{f16,bf16} accumulates in FP32 registers;
//  * out-of-range rows/columns are never stored; out-of-range k reads as
//    zero through the buffer descriptors' range check, so ragged K needs no
//    separate path;
//  * the epilogue rounds each FP32 sum once to FP16/BF16 (nearest even) and
//    stores it directly: no FP32 copy of C ever reaches memory.
#include "common.hpp"
#include "tile_map.hpp"
#include "kernels.hpp"

namespace migemm {

// LDS swizzles: XOR on the 16-byte chunk index within a row, so the rows a
// 16-lane group reads in one LDS instruction fall in different banks.
// A stage rows are k (BM elements each); B stage rows are n (BK elements).
template <int BM>
__device__ inline int swz_a(int kk) { return (((kk & 7) << 1) ^ (kk & 8)) & (BM / 8 - 1); }
template <int BK>
__device__ inline int swz_b(int nn)
{
    if constexpr (BK == 64)
        return (nn ^ (nn >> 3)) & 7;
    else
        return ((nn >> 1) ^ (nn >> 3)) & 3;
}

// Raw buffer descriptor words over [base, base + nbytes), wave-uniform:
// loads past nbytes return zero and never fault.  Word 3 selects 32-bit data
// format, no swizzle; the stride is zero (raw byte offsets).
__device__ inline u32x4 make_desc(const void *base, uint32_t nbytes)
{
    uint64_t a = (uint64_t)base;
    u32x4 d;
    d[0] = (uint32_t)uniform((int)(uint32_t)a);
    d[1] = (uint32_t)uniform((int)((uint32_t)(a >> 32) & 0xffffu));
    d[2] = (uint32_t)uniform((int)nbytes);
    d[3] = 0x00020000u;
    return d;
}

// Direct HBM -> LDS load of BYTES per lane: lane l's bytes land at LDS address
// lds + l*BYTES (M0 holds the wave-uniform base).  Only the 4- and 16-byte
// forms are used; their lane-linear placement and zero fill past the
// descriptor's records are what the kernel relies on.  Issued as inline
// assembly so that the compiler does not make every later LDS read wait for
// these loads: the kernel orders them itself with explicit vmcnt waits and a
// barrier before any wave reads the stage they fill.
template <int BYTES>
__device__ inline void dma_to_lds(u32x4 desc, uint32_t lds, uint32_t voff)
{
    static_assert(BYTES == 16 || BYTES == 4, "LDS load size");
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                     :: "v"(voff), "s"(lds), "s"(desc) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, 0 offen lds"
                     :: "v"(voff), "s"(lds), "s"(desc) : "memory", "m0");
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15).
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int DT>
__device__ inline f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int DT, int BM, int BN, int BK, int WGM, int WGN, int S, int VA, int VB, int OCC>
__global__ void __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
gemm_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
            uint16_t *__restrict__ C, int M, int N, int K, int num_pid_m, int num_pid_n,
            int group_m, int num_xcd, int c_vec)
{
    constexpr int NW = WGM * WGN;
    constexpr int TM = BM / WGM, TN = BN / WGN;   // wave tile
    constexpr int FM = TM / 16, FN = TN / 16;     // 16x16 MFMA blocks per wave
    constexpr int KS = BK / 32;                   // 32-wide k slices per K-step
    constexpr int A_BYTES = BK * BM * 2, B_BYTES = BN * BK * 2;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_PIECE = 64 * VA * 2, B_PIECE = 64 * VB * 2;   // bytes per wave load
    constexpr int A_LOADS = A_BYTES / (A_PIECE * NW), B_LOADS = B_BYTES / (B_PIECE * NW);
    // direct-to-LDS loads per wave per K-step (single-element paths are synchronous)
    constexpr int LPS = (VA > 1 ? A_LOADS : 0) + (VB > 1 ? B_LOADS : 0);
    static_assert(A_BYTES % (A_PIECE * NW) == 0 && B_BYTES % (B_PIECE * NW) == 0, "loader split");
    static_assert(TM % 16 == 0 && TN % 16 == 0 && BK % 32 == 0, "tile shape");
    static_assert(S >= 3 && S * STAGE <= 163840, "LDS ring");
    static_assert(LPS * (S - 2) < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[S * STAGE];

    int pid_m, pid_n;
    tile_coord<int>((int)blockIdx.x, num_pid_m, num_pid_n, group_m, num_xcd, pid_m, pid_n);
    const int m0 = pid_m * BM, n0 = pid_n * BN;
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int wm = wave % WGM, wn = wave / WGM;
    const int g = lane >> 4, ig = lane & 15;

    // Which global element each lane fetches for each of its loads.  A load
    // writes lane-linear LDS bytes [piece + lane*size, +size); the swizzle is
    // applied by choosing the global source of that LDS slot.
    uint32_t a_off[A_LOADS];
#pragma unroll
    for (int q = 0; q < (VA > 1 ? A_LOADS : 0); ++q) {
        int P = (q * NW + wave) * A_PIECE + lane * VA * 2;
        int kk = P / (BM * 2), b = P % (BM * 2);
        int m = (((b >> 4) ^ swz_a<BM>(kk)) << 3) + ((b & 15) >> 1);
        a_off[q] = (uint32_t)(((int64_t)kk * M + m0 + m) * 2);
    }
    uint32_t b_off[B_LOADS];
    int b_k[B_LOADS];
#pragma unroll
    for (int q = 0; q < (VB > 1 ? B_LOADS : 0); ++q) {
        int P = (q * NW + wave) * B_PIECE + lane * VB * 2;
        int nn = P / (BK * 2), b = P % (BK * 2);
        int kk = (((b >> 4) ^ swz_b<BK>(nn)) << 3) + ((b & 15) >> 1);
        b_off[q] = (uint32_t)(((int64_t)nn * K + kk) * 2);
        b_k[q] = kk;
    }

    // Issue the loads of the K-step starting at k0 into stage `st`.
    // Descriptors are rebased per step: A at column k0 with (K - k0) columns
    // of records, so k >= K reads zero; B at column n0, row k0, where rows
    // n >= N fall past the records and k >= K is pushed out of range.
    auto issue = [&](int st, int k0) {
        MIGEMM_LDS unsigned char *sa = (MIGEMM_LDS unsigned char *)(smem + st * STAGE);
        MIGEMM_LDS unsigned char *sb = sa + A_BYTES;
        if constexpr (VA > 1) {
            const u32x4 da = make_desc(A + (size_t)k0 * M, clamp_records((int64_t)(K - k0) * M * 2));
            const uint32_t base = (uint32_t)(uintptr_t)sa;
#pragma unroll
            for (int q = 0; q < A_LOADS; ++q)
                dma_to_lds<VA * 2>(da, (uint32_t)uniform((int)(base + (q * NW + wave) * A_PIECE)), a_off[q]);
        } else {
            // one element per lane through a register: zero outside the matrix
#pragma unroll
            for (int q = 0; q < A_LOADS; ++q) {
                int P = (q * NW + wave) * A_PIECE + lane * 2;
                int kk = P / (BM * 2), b = P % (BM * 2);
                int m = (((b >> 4) ^ swz_a<BM>(kk)) << 3) + ((b & 15) >> 1);
                uint16_t v = 0;
                if (m0 + m < M && k0 + kk < K) v = A[(size_t)(k0 + kk) * M + m0 + m];
                *(MIGEMM_LDS uint16_t *)(sa + P) = v;
            }
        }
        if constexpr (VB > 1) {
            const u32x4 db = make_desc(B + (size_t)n0 * K + k0,
                                       clamp_records((int64_t)(N - n0) * K * 2 - (int64_t)k0 * 2));
            const uint32_t base = (uint32_t)(uintptr_t)sb;
#pragma unroll
            for (int q = 0; q < B_LOADS; ++q) {
                uint32_t off = (k0 + b_k[q] < K) ? b_off[q] : kOutOfRange;
                dma_to_lds<VB * 2>(db, (uint32_t)uniform((int)(base + (q * NW + wave) * B_PIECE)), off);
            }
        } else {
#pragma unroll
            for (int q = 0; q < B_LOADS; ++q) {
                int P = (q * NW + wave) * B_PIECE + lane * 2;
                int nn = P / (BK * 2), b = P % (BK * 2);
                int kk = (((b >> 4) ^ swz_b<BK>(nn)) << 3) + ((b & 15) >> 1);
                uint16_t v = 0;
                if (n0 + nn < N && k0 + kk < K) v = B[(size_t)(n0 + nn) * K + k0 + kk];
                *(MIGEMM_LDS uint16_t *)(sb + P) = v;
            }
        }
    };

    // Wait until this wave's loads of a step have landed while at most
    // `ahead` later steps' loads stay in flight.
    auto wait_steps = [&](int ahead) {
        if constexpr (S >= 5) {
            if (ahead >= 2) { wait_vmcnt<2 * LPS>(); return; }
        }
        if constexpr (S >= 4) {
            if (ahead >= 1) { wait_vmcnt<LPS>(); return; }
        }
        wait_vmcnt<0>();
    };

    // Operand fragments of one 32-wide k slice.
    struct Frag { u32x4 a[FM]; u32x4 b[FN]; };
    auto read_frag = [&](int st, int s, Frag &f) {
        const MIGEMM_LDS unsigned char *sa = (const MIGEMM_LDS unsigned char *)(smem + st * STAGE);
        const MIGEMM_LDS unsigned char *sb = sa + A_BYTES;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            // Lane t of a 16-lane group points at row k = kb + t/4, columns
            // m = mb + 4*(t%4) .. +3; the transposing read hands lane i the
            // four k of column mb + i.
            int m = wm * TM + i * 16 + 4 * (ig & 3);
            i16x4 lo, hi;
            {
                int kk = 32 * s + 8 * g + (ig >> 2);
                int byte = kk * (BM * 2) + (((m >> 3) ^ swz_a<BM>(kk)) << 4) + (m & 7) * 2;
                lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIGEMM_LDS i16x4 *)(sa + byte));
            }
            {
                int kk = 32 * s + 8 * g + 4 + (ig >> 2);
                int byte = kk * (BM * 2) + (((m >> 3) ^ swz_a<BM>(kk)) << 4) + (m & 7) * 2;
                hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIGEMM_LDS i16x4 *)(sa + byte));
            }
            typedef __attribute__((ext_vector_type(8))) short i16x8;
            i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            f.a[i] = __builtin_bit_cast(u32x4, v);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            int nn = wn * TN + j * 16 + ig;
            int byte = nn * (BK * 2) + (((4 * s + g) ^ swz_b<BK>(nn)) << 4);
            f.b[j] = *(const MIGEMM_LDS u32x4 *)(sb + byte);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = (K + BK - 1) / BK;
    if (KT > 0) {
#pragma unroll
        for (int p = 0; p < S - 1; ++p)
            if (p < KT) issue(p, p * BK);
        wait_steps(min(S - 2, KT - 1));
        __syncthreads();
        Frag cur;
        read_frag(0, 0, cur);
        int st = 0;
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                Frag nxt;
                bool more = true;
                // The current fragments were read a whole MFMA block ago and
                // have landed; retire them here so that the MFMAs below need
                // no wait while the next fragments' reads are in flight (the
                // LDS counter cannot count past 15 outstanding reads).
                __builtin_amdgcn_s_waitcnt((7 << 4) | 0xc00f);   // lgkmcnt(0)
                if (s + 1 < KS) {
                    read_frag(st, s + 1, nxt);
                } else if (kt + 1 < KT) {
                    // Step kt+1 becomes readable once every wave's loads into
                    // it landed.  After this barrier no wave reads step kt-1's
                    // stage any more: refill it with step kt+S-1.
                    wait_steps(min(S - 3, KT - 2 - kt));
                    __syncthreads();
                    if (kt + S - 1 < KT) issue((st + S - 1) % S, (kt + S - 1) * BK);
                    st = (st + 1 == S) ? 0 : st + 1;
                    read_frag(st, 0, nxt);
                } else {
                    more = false;
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32<DT>(cur.a[i], cur.b[j], acc[i][j]);
                if (more) cur = nxt;
            }
        }
    }

    // Epilogue: lane (g, ig) of block (i, j) holds rows 4g..4g+3 of column ig.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * TM + i * 16 + 4 * g;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * TN + j * 16 + ig;
            if (n >= N) continue;
            uint16_t *dst = C + (size_t)n * M + m;
            if (c_vec && m + 3 < M) {
                u16x4 v = {to_out<DT>(acc[i][j][0]), to_out<DT>(acc[i][j][1]),
                           to_out<DT>(acc[i][j][2]), to_out<DT>(acc[i][j][3])};
                *(u16x4 *)dst = v;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (m + r < M) dst[r] = to_out<DT>(acc[i][j][r]);
            }
        }
    }
}

// ---------------------------------------------------------------------------

template <int DT, int BM, int BN, int BK, int WGM, int WGN, int S, int VA, int VB, int OCC>
static hipError_t launch_t(const GemmLaunch &L, hipStream_t stream)
{
    dim3 grid((unsigned)L.grid), block(WGM * WGN * 64);
    hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, BK, WGM, WGN, S, VA, VB, OCC>), grid, block, 0,
                       stream, L.A, L.B, L.C, L.M, L.N, L.K, L.num_pid_m, L.num_pid_n, L.group_m,
                       L.num_xcd, L.c_vec);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(const GemmLaunch &L, hipStream_t s)
{
    switch (L.tile) {
    case TILE_256x256:
        return launch_t<DT, 256, 256, 32, 2, 2, 4, 8, 8, 1>(L, s);
    case TILE_256x128:
        return launch_t<DT, 256, 128, 64, 2, 2, 3, 8, 8, 1>(L, s);
    case TILE_256x256_S5:
        return launch_t<DT, 256, 256, 32, 2, 2, 5, 8, 8, 1>(L, s);
    case TILE_256x256_S3:
        return launch_t<DT, 256, 256, 32, 2, 2, 3, 8, 8, 1>(L, s);
    case TILE_256x128_K32:
        return launch_t<DT, 256, 128, 32, 2, 2, 5, 8, 8, 1>(L, s);
    case TILE_128x128:
#define MIGEMM_V(va, vb) \
    if (L.vec_a == va && L.vec_b == vb) return launch_t<DT, 128, 128, 32, 2, 2, 4, va, vb, 2>(L, s);
        MIGEMM_V(8, 8) MIGEMM_V(8, 2) MIGEMM_V(8, 1)
        MIGEMM_V(2, 8) MIGEMM_V(2, 2) MIGEMM_V(2, 1)
        MIGEMM_V(1, 8) MIGEMM_V(1, 2) MIGEMM_V(1, 1)
#undef MIGEMM_V
        break;
    }
    return hipErrorInvalidValue;
}

hipError_t gemm_launch(const GemmLaunch &L, hipStream_t stream)
{
    return L.dtype == DT_F16 ? launch_dt<DT_F16>(L, stream) : launch_dt<DT_BF16>(L, stream);
}

}  // namespace migemm
