// gemm.hip -- dense column-major C = A x B on gfx950 MFMA.
//
// Defined by the MTT S4000 GEMM write-up (blog.mthreads.com GEMM03):
// section 1 (16-bit inputs, FP32 accumulation, 16-bit output, column-major),
// section 2 (C(m,n) = sum_k A(m,k) B(k,n), A(m,k) = A[m + k*M],
// B(k,n) = B[k + n*K], C(m,n) = C[m + n*M]).  The kernel design is ours:
//
//  * one workgroup owns a BM x BN tile of C, picked by tile_coord() (XCD
//    renumbering + the grouped ordering of the FlagGems Hygon page);
//  * K advances in 32-wide steps through a ring of S LDS stages (S = 3..5).
//    Each step's A tile (32 k-rows of BM m-contiguous elements) and B tile
//    go straight from HBM into LDS with buffer loads that write LDS directly
//    (no VGPR staging), issued S steps ahead of the step being computed, with
//    explicit vmcnt waits and one barrier per step.  When every load of the
//    launch lies inside A and B (the full-line tiles 9-13, 16 and 17, M and N
//    multiples of the tile, K of 64, 16-byte rows) the same loads go through global
//    addresses instead: they issue faster from L2, and nothing needs the
//    buffer descriptors' range check;
//  * A is m-contiguous, but an MFMA operand needs 8 consecutive k of one row
//    per lane, so A is read out of LDS with the transposing ds_read_b64_tr_b16
//    (lane i of each 16-lane group receives row i of a 16 x 4 block), from a
//    row-XOR-swizzled layout that keeps the four rows of a read in different
//    banks;
//  * B is k-contiguous, so the loads place every 16-column x 32-k operand
//    fragment as one KiB in exactly the order the lanes read it: the B
//    fragment reads are linear ds_read_b128 (the fastest LDS pattern);
//  * operand fragments are double-buffered in registers: the LDS reads of the
//    next step and the loads of step + S are interleaved between the MFMAs of
//    the current step at fixed positions (sched_barrier), all from per-lane
//    base addresses plus immediate offsets;
//  * v_mfma_f32_16x16x32_{f16,bf16} accumulates in FP32 AGPRs, each
//    accumulator tied to a fixed register;
//  * out-of-range rows/columns are never stored; out-of-range k reads as
//    zero through the buffer descriptors' range check, so ragged K needs no
//    separate path;
//  * the epilogue rounds each FP32 sum once to FP16/BF16 (nearest even); no
//    FP32 copy of C ever reaches memory.  In range, the full-line tiles with
//    64-row wave tiles pass the rounded tile through LDS and store whole
//    128-byte lines of C; otherwise each lane stores its 4 rows directly.
#include <type_traits>

#include <algorithm>

#include "common.hpp"
#include "dma.hpp"
#include "tile_map.hpp"
#include "kernels.hpp"

namespace migemm {

// A-stage swizzle: XOR on the 16-byte chunk index within a k row, so that
// the four rows a 16-lane group reads in one transposing LDS read (and the
// rows of the neighbouring group) fall in different banks.
template <int BM>
__device__ inline int swz_a(int kk) { return (((kk & 7) << 1) ^ (kk & 8)) & (BM / 8 - 1); }

// acc += a * b on one 16x16x32 block, accumulating in place in AGPRs.  Written
// as (non-volatile) inline assembly with the accumulator tied to an AGPR
// operand: the compiler keeps each accumulator in one fixed register instead
// of rotating it through copies, and may still schedule these freely.  It
// does not see the MFMA's result latency, so nothing but another MFMA may
// read an accumulator until mfma_drain() has run.
//
// The 16-byte fragments are the same bytes for every element type; only the
// instruction changes.  8-bit types: a fragment is 16 k of INT8 (one
// v_mfma_i32_16x16x64_i8 takes the 16 bytes of every lane, 64 k) or two
// 8-k halves of FP8 (two v_mfma_f32_16x16x32_{fp8,bf8} take bytes 0-7, then
// 8-15).  A and B fragments pair the same bytes of the same lanes, so which
// k a byte holds inside a step does not matter, and the 16x16 result layout
// is the same for all of them.
template <int DT>
__device__ inline void mfma16x16x32(f32x4 &acc, u32x4 a, u32x4 b)
{
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
    if constexpr (DT == DT_F16) {
        asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    } else if constexpr (DT == DT_BF16) {
        asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    } else if constexpr (DT == DT_I8) {
        asm("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    } else {
        const u32x2 alo = {a[0], a[1]}, ahi = {a[2], a[3]}, blo = {b[0], b[1]}, bhi = {b[2], b[3]};
        if constexpr (DT == DT_F8E4M3) {
            asm("v_mfma_f32_16x16x32_fp8_fp8 %0, %1, %2, %0" : "+a"(acc) : "v"(alo), "v"(blo));
            asm("v_mfma_f32_16x16x32_fp8_fp8 %0, %1, %2, %0" : "+a"(acc) : "v"(ahi), "v"(bhi));
        } else {
            asm("v_mfma_f32_16x16x32_bf8_bf8 %0, %1, %2, %0" : "+a"(acc) : "v"(alo), "v"(blo));
            asm("v_mfma_f32_16x16x32_bf8_bf8 %0, %1, %2, %0" : "+a"(acc) : "v"(ahi), "v"(bhi));
        }
    }
}

// Wait states after the last MFMA before its results are read by other
// instructions (more than the longest MFMA write-to-read requirement).
// acc += a * b on one 16x16 block over 128 k of FP8 (E4M3 or E5M2 in both
// operands), the double-rate gfx950 instruction: 32 bytes of A and of B per
// lane.  Like mfma16x16x32, A and B fragments pair the same bytes of the same
// lanes (lane l: row / column l % 16), so which k each byte holds does not
// matter, and the result has the 16x16x32 layout.
typedef __attribute__((ext_vector_type(8))) unsigned u32x8;
template <int DT>
__device__ inline void mfma16x16x128_f8(f32x4 &acc, u32x8 a, u32x8 b)
{
    // the accumulators stay in VGPRs: with them in AGPRs the compiler splits
    // the 256 registers evenly and the two 32-byte fragment sets spill
    static_assert(DT == DT_F8E4M3 || DT == DT_F8E5M2, "FP8 only");
    if constexpr (DT == DT_F8E4M3)
        asm("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
    else
        asm("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 cbsz:1 blgp:1" : "+v"(acc) : "v"(a), "v"(b));
}

__device__ inline void mfma_drain()
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

template <int DT, int BM, int BN, int WGM, int WGN, int S, int VA, int VB, int OCC>
__global__ void __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
gemm_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
            uint16_t *__restrict__ C, int M, int N, int K, int num_pid_m, int num_pid_n,
            int group_m, int num_xcd, int c_vec)
{
    constexpr int BK = 32;                        // K-step = one MFMA k slice
    constexpr int NW = WGM * WGN;
    constexpr int TM = BM / WGM, TN = BN / WGN;   // wave tile
    constexpr int FM = TM / 16, FN = TN / 16;     // 16x16 MFMA blocks per wave
    constexpr int NBJ = BN / 16;                  // B fragments per step
    constexpr int A_BYTES = BK * BM * 2, B_BYTES = BN * BK * 2;
    // LDS: a ring of S stages, each [A tile | B tile].
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int LDS_BYTES = S * STAGE;
    constexpr int A_PIECE = 64 * VA * 2, B_PIECE = 64 * VB * 2;   // bytes per wave load
    constexpr int A_LOADS = A_BYTES / (A_PIECE * NW), B_LOADS = B_BYTES / (B_PIECE * NW);
    constexpr int NLOAD = A_LOADS + B_LOADS;
    // direct-to-LDS loads per wave per K-step (single-element paths are synchronous)
    constexpr int LPS = (VA > 1 ? A_LOADS : 0) + (VB > 1 ? B_LOADS : 0);
    static_assert(A_BYTES % (A_PIECE * NW) == 0 && B_BYTES % (B_PIECE * NW) == 0, "loader split");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "tile shape");
    static_assert(S >= 2 && LDS_BYTES <= 163840, "LDS ring");
    static_assert(LPS * (S - 2) < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

    int pid_m, pid_n;
    tile_coord<int>((int)blockIdx.x, num_pid_m, num_pid_n, group_m, num_xcd, pid_m, pid_n);
    const int m0 = pid_m * BM, n0 = pid_n * BN;
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int wm = wave % WGM, wn = wave / WGM;
    const int g = lane >> 4, ig = lane & 15;

    // ---- where each LDS byte of a stage comes from ----
    // A tile: row kk (k0 + kk), BM elements, 16-byte chunks XOR-swizzled.
    // B tile: fragment jb is one KiB; its lane slot l = 16g' + i' holds
    // B(k0 + 8g' .. +7, n0 + 16jb + i').
    auto a_src = [&](int P, int &kk, int &m) {
        kk = P / (BM * 2);
        int b = P % (BM * 2);
        m = (((b >> 4) ^ swz_a<BM>(kk)) << 3) + ((b & 15) >> 1);
    };
    auto b_src = [&](int P, int &kk, int &nn) {
        int f = P >> 10, l = (P >> 4) & 63, o = P & 15;
        kk = 8 * (l >> 4) + (o >> 1);
        nn = 16 * f + (l & 15);
    };

    uint32_t a_off[A_LOADS];
#pragma unroll
    for (int q = 0; q < (VA > 1 ? A_LOADS : 0); ++q) {
        int kk, m;
        a_src((q * NW + wave) * A_PIECE + lane * VA * 2, kk, m);
        a_off[q] = (uint32_t)(((int64_t)kk * M + m0 + m) * 2);
    }
    uint32_t b_off[B_LOADS];
    int b_k[B_LOADS];
#pragma unroll
    for (int q = 0; q < (VB > 1 ? B_LOADS : 0); ++q) {
        int kk, nn;
        b_src((q * NW + wave) * B_PIECE + lane * VB * 2, kk, nn);
        b_off[q] = (uint32_t)(((int64_t)nn * K + kk) * 2);
        b_k[q] = kk;
    }

    // Loads of the K-step starting at k0 into stage `st`.  Descriptors are
    // rebased per step: A at column k0 with (K - k0) columns of records, so
    // k >= K reads zero; B at column n0, row k0, where rows n >= N fall past
    // the records and k >= K is pushed out of range.  Load q < A_LOADS is
    // A's q-th, the rest are B's; issue_one() issues one of them so that the
    // loads can be spread between MFMAs.
    struct StepDesc { u32x4 da, db; uint32_t sa, sb; int k0; };
    auto step_desc = [&](int st, int k0) {
        StepDesc d;
        d.sa = (uint32_t)(uintptr_t)(MIGEMM_LDS unsigned char *)smem + st * STAGE;
        d.sb = d.sa + A_BYTES;
        d.k0 = k0;
        // a step before k = 0 (the zero step that evens out the step count)
        // gets empty descriptors: all of its loads read zeros
        const bool live = k0 >= 0;
        d.da = make_desc(A + (int64_t)k0 * M, live ? clamp_records((int64_t)(K - k0) * M * 2) : 0u);
        d.db = make_desc(B + (size_t)n0 * K + k0,
                         live ? clamp_records((int64_t)(N - n0) * K * 2 - (int64_t)k0 * 2) : 0u);
        return d;
    };
    auto issue_one = [&](const StepDesc &d, int q) {
        if (q < A_LOADS) {
            if constexpr (VA > 1) {
                dma_to_lds<VA * 2>(d.da, (uint32_t)uniform((int)(d.sa + (q * NW + wave) * A_PIECE)), a_off[q]);
            } else {
                // one element per lane through a register: zero outside the matrix
                int P = (q * NW + wave) * A_PIECE + lane * 2, kk, m;
                a_src(P, kk, m);
                uint16_t v = 0;
                if (m0 + m < M && d.k0 + kk >= 0 && d.k0 + kk < K) v = A[(size_t)(d.k0 + kk) * M + m0 + m];
                *(MIGEMM_LDS uint16_t *)((MIGEMM_LDS unsigned char *)smem + (d.sa - (uint32_t)(uintptr_t)(MIGEMM_LDS unsigned char *)smem) + P) = v;
            }
        } else {
            const int qb = q - A_LOADS;
            if constexpr (VB > 1) {
                uint32_t off = (d.k0 + b_k[qb] < K) ? b_off[qb] : kOutOfRange;
                dma_to_lds<VB * 2>(d.db, (uint32_t)uniform((int)(d.sb + (qb * NW + wave) * B_PIECE)), off);
            } else {
                int P = (qb * NW + wave) * B_PIECE + lane * 2, kk, nn;
                b_src(P, kk, nn);
                uint16_t v = 0;
                if (n0 + nn < N && d.k0 + kk >= 0 && d.k0 + kk < K) v = B[(size_t)(n0 + nn) * K + d.k0 + kk];
                *(MIGEMM_LDS uint16_t *)((MIGEMM_LDS unsigned char *)smem + (d.sb - (uint32_t)(uintptr_t)(MIGEMM_LDS unsigned char *)smem) + P) = v;
            }
        }
    };
    auto issue = [&](int st, int k0) {
        const StepDesc d = step_desc(st, k0);
#pragma unroll
        for (int q = 0; q < NLOAD; ++q) issue_one(d, q);
    };

    // ---- operand fragment reads: per-lane stage-relative addresses ----
    // A: for block i and half h (k rows 0-3 / 4-7 of the lane group's 8), lane
    // t of a 16-lane group points at row 8g + 4h + t/4, columns
    // m = wm*TM + 16i + 4*(t%4) .. +3.  B: linear KiB fragments.
    uint32_t a_rel[FM][2];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int kk = 8 * g + 4 * h + (ig >> 2);
            int m = wm * TM + i * 16 + 4 * (ig & 3);
            a_rel[i][h] = kk * (BM * 2) + ((((m >> 3) ^ swz_a<BM>(kk))) << 4) + (m & 7) * 2;
        }
    const uint32_t b_rel = A_BYTES + lane * 16 + wn * FN * 1024;

    // Operand fragments of one K-step.  read_one(r) issues item r of the NR
    // items that fill it: for r < FM the two transposing reads of A block r,
    // otherwise the linear read of B block r - FM.
    struct Frag { u32x4 a[FM]; u32x4 b[FN]; };
    constexpr int NR = FM + FN;
    auto read_one = [&](uint32_t stage_off, int r, Frag &f) {
        const MIGEMM_LDS unsigned char *base = (const MIGEMM_LDS unsigned char *)smem + stage_off;
        if (r < FM) {
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIGEMM_LDS i16x4 *)(base + a_rel[r][0]));
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIGEMM_LDS i16x4 *)(base + a_rel[r][1]));
            typedef __attribute__((ext_vector_type(8))) short i16x8;
            i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            f.a[r] = __builtin_bit_cast(u32x4, v);
        } else {
            f.b[r - FM] = *(const MIGEMM_LDS u32x4 *)(base + b_rel + (r - FM) * 1024);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K-steps, evened out: with an odd count one zero step (k0 = -BK, whose
    // loads all read zeros) goes first, so the loop below always runs pairs.
    const int KT_ = (((K + BK - 1) / BK) + 1) & ~1;
    const int kbase = ((K + BK - 1) / BK) & 1 ? -BK : 0;

    // The FM*FN MFMAs of one step, with `extra(x)` for x < NX (the next
    // step's fragment reads and later steps' loads) issued between them --
    // one item after every EV MFMAs -- and sched_barrier pinning that order,
    // so no burst of loads or reads holds up the in-order MFMA issue.
    auto mma = [&](const Frag &f, auto nx_c, auto every_c, auto &&extra) {
        constexpr int NXI = decltype(nx_c)::value, EV = decltype(every_c)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                mfma16x16x32<DT>(acc[i][j], f.a[i], f.b[j]);
                const int t = i * FN + j;
                if (t % EV == EV - 1 && t / EV < NXI) extra(t / EV);
                __builtin_amdgcn_sched_barrier(0);
            }
        constexpr int DONE = (FM * FN / EV < NXI ? FM * FN / EV : NXI);
#pragma unroll
        for (int x = DONE; x < NXI; ++x) extra(x);
    };

    // One K-step: compute `cur` (step kt, stage st) while reading step kt+1
    // into `nxt` and refilling stage st with step kt+S.  Before any of that:
    // this wave's reads of stage st have landed (lgkmcnt), step kt+1's loads
    // have landed (vmcnt, letting later steps' loads fly), and after the
    // barrier no wave reads stage st any more.  On the last step the reads
    // fetch stale data that is never used (no load is in flight then).
    auto step = [&](int kt, int st, Frag &cur, Frag &nxt) {
        __builtin_amdgcn_s_waitcnt((7 << 4) | 0xc00f);   // lgkmcnt(0)
        const int ahead = min(S - 2, KT_ - 2 - kt);
        if (kt + 1 < KT_) {
            if constexpr (S >= 5) {
                if (ahead >= 3) wait_vmcnt<3 * LPS>();
                else if (ahead == 2) wait_vmcnt<2 * LPS>();
                else if (ahead == 1) wait_vmcnt<LPS>();
                else wait_vmcnt<0>();
            } else if constexpr (S >= 4) {
                if (ahead >= 2) wait_vmcnt<2 * LPS>();
                else if (ahead == 1) wait_vmcnt<LPS>();
                else wait_vmcnt<0>();
            } else if constexpr (S >= 3) {
                if (ahead >= 1) wait_vmcnt<LPS>();
                else wait_vmcnt<0>();
            } else {
                wait_vmcnt<0>();
            }
            __syncthreads();
        }
        const bool refill = kt + S < KT_;
        const StepDesc d = step_desc(st, (kt + S) * BK + kbase);
        const int nst = (st + 1 == S) ? 0 : st + 1;
        const uint32_t noff = (uint32_t)(nst * STAGE);
        constexpr int NX = NLOAD + NR, NMF = FM * FN;
        mma(cur, std::integral_constant<int, NX>{}, std::integral_constant<int, (NMF / NX > 0 ? NMF / NX : 1)>{},
            [&](int x) {
                // alternate reads and loads so both streams start early
                constexpr int MN = NLOAD < NR ? NLOAD : NR;
                if (x < 2 * MN) {
                    if ((x & 1) == 0) {
                        read_one(noff, x >> 1, nxt);
                    } else {
                        if (refill) issue_one(d, x >> 1);
                    }
                } else {
                    const int t = MN + (x - 2 * MN);
                    if constexpr (NLOAD > NR) {
                        if (refill) issue_one(d, t);
                    } else {
                        read_one(noff, t, nxt);
                    }
                }
            });
        return nst;
    };

    if (KT_ > 0) {
#pragma unroll
        for (int p = 0; p < S; ++p)
            if (p < KT_) issue(p, p * BK + kbase);
        // step 0 landed; steps 1 .. S-1 may fly
        {
            const int ahead = min(S - 1, KT_ - 1);
            if constexpr (S >= 5) {
                if (ahead >= 4) wait_vmcnt<4 * LPS>();
                else if (ahead == 3) wait_vmcnt<3 * LPS>();
                else if (ahead == 2) wait_vmcnt<2 * LPS>();
                else if (ahead == 1) wait_vmcnt<LPS>();
                else wait_vmcnt<0>();
            } else if constexpr (S >= 4) {
                if (ahead >= 3) wait_vmcnt<3 * LPS>();
                else if (ahead == 2) wait_vmcnt<2 * LPS>();
                else if (ahead == 1) wait_vmcnt<LPS>();
                else wait_vmcnt<0>();
            } else {
                if (ahead >= 2) wait_vmcnt<2 * LPS>();
                else if (ahead == 1) wait_vmcnt<LPS>();
                else wait_vmcnt<0>();
            }
        }
        __syncthreads();
        Frag f0, f1;
#pragma unroll
        for (int r = 0; r < NR; ++r) read_one(0, r, f0);
        int st = 0;
        int kt = 0;
        for (; kt < KT_; kt += 2) {
            st = step(kt, st, f0, f1);
            st = step(kt + 1, st, f1, f0);
        }
        wait_vmcnt<0>();   // no load may still target LDS when the workgroup ends
    }

    // Epilogue: lane (g, ig) of block (i, j) holds rows 4g..4g+3 of column ig.
    mfma_drain();
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
// Full-line variant: A as above (a ring of SA stages of 32 k-rows), B through
// its own ring of SB stages that each hold 64 k of every tile column.
//
// Why: an MFMA B operand spans 16 columns x 32 k, i.e. half of each column's
// 128-byte line, so a wave load that fills one operand touches 16 lines half
// each.  A wave load over eight columns x 64 k touches 8 whole lines instead,
// and the fetch path (L1, L2) then moves the same bytes in markedly less
// time.  In the B stage, column c sits at byte c*128 with its eight 16-byte
// k-chunks permuted: chunk x at position x ^ ((c >> 1) & 7).  A wave load
// fills eight consecutive columns (lane l: column 8p + l/8, position l%8),
// so each group of 8 lanes fetches one whole line; an operand read (lane
// (g, i): column 16j + i, chunk 4s + g) then spreads every 16 lanes over all
// LDS banks.
//
// Sub-step j (32 k) reads A stage j % SA and half j & 1 of B stage
// (j / 2) % SB.  Sub-step j issues the A loads of sub-step j + SA, then half
// of the B loads of one B stage: for odd j the first half of pair
// (j-1)/2 + SB, for even j the second half of pair (j-2)/2 + SB (both into
// the stage freed by pair (j-1)/2 resp. (j-2)/2), so every sub-step issues
// the same number of loads.  The prologue issues what the sub-steps before 0
// would have.  fl_loads_after() counts, from that fixed order, how many
// loads may still fly when a sub-step's data is needed.
template <bool AK, int SA, int SB, int LA, int LBH>
constexpr int fl_loads_after(int j, int need_a, int need_b)
{
    int n = 0;
    for (int i = j - 1; i >= -2 * (SA + SB) - 4; --i) {
        // sub-step i issued its A part, then one half of a B stage: undo in
        // reverse.  The A part is sub-step i + SA (m-major A) or one half of
        // A stage base + SA (k-major A), like B.
        const int base = (i & 1) ? (i - 1) / 2 : (i - 2) / 2;
        const int p = base + SB;
        if (p >= 0) {
            if (p == need_b) return n;
            n += LBH;
        }
        const int a = AK ? base + SA : i + SA;
        if (a >= 0) {
            if (a == need_a) return n;
            n += LA;
        }
    }
    return -1;
}

// AK = false: A m-major (A(m,k) = A[m + k*M]), A ring of SA stages of 32 k
// rows read with transposing LDS reads.  AK = true: A k-major (A(m,k) =
// A[k + m*K]), A ring of SA stages of 64 k laid out, loaded and read exactly
// like B (rows of A in place of columns of B).
// Ping-pong tile: MFMAs of a sub-step issued in its load phase (the rest go
// into its compute phase), and the spacing, in compute-phase MFMAs, of the B
// fragment reads there.  PP_PRE applies when the loads go through global
// addresses (every load in range), PP_PRE_BUF with the range-checked buffer
// loads, whose slower issue leaves less room in the load phase.  Measured
// (ms per launch, B read after every 2nd MFMA): in range, 8192^2 x 16384
// FP16, 0 / 2 / 4 / 6 / 8 / 10 / 12 / 16 load-phase MFMAs 1.70 / 1.71 /
// 1.65 / 1.64 / 1.61 / 1.62 / 1.69 / 1.68, and with a read after every MFMA
// 8 / 16 / 24 take 1.62 / 1.72 / 1.85, every 3rd 1.68 (2 or 4 load-phase
// MFMAs) and, in another run, 1.64 / 1.62 (8 / 6) against 1.56; ragged,
// 8000 x 8192 x 16384 FP16, 0 / 2 / 4 / 6 / 8: 1.61 / 1.59 / 1.61 / 1.65 /
// 1.71, and 5000 x 3000 x 4100 BF16 0.115 / 0.113 / 0.114 / 0.118 / 0.120.
#ifndef PP_PRE
#define PP_PRE 8
#endif
#ifndef PP_PRE_BUF
#define PP_PRE_BUF 2
#endif
#ifndef PP_BREAD_EVERY
#define PP_BREAD_EVERY 2
#endif

// Ping-pong schedule (PP below): loads in flight after the last one that
// sub-step t needs, once load phases up to L have issued.  Load phase i
// issues A sub-step i + SA - 1 (LA loads), then half (i & 1) of B stage
// (i >> 1) + SB - 1 (LBH loads).
template <int SA, int SB, int LA, int LBH>
constexpr int pp_loads_after(int L, int t)
{
    const int ia = t - SA + 1;                     // phase that issued A(t)
    const int na = LBH + (L - ia) * (LA + LBH);
    const int ib = 2 * ((t >> 1) - SB + 1) + 1;    // phase that issued B stage t/2's second half
    const int nb = (L - ib) * (LA + LBH);
    return na < nb ? na : nb;
}

// GL: every load lies inside A and B (the caller checked M, N, K and the row
// alignment against the tile), so the loads may use global addresses, which
// issue faster from L2 than the range-checked buffer form.  GL with EDGE (the
// full-line tiles, unsplit): the k loop stays inside K
// and the rows are 16-byte aligned (an m-major A's 8-element pieces never
// straddle M), but the tile may pass M or N; the lanes whose piece or row of
// A lies past M or whose column of B lies past N load row 0 (column 0) of
// the tile at the same k instead, so every address is inside A and B and
// every load is issued (the exact vmcnt counts hold).  Those LDS rows and
// columns only feed outputs past M or N, which are never stored.
template <int DT, bool AK, int BM, int BN, int WGM, int WGN, int SA, int SB, int OCC, bool SPLIT,
          bool PP = false, bool WIDE = false, bool GL = false, bool EDGE = false>
__global__ void __launch_bounds__(WGM * WGN * 64)
__attribute__((amdgpu_waves_per_eu(OCC, OCC)))
gemm_fl_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
               uint16_t *__restrict__ C, int M, int N, int K_total, int num_pid_m, int num_pid_n,
               int group_m, int num_xcd, int c_vec, float scale, int ks, float *__restrict__ part)
{
    // K counts 2-byte units: for 8-bit element types the caller passes half
    // the element count, and each unit holds two elements.
    static_assert(AK || !dt_is_8bit(DT), "8-bit types take a k-major A");
    // SPLIT: workgroup row blockIdx.y sums k in [kb, kb + ks) (ks a multiple
    // of 64) into FP32 partials part[blockIdx.y][n][m]; rows of k-major
    // operands keep their full stride K_total.  Otherwise the k loop covers
    // [0, ks), ks = K_total rounded down to a multiple of 8, so that every
    // 16-byte piece of a k-major row it loads lies inside the row; one more
    // MFMA per block adds the last K_total - ks (< 8) k, and the kernel
    // writes C.
    static_assert(!SPLIT || !dt_is_8bit(DT), "split-K: 16-bit types");
    static_assert(!EDGE || (GL && !SPLIT), "edge-clamped global loads: unsplit launches");
    const int kb = SPLIT ? (int)blockIdx.y * ks : 0;
    const int K = SPLIT ? min(ks, K_total - kb) : ks;
    const int ldk = K_total;
    constexpr int BK = 32;                        // sub-step = one MFMA k slice
    constexpr int NW = WGM * WGN;
    constexpr int TM = BM / WGM, TN = BN / WGN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int A_BYTES = AK ? BM * 128 : BK * BM * 2;   // one A stage
    constexpr int B_BYTES = BN * 128;             // one B stage: 64 k of each column
    constexpr int B_BASE = SA * A_BYTES;
    constexpr int LDS_BYTES = B_BASE + SB * B_BYTES;
    // A loads per wave per sub-step (m-major) or per half stage (k-major)
    constexpr int LA = AK ? A_BYTES / (2048 * NW) : A_BYTES / (1024 * NW);
    constexpr int LB = B_BYTES / (1024 * NW);     // B loads per wave per B stage
    constexpr int LBH = LB / 2;                   // ... per sub-step
    static_assert(A_BYTES % ((AK ? 2048 : 1024) * NW) == 0 && B_BYTES % (2048 * NW) == 0, "loader split");
    static_assert(NW % 2 == 0, "one chunk swizzle per wave for all its B loads");
    static_assert(TM % 16 == 0 && TN % 16 == 0 && BN % 16 == 0, "tile shape");
    static_assert(LDS_BYTES <= 163840, "LDS rings");
    constexpr int W_EVEN = fl_loads_after<AK, SA, SB, LA, LBH>(64, AK ? 32 : 65, 32);
    constexpr int W_ODD = fl_loads_after<AK, SA, SB, LA, LBH>(65, AK ? 33 : 66, 33);
    constexpr int W_PRO = fl_loads_after<AK, SA, SB, LA, LBH>(0, 0, 0);
    static_assert(W_EVEN >= 0 && W_EVEN < 64 && W_ODD >= 0 && W_ODD < 64 && W_PRO >= 0 && W_PRO < 64,
                  "vmcnt range");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[LDS_BYTES];

    int pid_m, pid_n;
    tile_coord<int>((int)blockIdx.x, num_pid_m, num_pid_n, group_m, num_xcd, pid_m, pid_n);
    const int m0 = pid_m * BM, n0 = pid_n * BN;
    // Measurement only (part is free when the k loop is not split): with
    // part non-null, wave 0 of each workgroup records the shader-clock and
    // 100 MHz real-time counts it ran for, as two 64-bit words per workgroup.
    const bool clocked = !SPLIT && part != nullptr;
    uint64_t clk_t0 = 0, clk_r0 = 0;
    if (clocked) {
        clk_t0 = __builtin_amdgcn_s_memtime();
        clk_r0 = __builtin_amdgcn_s_memrealtime();
    }
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int wm = wave % WGM, wn = wave / WGM;
    const int g = lane >> 4, ig = lane & 15;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(MIGEMM_LDS unsigned char *)smem;

    // k-major loads (B, and A when AK): lane l of load q fills row/column
    // c = 8p + l/8 of the tile at chunk position l%8, i.e. k chunk
    // x = (l%8) ^ ((c >> 1) & 7) of the stage's 64 k
    auto kmajor_lane = [&](int q, int stride, uint32_t &off, int &kk) {
        const int c = 8 * (q * NW + wave) + (lane >> 3);
        const int x = (lane & 7) ^ ((c >> 1) & 7);
        off = (uint32_t)(((int64_t)c * stride + 8 * x) * 2);
        kk = 8 * x;
    };
    constexpr int NAO = AK ? 2 * LA : LA;
    uint32_t a_off[NAO];
    int a_k[AK ? NAO : 1];
#pragma unroll
    for (int q = 0; q < NAO; ++q) {
        if constexpr (AK) {
            kmajor_lane(q, ldk, a_off[q], a_k[q]);
            if constexpr (EDGE)   // row 8(q NW + wave) + l/8 past M: row 0, same k piece
                if (m0 + 8 * (q * NW + wave) + (lane >> 3) >= M) a_off[q] = (uint32_t)(a_k[q] * 2);
        } else {
            // m-major A: piece P = (q*NW + wave) KiB of the stage, row kk,
            // swizzled 16-byte chunks
            const int P = (q * NW + wave) * 1024 + lane * 16;
            const int kk = P / (BM * 2), b = P % (BM * 2);
            const int m = (((b >> 4) ^ swz_a<BM>(kk)) << 3);
            a_off[q] = (uint32_t)(((int64_t)kk * M + m0 + m) * 2);
            if constexpr (EDGE)
                if (m0 + m >= M) a_off[q] = (uint32_t)((int64_t)kk * M * 2);   // row 0 of the tile
        }
    }
    // every B load of a wave has the same chunk swizzle (it depends on the
    // column group's parity only, and NW is even): one base offset and k,
    // load q adding q*NW column groups
    uint32_t b_off0;
    int b_k0;
    kmajor_lane(0, ldk, b_off0, b_k0);
    auto b_offq = [&](int q) { return b_off0 + (uint32_t)(8 * q * NW) * (uint32_t)uniform(ldk * 2); };

    // Sub-steps, evened out: with an odd count a zero sub-step (k0 = -BK,
    // every element read as zero) goes first.  P_ = number of 64-k stages.
    const int J = (((K + BK - 1) / BK) + 1) & ~1;
    const int P_ = J / 2;
    const int kbase = ((K + BK - 1) / BK) & 1 ? -BK : 0;

    // Descriptors.  m-major A: rebased at sub-step jj's first k row (k >= K
    // reads zero; the leading zero sub-step gets no records).  k-major
    // operands: rebased at X + r0*K + k0 elements for the stage starting at
    // k0 (k0 may be -BK: the lanes below k = 0 are sent out of range, so
    // nothing below X is read), with rows/columns >= R past the records.
    auto desc_kmajor = [&](const uint16_t *X, int r0, int R, int pp) {
        const int k0 = kb + kbase + pp * 2 * BK;
        const uint64_t base = (uint64_t)(uintptr_t)X + ((int64_t)r0 * ldk + k0) * 2;
        return make_desc((const void *)(uintptr_t)base,
                         clamp_records((int64_t)(R - r0) * ldk * 2 - (int64_t)k0 * 2));
    };
    auto desc_a = [&](int jj) {
        if constexpr (AK) {
            return desc_kmajor(A, m0, M, jj);
        } else {
            const int k0 = kbase + jj * BK;
            return make_desc(A + (int64_t)(kb + k0) * M,
                             k0 >= 0 ? clamp_records((int64_t)(K - k0) * M * 2) : 0u);
        }
    };
    auto desc_b = [&](int pp) { return desc_kmajor(B, n0, N, pp); };
    auto kmajor_off = [&](int pp, int kk, uint32_t off) {
        const int k = kbase + pp * 2 * BK + kk;
        return (k >= 0 && k < K) ? off : kOutOfRange;
    };
    // issue_a: m-major: load q of sub-step jj into A stage sa; k-major: load
    // q (of 2*LA) of A stage jj into stage sa
    // (GL: the same bytes from the same offsets, relative to the pointer the
    // descriptor would have been built on; every k then lies in [0, K))
    auto issue_a = [&](const u32x4 &d, int jj, int sa, int q) {
        const uint32_t lds = (uint32_t)uniform((int)(lds0 + sa * A_BYTES + (q * NW + wave) * 1024));
        if constexpr (GL) {
            const uint16_t *base = AK ? A + ((int64_t)m0 * ldk + kb + kbase + jj * 2 * BK)
                                      : A + (int64_t)(kb + kbase + jj * BK) * M;
            gdma16_to_lds((const void *)base, a_off[q], lds);
        } else {
            uint32_t off = a_off[q];
            if constexpr (AK) off = kmajor_off(jj, a_k[q], off);
            dma_to_lds<16>(d, lds, off);
        }
    };
    auto issue_b = [&](const u32x4 &d, int pp, int sb, int q) {
        const uint32_t lds = (uint32_t)uniform((int)(lds0 + B_BASE + sb * B_BYTES + (q * NW + wave) * 1024));
        if constexpr (GL) {
            uint32_t off = b_offq(q);
            if constexpr (EDGE)   // column 8(q NW + wave) + l/8 past N: column 0, same k piece
                if (n0 + 8 * (q * NW + wave) + (lane >> 3) >= N) off = (uint32_t)(b_k0 * 2);
            gdma16_to_lds((const void *)(B + ((int64_t)n0 * ldk + kb + kbase + pp * 2 * BK)), off, lds);
        }
        else
            dma_to_lds<16>(d, lds, kmajor_off(pp, b_k0, b_offq(q)));
    };

    // operand reads (stage-relative): m-major A through transposing reads;
    // k-major operands per half s of the stage
    uint32_t a_rel[AK ? 2 : FM][2];
    if constexpr (AK) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
            a_rel[s][0] = (wm * TM + ig) * 128 + 16 * ((4 * s + g) ^ ((ig >> 1) & 7));
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                int kk = 8 * g + 4 * h + (ig >> 2);
                int m = wm * TM + i * 16 + 4 * (ig & 3);
                a_rel[i][h] = kk * (BM * 2) + ((((m >> 3) ^ swz_a<BM>(kk))) << 4) + (m & 7) * 2;
            }
    }
    uint32_t b_rel[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        b_rel[s] = B_BASE + (wn * TN + ig) * 128 + 16 * ((4 * s + g) ^ ((ig >> 1) & 7));

    struct Frag { u32x4 a[FM]; u32x4 b[FN]; };
    constexpr int NR = FM + FN;
    // item r of the NR reads that fill a fragment set: A block r or B block
    // r - FM, from A stage sa and B stage sb (half s of the 64-k stages)
    auto read_one = [&](int sa, int sb, int s, int r, Frag &f) {
        const MIGEMM_LDS unsigned char *base = (const MIGEMM_LDS unsigned char *)smem;
        if (r < FM) {
            const MIGEMM_LDS unsigned char *ab = base + sa * A_BYTES;
            if constexpr (AK) {
                f.a[r] = *(const MIGEMM_LDS u32x4 *)(ab + a_rel[s][0] + r * 2048);
            } else {
                i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIGEMM_LDS i16x4 *)(ab + a_rel[r][0]));
                i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIGEMM_LDS i16x4 *)(ab + a_rel[r][1]));
                typedef __attribute__((ext_vector_type(8))) short i16x8;
                i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                f.a[r] = __builtin_bit_cast(u32x4, v);
            }
        } else {
            f.b[r - FM] = *(const MIGEMM_LDS u32x4 *)(base + sb * B_BYTES + b_rel[s] + (r - FM) * 2048);
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if constexpr (!SPLIT && !dt_is_8bit(DT)) {
        if (K < K_total) {
            // k in [K, K_total) (fewer than 8), before the loop: one MFMA
            // per block on those k.  The workgroup stages them (zero past M,
            // N and K_total) as 8 elements per A row and per B column in LDS
            // (the rings' first bytes, refilled only after the second
            // barrier); lanes 0-15 of each operand take their row's or
            // column's 8, lanes 16-63 zero.
            uint16_t *t16 = (uint16_t *)smem;
            static_assert((BM + BN) * 16 <= LDS_BYTES, "k-tail staging");
            for (int e = threadIdx.x; e < (BM + BN) * 8; e += NW * 64) {
                const int k = K + (e & 7);
                uint16_t v = 0;
                if (e < BM * 8) {
                    const int m = m0 + (e >> 3);
                    if (m < M && k < K_total) v = A[AK ? (size_t)m * ldk + k : (size_t)k * M + m];
                } else {
                    const int n = n0 + (e >> 3) - BM;
                    if (n < N && k < K_total) v = B[(size_t)n * ldk + k];
                }
                t16[e] = v;
            }
            __syncthreads();
            Frag tf;
            const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < FM; ++i)
                tf.a[i] = g == 0 ? *(const u32x4 *)&t16[(wm * TM + i * 16 + ig) * 8] : z;
#pragma unroll
            for (int j = 0; j < FN; ++j)
                tf.b[j] = g == 0 ? *(const u32x4 *)&t16[(BM + wn * TN + j * 16 + ig) * 8] : z;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) mfma16x16x32<DT>(acc[i][j], tf.a[i], tf.b[j]);
            __syncthreads();
        }
    }

    auto mma = [&](const Frag &f, auto nx_c, auto every_c, auto &&extra) {
        constexpr int NXI = decltype(nx_c)::value, EV = decltype(every_c)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                mfma16x16x32<DT>(acc[i][j], f.a[i], f.b[j]);
                const int t = i * FN + j;
                if (t % EV == EV - 1 && t / EV < NXI) extra(t / EV);
                __builtin_amdgcn_sched_barrier(0);
            }
        constexpr int DONE = (FM * FN / EV < NXI ? FM * FN / EV : NXI);
#pragma unroll
        for (int x = DONE; x < NXI; ++x) extra(x);
    };

    // Sub-step j (parity PAR) on fragments `cur`.  Ring positions: sa / sb
    // the stages of sub-step j, sap / sbp the 64-k stages before them.
    // Reads sub-step j+1 into `nxt`, refills A (m-major: stage sa with
    // sub-step j+SA; k-major: half of a freed stage, like B) and half of a
    // freed B stage.  Before that, this wave's reads have landed (lgkmcnt),
    // sub-step j+1's loads have landed (vmcnt: exact count while every load
    // of the fixed order was issued, else all), and after the barrier no
    // wave reads the stages being refilled.
    auto step = [&](int j, auto par_c, int &sa, int &sap, int &sb, int &sbp, Frag &cur, Frag &nxt) {
        constexpr int PAR = decltype(par_c)::value;
        __builtin_amdgcn_s_waitcnt((7 << 4) | 0xc00f);   // lgkmcnt(0)
        const int base_prev = PAR ? (j - 3) / 2 : (j - 2) / 2;   // stage base issued in sub-step j-1
        const int base_cur = PAR ? (j - 1) / 2 : (j - 2) / 2;    // ... in sub-step j
        if (j + 1 < J) {
            const bool a_all = AK ? (base_prev + SA < P_) : (j - 1 + SA < J);
            const bool exact = a_all && (base_prev + SB < P_);
            if (exact) wait_vmcnt<PAR ? W_ODD : W_EVEN>();
            else wait_vmcnt<0>();
            __syncthreads();
        }
        const int ja = AK ? base_cur + SA : j + SA;     // A unit refilled
        const bool ra = AK ? ja < P_ : ja < J;
        const int sar = AK ? (PAR ? sa : sap) : sa;
        const int pr = base_cur + SB;                  // B stage refilled
        const bool rb = pr < P_;
        const int sbr = PAR ? sb : sbp;
        const u32x4 da = desc_a(ja), db = desc_b(pr);
        const int nsa = AK ? (PAR ? ((sa + 1 == SA) ? 0 : sa + 1) : sa) : ((sa + 1 == SA) ? 0 : sa + 1);
        const int nsb = PAR ? ((sb + 1 == SB) ? 0 : sb + 1) : sb;
        constexpr int NL = LA + LBH;
        constexpr int NX = NL + NR, NMF = FM * FN;
        mma(cur, std::integral_constant<int, NX>{}, std::integral_constant<int, (NMF / NX > 0 ? NMF / NX : 1)>{},
            [&](int x) {
                constexpr int MN = NL < NR ? NL : NR;
                auto load = [&](int q) {
                    if (q < LA) {
                        if (ra) issue_a(da, ja, sar, (AK && !PAR ? LA : 0) + q);
                    } else {
                        if (rb) issue_b(db, pr, sbr, (PAR ? 0 : LBH) + q - LA);
                    }
                };
                // With two waves per SIMD (8 waves) the loads go first, so
                // that a load stalled at issue holds up this wave's MFMAs
                // while the other wave's run; with one wave per SIMD reads
                // and loads alternate.  Measured, same box (ms): 8192^2 x
                // 16384 BF16 on tile 10, k-major A 1.545 against 1.626
                // alternating, m-major 1.531 against 1.566, INT8 0.777
                // against 0.792; tile 13 at 2048^2 x 16384 0.1605 against
                // 0.1577 alternating, tile 9 the same either way.
                if constexpr (NW == 8) {
                    if (x < NL) load(x);
                    else read_one(nsa, nsb, 1 - PAR, x - NL, nxt);
                } else if (x < 2 * MN) {
                    if ((x & 1) == 0) read_one(nsa, nsb, 1 - PAR, x >> 1, nxt);
                    else load(x >> 1);
                } else {
                    const int t = MN + (x - 2 * MN);
                    if constexpr (NL > NR) load(t);
                    else read_one(nsa, nsb, 1 - PAR, t, nxt);
                }
            });
        if (PAR) {
            sbp = sb;
            if constexpr (AK) sap = sa;
        }
        sa = nsa;
        sb = nsb;
    };

    if constexpr (WIDE) {
        // FP8 on the double-rate MFMA (tile 17): every step covers a whole
        // 64-unit stage (128 FP8 k); a lane's fragment of a block is the two
        // 16-byte chunks it reads from the stage's halves, 32 bytes, one
        // v_mfma_f32_16x16x128 per block and step.  Fragments double-buffered
        // (stage p + 1 is read while stage p's MFMAs run), S stages in each
        // ring, step p loading stage p + S into the slot stage p left (read
        // into registers during step p - 1), so a stage's loads have S - 1
        // steps to land.
        static_assert(AK && (DT == DT_F8E4M3 || DT == DT_F8E5M2) && SA == SB && !SPLIT && !PP,
                      "wide steps: FP8, k-major A, equal rings");
        constexpr int S = SA;
        constexpr int NLS = 2 * LA + LB;                 // loads per wave per stage
        static_assert(NLS * (S - 1) < 64, "vmcnt range");
        struct FragW { u32x8 a[FM]; u32x8 b[FN]; };
        auto read_w = [&](int slot, int r, FragW &f) {
            const MIGEMM_LDS unsigned char *base = (const MIGEMM_LDS unsigned char *)smem;
            u32x4 lo, hi;
            if (r < FM) {
                const MIGEMM_LDS unsigned char *ab = base + slot * A_BYTES + r * 2048;
                lo = *(const MIGEMM_LDS u32x4 *)(ab + a_rel[0][0]);
                hi = *(const MIGEMM_LDS u32x4 *)(ab + a_rel[1][0]);
                f.a[r] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                const MIGEMM_LDS unsigned char *bb = base + slot * B_BYTES + (r - FM) * 2048;
                lo = *(const MIGEMM_LDS u32x4 *)(bb + b_rel[0]);
                hi = *(const MIGEMM_LDS u32x4 *)(bb + b_rel[1]);
                f.b[r - FM] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        };
        if (P_ > 0) {
            // load item x < NLS of stage p: A loads first, then B
            auto stage_load = [&](int p, int x, const u32x4 &da, const u32x4 &db) {
                if (p < P_) {
                    if (x < 2 * LA) issue_a(da, p, p % S, x);
                    else issue_b(db, p, p % S, x - 2 * LA);
                }
            };
#pragma unroll
            for (int p = 0; p < S; ++p) {
                const u32x4 da = desc_a(p), db = desc_b(p);
#pragma unroll
                for (int x = 0; x < NLS; ++x) stage_load(p, x, da, db);
            }
            if (S <= P_) wait_vmcnt<(S - 1) * NLS>();   // stage 0 landed
            else wait_vmcnt<0>();
            __syncthreads();
            FragW f0, f1;
#pragma unroll
            for (int r = 0; r < NR; ++r) read_w(0, r, f0);
            // step p: stage p + 1 landed (it was issued two steps ago; only
            // stage p + 2's loads came after it), everyone has read stage p;
            // then the MFMAs of stage p with the loads of stage p + S and
            // then the reads of stage p + 1 between them
            auto wstep = [&](int p, FragW &cur, FragW &nxt) {
                __builtin_amdgcn_s_waitcnt((7 << 4) | 0xc00f);   // lgkmcnt(0)
                if (p + 2 < P_) wait_vmcnt<NLS>();
                else wait_vmcnt<0>();
                __syncthreads();
                const int pl = p + S;
                const u32x4 da = desc_a(pl), db = desc_b(pl);
                const int ns = (p + 1) % S;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int jj = 0; jj < FN; ++jj) {
                        mfma16x16x128_f8<DT>(acc[i][jj], cur.a[i], cur.b[jj]);
                        const int t = i * FN + jj;
                        // loads first (FP8 8192^2 x 16384, same box: E4M3
                        // 0.906-0.915 ms against 0.928-0.936 reads first,
                        // E5M2 0.889-0.892 against 0.910-0.913)
                        if (t < NLS) stage_load(pl, t, da, db);
                        else if (t - NLS < NR) read_w(ns, t - NLS, nxt);
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                for (int x = (FM * FN > NLS ? FM * FN - NLS : 0); x < NR; ++x) read_w(ns, x, nxt);
            };
            for (int p = 0; p < P_; p += 2) {
                wstep(p, f0, f1);
                if (p + 1 < P_) wstep(p + 1, f1, f0);
            }
            wait_vmcnt<0>();   // no load may still target LDS when the workgroup ends
        }
    } else if constexpr (PP) {
        // Ping-pong: two groups of four waves, one wave of each group per
        // SIMD (waves w and w + 4 share a SIMD).  Each sub-step j is a load
        // phase (issue the LDS-direct loads of a later sub-step, then the
        // transposing reads of sub-step j's own A fragments, then its first
        // PRE MFMAs) and a compute phase (the other MFMAs of sub-step j, with
        // the B fragment reads of sub-step j + 1 into the other fragment set
        // between them).  Group 1 runs one phase behind group 0, a workgroup
        // barrier between phases, so on each SIMD one wave streams MFMAs
        // while the other waits for the memory pipe to take its loads: a load
        // stalled at issue never holds up an MFMA.  A wave's LDS reads are
        // split over its two phases because one wave's reads are served at
        // a limited rate (about one KiB per 31 cycles with linear reads, 512
        // bytes per 41 with transposing ones, measured), which with all of
        // them in the compute phase made that phase the longest.
        //
        // Load phase i issues A sub-step i + SA - 1 and half (i & 1) of B
        // stage (i >> 1) + SB - 1: the largest distances at which no load
        // targets a stage still to be read.  Before the barrier that ends its
        // compute phase j, a wave waits for its own loads of sub-step j + 2,
        // which the group one phase ahead starts reading right after it.
        static_assert(!AK && !SPLIT && NW == 8, "ping-pong: 8 waves, m-major A");
        const int role = wave >> 2;
        if (J > 0) {
            auto phase_loads = [&](int i) {
                const int ja = i + SA - 1;
                if (ja >= 0 && ja < J) {
                    const u32x4 d = desc_a(ja);
#pragma unroll
                    for (int q = 0; q < LA; ++q) issue_a(d, ja, ja % SA, q);
                }
                const int pb = (i >> 1) + SB - 1;
                if (pb >= 0 && pb < P_) {
                    const u32x4 d = desc_b(pb);
#pragma unroll
                    for (int q = 0; q < LBH; ++q) issue_b(d, pb, pb % SB, (i & 1) * LBH + q);
                }
            };
            // wait until sub-step t's loads have landed, load phases up to L
            // issued; the exact count holds while phase L issued every load of
            // the fixed order (then so did all phases before it)
            auto wait_for = [&](auto lpar_c, auto dt_c, int L) {
                constexpr int LP = decltype(lpar_c)::value, DT_ = decltype(dt_c)::value;
                constexpr int W = pp_loads_after<SA, SB, LA, LBH>(64 + LP, 64 + LP + DT_);
                static_assert(W >= 0 && W < 64, "vmcnt range");
                if (L + SA - 1 < J && (L >> 1) + SB - 1 < P_) wait_vmcnt<W>();
                else wait_vmcnt<0>();
            };
            constexpr int FIRST = -(SA - 1) < -2 * (SB - 1) ? -(SA - 1) : -2 * (SB - 1);
#pragma unroll
            for (int i = FIRST; i < 0; ++i) phase_loads(i);
            Frag f0, f1;
            wait_for(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}, -1);   // sub-step 0
            __syncthreads();
#pragma unroll
            for (int r = FM; r < NR; ++r) read_one(0, 0, 0, r, f0);   // its B fragments
            if (J > 1) wait_for(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{}, -1);   // sub-step 1
            __syncthreads();
            if (role) __syncthreads();
            // Load phase of sub-step j: its loads; then the A fragments of
            // sub-step j (stage j of the A ring, complete since the barrier
            // that ended the phase before, and refilled only two phases
            // after this one), into the set whose B fragments the compute
            // phase before read; then the first PRE MFMAs of sub-step j, so
            // that for part of every phase both waves of a SIMD issue MFMAs.
            constexpr int NMF = FM * FN;
            constexpr int PRE_ = GL ? PP_PRE : PP_PRE_BUF;
            constexpr int PRE = PRE_ < NMF ? PRE_ : 0;
            auto load_phase = [&](int j, Frag &cur) {
                phase_loads(j);
#pragma unroll
                for (int r = 0; r < FM; ++r) read_one(j % SA, 0, 0, r, cur);
#pragma unroll
                for (int t = 0; t < PRE; ++t) {
                    mfma16x16x32<DT>(acc[t / FN][t % FN], cur.a[t / FN], cur.b[t % FN]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            // compute phase of sub-step j on `cur` (its MFMAs from PRE on),
            // reading sub-step j + 1's B fragments into `nxt` (one read after
            // every EV MFMAs, early enough that the last has landed when the
            // phase ends; after the last sub-step these read stale ring
            // contents that are never used)
            auto compute = [&](int j, auto par_c, Frag &cur, Frag &nxt) {
                constexpr int PAR = decltype(par_c)::value;
                constexpr int EV = PP_BREAD_EVERY;
                static_assert(EV >= 1 && FN * EV <= NMF - PRE, "B reads fit the compute phase");
                const int nb = ((j + 1) >> 1) % SB;
#pragma unroll
                for (int t = PRE; t < NMF; ++t) {
                    mfma16x16x32<DT>(acc[t / FN][t % FN], cur.a[t / FN], cur.b[t % FN]);
                    const int u = t - PRE;
                    if (u % EV == EV - 1 && u / EV < FN) read_one(0, nb, 1 - PAR, FM + u / EV, nxt);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (j + 2 < J) wait_for(std::integral_constant<int, PAR>{}, std::integral_constant<int, 2>{}, j);
                __syncthreads();
            };
            for (int j = 0; j < J; j += 2) {
                load_phase(j, f0);
                __syncthreads();
                compute(j, std::integral_constant<int, 0>{}, f0, f1);
                if (j + 1 < J) {
                    load_phase(j + 1, f1);
                    __syncthreads();
                    compute(j + 1, std::integral_constant<int, 1>{}, f1, f0);
                }
            }
            if (!role) __syncthreads();
            wait_vmcnt<0>();   // no load may still target LDS when the workgroup ends
        }
    } else if (J > 0) {
        // prologue: the loads of the sub-steps before 0, in the fixed order
#pragma unroll
        for (int i = -2 * (SA + SB) - 4; i < 0; ++i) {
            const int base = (i & 1) ? (i - 1) / 2 : (i - 2) / 2;
            const int a = AK ? base + SA : i + SA;
            if (a >= 0 && a < (AK ? P_ : J)) {
                const u32x4 d = desc_a(a);
#pragma unroll
                for (int q = 0; q < LA; ++q) issue_a(d, a, a, (AK && !(i & 1) ? LA : 0) + q);
            }
            const int p = base + SB;
            if (p >= 0 && p < P_) {
                const u32x4 d = desc_b(p);
#pragma unroll
                for (int q = 0; q < LBH; ++q) issue_b(d, p, p, ((i & 1) ? 0 : LBH) + q);
            }
        }
        if ((AK ? SA - 1 < P_ : SA - 1 < J) && SB - 1 < P_) wait_vmcnt<W_PRO>();
        else wait_vmcnt<0>();
        __syncthreads();
        Frag f0, f1;
#pragma unroll
        for (int r = 0; r < NR; ++r) read_one(0, 0, 0, r, f0);
        int sa = 0, sap = SA - 1, sb = 0, sbp = SB - 1;
        for (int j = 0; j < J; j += 2) {
            step(j, std::integral_constant<int, 0>{}, sa, sap, sb, sbp, f0, f1);
            step(j + 1, std::integral_constant<int, 1>{}, sa, sap, sb, sbp, f1, f0);
        }
        wait_vmcnt<0>();   // no load may still target LDS when the workgroup ends
    }
    mfma_drain();
    if constexpr (SPLIT) {
        // FP32 partial sums of this k slice (16-bit types only)
        float *pz = part + (size_t)blockIdx.y * M * N;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * TM + i * 16 + 4 * g;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * TN + j * 16 + ig;
                if (n >= N) continue;
                float *dst = pz + (size_t)n * M + m;
                if (c_vec && m + 3 < M) {
                    *(f32x4 *)dst = acc[i][j];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (m + r < M) dst[r] = acc[i][j][r];
                }
            }
        }
        return;
    }
    // With 64-row wave tiles, C on a 16-byte boundary and M a multiple of 8:
    // each wave converts its tile into its own LDS window (the rings are free
    // once every wave has passed the barrier below: all operand reads done,
    // no load in flight), one 128-byte column of 64 outputs every CS bytes,
    // and writes C back in whole lines: lane l stores 16 bytes, rows
    // 8(l%8).. of column l/8 of an 8-column group.  With M a multiple of 8
    // each such piece lies wholly inside or wholly outside C, so a ragged
    // edge only drops pieces.  The direct stores below write each line in
    // four 32-byte pieces.
    constexpr int CS = TM * 2 + 16;
    constexpr bool STAGE_C = TM == 64 && NW * TN * CS <= LDS_BYTES;
    if (STAGE_C && uniform((int)(((uintptr_t)C & 15) == 0 && (M & 7) == 0))) {
        __syncthreads();
        // lane indices taken afresh (an opaque copy of the thread id), so
        // that none is computed before the k loop and held through it
        int t = (int)threadIdx.x;
        asm volatile("" : "+v"(t));
        const int eg = (t >> 4) & 3, eig = t & 15, el = t & 63;
        MIGEMM_LDS unsigned char *win = (MIGEMM_LDS unsigned char *)smem + wave * (TN * CS);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const u16x4 v = {out16<DT>(acc[i][j][0], scale), out16<DT>(acc[i][j][1], scale),
                                 out16<DT>(acc[i][j][2], scale), out16<DT>(acc[i][j][3], scale)};
                *(MIGEMM_LDS u16x4 *)(win + (j * 16 + eig) * CS + (i * 16 + 4 * eg) * 2) = v;
                __builtin_amdgcn_sched_barrier(0);   // convert and write block by block
            }
        }
        const int gm = m0 + wm * TM + (el & 7) * 8, gn = n0 + wn * TN;
        uint16_t *cw = C + (size_t)gn * M + gm;
#pragma unroll
        for (int s = 0; s < TN / 8; ++s) {
            const int c = s * 8 + (el >> 3);
            const u32x4 v = *(MIGEMM_LDS const u32x4 *)(win + c * CS + (el & 7) * 16);
            if ((GL && !EDGE) || (gm < M && gn + c < N)) *(u32x4 *)(cw + (size_t)c * M) = v;
        }
    } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * TM + i * 16 + 4 * g;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * TN + j * 16 + ig;
            if (n >= N) continue;
            uint16_t *dst = C + (size_t)n * M + m;
            if (c_vec && m + 3 < M) {
                u16x4 v = {out16<DT>(acc[i][j][0], scale), out16<DT>(acc[i][j][1], scale),
                           out16<DT>(acc[i][j][2], scale), out16<DT>(acc[i][j][3], scale)};
                *(u16x4 *)dst = v;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (m + r < M) dst[r] = out16<DT>(acc[i][j][r], scale);
            }
        }
    }
    }
    if (clocked && threadIdx.x == 0) {
        const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
        uint64_t *rec = (uint64_t *)part + 2 * ((size_t)blockIdx.y * gridDim.x + blockIdx.x);
        rec[0] = t1 - clk_t0;
        rec[1] = r1 - clk_r0;
    }
}

// OCC: waves per SIMD the kernel is compiled for (its register budget is
// 512 / OCC per lane); 0 = one workgroup's waves spread one per SIMD.
// Split-K variants exist for the tiles 9 (256x128), 10 (256x256, 8 waves)
// and 13 (128x128) and the 16-bit types.
template <int DT, int BM, int BN, int WGM, int WGN>
constexpr bool kSplitTile = !dt_is_8bit(DT) && ((BM == 256 && BN == 128 && WGM * WGN == 4) ||
                                                (BM == 256 && BN == 256 && WGM * WGN == 8) ||
                                                (BM == 128 && BN == 128 && WGM * WGN == 4));

template <int DT, bool AK, int BM, int BN, int WGM, int WGN, int SA, int SB, int OCC = 0, bool PP = false,
          bool WIDE = false, bool GLOK = false>
static hipError_t launch_fl(const GemmLaunch &L, hipStream_t stream)
{
    constexpr int OC = OCC ? OCC : WGM * WGN / 4;
    const dim3 block(WGM * WGN * 64);
    if (L.splits > 1) {
        if constexpr (kSplitTile<DT, BM, BN, WGM, WGN> && !PP && !WIDE && GLOK) {
            if (L.in_range) {
                hipLaunchKernelGGL((gemm_fl_kernel<DT, AK, BM, BN, WGM, WGN, SA, SB, OC, true, false, false, true>),
                                   dim3((unsigned)L.grid, (unsigned)L.splits), block, 0, stream, L.A, L.B,
                                   L.C, L.M, L.N, L.K, L.num_pid_m, L.num_pid_n, L.group_m, L.num_xcd,
                                   L.c_vec, L.scale, L.ks, L.part);
                return hipGetLastError();
            }
        }
        if constexpr (kSplitTile<DT, BM, BN, WGM, WGN> && !PP && !WIDE) {
            hipLaunchKernelGGL((gemm_fl_kernel<DT, AK, BM, BN, WGM, WGN, SA, SB, OC, true>),
                               dim3((unsigned)L.grid, (unsigned)L.splits), block, 0, stream, L.A, L.B,
                               L.C, L.M, L.N, L.K, L.num_pid_m, L.num_pid_n, L.group_m, L.num_xcd,
                               L.c_vec, L.scale, L.ks, L.part);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if constexpr (GLOK) {
        if (L.in_range) {
            hipLaunchKernelGGL((gemm_fl_kernel<DT, AK, BM, BN, WGM, WGN, SA, SB, OC, false, PP, WIDE, true>),
                               dim3((unsigned)L.grid), block, 0, stream, L.A, L.B, L.C, L.M, L.N, L.K,
                               L.num_pid_m, L.num_pid_n, L.group_m, L.num_xcd, L.c_vec, L.scale, L.K & ~7,
                               (float *)L.clocks);
            return hipGetLastError();
        }
        {
            if (L.edge_gl) {
                hipLaunchKernelGGL((gemm_fl_kernel<DT, AK, BM, BN, WGM, WGN, SA, SB, OC, false, PP, WIDE, true, true>),
                                   dim3((unsigned)L.grid), block, 0, stream, L.A, L.B, L.C, L.M, L.N, L.K,
                                   L.num_pid_m, L.num_pid_n, L.group_m, L.num_xcd, L.c_vec, L.scale, L.K & ~7,
                                   (float *)L.clocks);
                return hipGetLastError();
            }
        }
    }
    hipLaunchKernelGGL((gemm_fl_kernel<DT, AK, BM, BN, WGM, WGN, SA, SB, OC, false, PP, WIDE>),
                       dim3((unsigned)L.grid), block, 0, stream, L.A, L.B, L.C, L.M, L.N, L.K,
                       L.num_pid_m, L.num_pid_n, L.group_m, L.num_xcd, L.c_vec, L.scale, L.K & ~7,
                       (float *)L.clocks);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------

template <int DT, int BM, int BN, int WGM, int WGN, int S, int VA, int VB, int OCC>
static hipError_t launch_t(const GemmLaunch &L, hipStream_t stream)
{
    dim3 grid((unsigned)L.grid), block(WGM * WGN * 64);
    hipLaunchKernelGGL((gemm_kernel<DT, BM, BN, WGM, WGN, S, VA, VB, OCC>), grid, block, 0,
                       stream, L.A, L.B, L.C, L.M, L.N, L.K, L.num_pid_m, L.num_pid_n, L.group_m,
                       L.num_xcd, L.c_vec);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(const GemmLaunch &L, hipStream_t s)
{
    switch (L.tile) {
    case TILE_256x256:
        return launch_t<DT, 256, 256, 2, 2, 4, 8, 8, 1>(L, s);
    case TILE_256x128:
        return launch_t<DT, 256, 128, 2, 2, 5, 8, 8, 1>(L, s);
    case TILE_256x256_S5:
        return launch_t<DT, 256, 256, 2, 2, 5, 8, 8, 1>(L, s);
    case TILE_256x256_W41:
        return launch_t<DT, 256, 256, 4, 1, 4, 8, 8, 1>(L, s);
    case TILE_256x256_S3:
        return launch_t<DT, 256, 256, 2, 2, 3, 8, 8, 1>(L, s);
    case TILE_256x256_FL:
        return L.a_kmajor ? launch_fl<DT, true, 256, 256, 4, 1, 2, 3>(L, s)
                          : launch_fl<DT, false, 256, 256, 4, 1, 4, 3>(L, s);
    case TILE_256x256_FL22:
        return L.a_kmajor ? launch_fl<DT, true, 256, 256, 2, 2, 2, 3>(L, s)
                          : launch_fl<DT, false, 256, 256, 2, 2, 4, 3>(L, s);
    case TILE_256x128_FL:
        return L.a_kmajor ? launch_fl<DT, true, 256, 128, 4, 1, 3, 4, 0, false, false, true>(L, s)
                          : launch_fl<DT, false, 256, 128, 4, 1, 4, 4, 0, false, false, true>(L, s);
    case TILE_256x256_FL8:
        return L.a_kmajor ? launch_fl<DT, true, 256, 256, 4, 2, 2, 3, 0, false, false, true>(L, s)
                          : launch_fl<DT, false, 256, 256, 4, 2, 4, 3, 0, false, false, true>(L, s);
    case TILE_256x256_PP:
        return L.a_kmajor ? hipErrorInvalidValue
                          : launch_fl<DT, false, 256, 256, 4, 2, 4, 3, 2, true, false, true>(L, s);
    case TILE_64x32_SK:
        return L.a_kmajor ? launch_fl<DT, true, 64, 32, 2, 1, 4, 2, 2, false, false, true>(L, s)
                          : launch_fl<DT, false, 64, 32, 2, 1, 4, 2, 2, false, false, true>(L, s);
    case TILE_64x64_SK:
        return L.a_kmajor ? launch_fl<DT, true, 64, 64, 2, 1, 4, 2, 2, false, false, true>(L, s)
                          : launch_fl<DT, false, 64, 64, 2, 1, 4, 2, 2, false, false, true>(L, s);
    case TILE_128x128_SK:
        return L.a_kmajor ? launch_fl<DT, true, 128, 128, 2, 2, 4, 3, 1, false, false, true>(L, s)
                          : launch_fl<DT, false, 128, 128, 2, 2, 4, 3, 1, false, false, true>(L, s);
    case TILE_128x128:
#define MIGEMM_V(va, vb) \
    if (L.vec_a == va && L.vec_b == vb) return launch_t<DT, 128, 128, 2, 2, 4, va, vb, 2>(L, s);
        MIGEMM_V(8, 8) MIGEMM_V(8, 2) MIGEMM_V(8, 1)
        MIGEMM_V(2, 8) MIGEMM_V(2, 2) MIGEMM_V(2, 1)
        MIGEMM_V(1, 8) MIGEMM_V(1, 2) MIGEMM_V(1, 1)
#undef MIGEMM_V
        break;
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Split-K: C = round(sum_z part[z]) over `splits` FP32 partial matrices of
// `count` elements each, one rounding.  VEC: 4 consecutive elements per
// thread (count % 4 == 0, part 16-byte and C 8-byte aligned).

template <int DT, bool VEC>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float *__restrict__ part, uint16_t *__restrict__ C, int64_t count, int splits)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * (VEC ? 4 : 1);
    for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * (VEC ? 4 : 1); i < count; i += stride) {
        if constexpr (VEC) {
            f32x4 acc = *(const f32x4 *)(part + i);
            for (int z = 1; z < splits; ++z) {
                const f32x4 v = *(const f32x4 *)(part + (size_t)z * count + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += v[e];
            }
            const u16x4 o = {to_out<DT>(acc[0]), to_out<DT>(acc[1]), to_out<DT>(acc[2]), to_out<DT>(acc[3])};
            *(u16x4 *)(C + i) = o;
        } else {
            float acc = part[i];
            for (int z = 1; z < splits; ++z) acc += part[(size_t)z * count + i];
            C[i] = to_out<DT>(acc);
        }
    }
}

hipError_t splitk_reduce_launch(int dtype, const float *part, uint16_t *C, int64_t count, int splits,
                                hipStream_t stream)
{
    if (count <= 0) return hipSuccess;
    const bool vec = count % 4 == 0 && (uintptr_t)part % 16 == 0 && (uintptr_t)C % 8 == 0;
    const int64_t items = vec ? count / 4 : count;
    const unsigned grid = (unsigned)std::min<int64_t>((items + 255) / 256, 8192);
    if (dtype == DT_F16) {
        if (vec) hipLaunchKernelGGL((splitk_reduce_kernel<DT_F16, true>), dim3(grid), dim3(256), 0, stream, part, C, count, splits);
        else hipLaunchKernelGGL((splitk_reduce_kernel<DT_F16, false>), dim3(grid), dim3(256), 0, stream, part, C, count, splits);
    } else {
        if (vec) hipLaunchKernelGGL((splitk_reduce_kernel<DT_BF16, true>), dim3(grid), dim3(256), 0, stream, part, C, count, splits);
        else hipLaunchKernelGGL((splitk_reduce_kernel<DT_BF16, false>), dim3(grid), dim3(256), 0, stream, part, C, count, splits);
    }
    return hipGetLastError();
}

// 8-bit inputs: the k-major full-line tiles 9 (256x128), 10 (256x256, 8
// waves) and 13 (128x128); L.K is in 2-byte units.
template <int DT>
static hipError_t launch_q(const GemmLaunch &L, hipStream_t s)
{
    if (!L.a_kmajor) return hipErrorInvalidValue;
    switch (L.tile) {
    case TILE_256x128_FL: return launch_fl<DT, true, 256, 128, 4, 1, 3, 4, 0, false, false, true>(L, s);
    case TILE_256x256_FL8: return launch_fl<DT, true, 256, 256, 4, 2, 2, 3, 0, false, false, true>(L, s);
    case TILE_128x128_SK: return launch_fl<DT, true, 128, 128, 2, 2, 4, 3, 1, false, false, true>(L, s);
    case TILE_256x128_F8W:
        if constexpr (DT == DT_F8E4M3 || DT == DT_F8E5M2)
            return launch_fl<DT, true, 256, 128, 4, 2, 3, 3, 2, false, true, true>(L, s);
        break;
    }
    return hipErrorInvalidValue;
}

hipError_t gemm_launch(const GemmLaunch &L, hipStream_t stream)
{
    switch (L.dtype) {
    case DT_F16: return launch_dt<DT_F16>(L, stream);
    case DT_BF16: return launch_dt<DT_BF16>(L, stream);
    case DT_F8E4M3: return launch_q<DT_F8E4M3>(L, stream);
    case DT_F8E5M2: return launch_q<DT_F8E5M2>(L, stream);
    case DT_I8: return launch_q<DT_I8>(L, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace migemm
