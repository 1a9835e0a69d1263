/*
 * migemm.h -- C ABI of the MI355X (gfx950) dense GEMM and decode GEMV.
 *
 * Element types.  Every matrix element is a raw 16-bit pattern (uint16_t):
 * IEEE binary16 for the *_f16 calls, bfloat16 for the *_bf16 calls.  The
 * library reinterprets the bits; it never converts the caller's data.
 *
 * Arithmetic (MTT S4000 GEMM write-up, blog.mthreads.com GEMM03, section 1,
 * rules table): 16-bit inputs, FP32 accumulation, 16-bit output rounded to
 * nearest-even.  The k-summation order is unspecified (any FP32 order).
 *
 * Pointers are DEVICE pointers (hipMalloc / torch CUDA tensors) unless noted.
 * The caller owns every buffer.  The library allocates no device memory,
 * creates no streams and keeps no mutable state, so calls on different
 * streams may run concurrently.
 *
 * stream: a hipStream_t passed as void*.  NULL means the null stream AND that
 * the call waits for its work to finish before returning (the "complete before
 * return" rule of the write-up's rules table).  A non-NULL stream makes the call
 * stream-ordered: it returns after enqueueing.
 *
 * Return codes: 0 on success; a negative MIGEMM_ERR_* code for argument
 * errors, detected on the host BEFORE any HIP call (nothing is launched or
 * written); a positive hipError_t if a launch or the synchronisation fails.
 * No exceptions cross the ABI and nothing is printed.
 */
#ifndef MIGEMM_H
#define MIGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIGEMM_OK            0
#define MIGEMM_ERR_DIM      (-1)  /* a dimension is negative                     */
#define MIGEMM_ERR_NULL     (-2)  /* NULL pointer where the extent is non-zero   */
#define MIGEMM_ERR_OVERLAP  (-3)  /* the output overlaps an input's byte range   */
#define MIGEMM_ERR_ALIGN    (-4)  /* a pointer or size is not aligned as needed  */
#define MIGEMM_ERR_CONFIG   (-5)  /* an explicit configuration is not offered    */
#define MIGEMM_ERR_SIZE     (-6)  /* a dimension exceeds the supported range     */

/* Largest supported dimensions (element offsets inside one tile must fit the
 * 31-bit range of a buffer descriptor): M and N up to 2^23, K up to 2^21. */
#define MIGEMM_MAX_MN  (1 << 23)
#define MIGEMM_MAX_K   (1 << 21)

/*
 * gemm_f16 / gemm_bf16 -- C = A x B, column-major.
 *
 * Defined by the write-up's section 2 (GEMM basics): the triple loop
 * C(m,n) = sum_k A(m,k) * B(k,n) and the column-major addressing
 *     A(m,k) = A[m + k*M]   (M x K, m fastest)
 *     B(k,n) = B[k + n*K]   (K x N, k fastest)
 *     C(m,n) = C[m + n*M]   (M x N, m fastest)
 * with the argument order (A, B, C, M, N, K) of the write-up's host entry
 * point (section 3.1); `stream` is appended.
 *
 * A and B are read only, never written.  C is written only at its M*N
 * elements.  Any shape is accepted: M == 0 or N == 0 returns 0 without a
 * launch; K == 0 writes +0.0 to every element of C (the empty sum).
 * Errors: MIGEMM_ERR_DIM, _NULL, _ALIGN, _OVERLAP (C's bytes intersect A's
 * or B's), _SIZE; see above.
 */
int gemm_f16(const uint16_t *A, const uint16_t *B, uint16_t *C,
             int M, int N, int K, void *stream);
int gemm_bf16(const uint16_t *A, const uint16_t *B, uint16_t *C,
              int M, int N, int K, void *stream);

/*
 * gemv_bf16 -- decode GEMV Y = X W^T (bfloat16).
 *
 * Defined by the DCU decode page (forum.sourcefind.cn db785961), section 6.1:
 * the linear layer Y = X W^T with X:[n,k] (tokens x input features),
 * W:[m,k] (output x input features) and Y:[n,m], all row-major here:
 *     Y[i*M + j] = sum_k X[i*K + k] * W[j*K + k],   i < n, j < M.
 * Section 6.2: every Y[i*M + j] is an independent full-K dot product; the
 * kernel splits W's output rows across workgroups.  No bias.
 *
 * W and X are read only.  n == 0 or M == 0 returns 0 without a launch;
 * K == 0 writes +0.0 to Y.  Errors as for the GEMM (Y must not overlap W, X).
 * n may be any positive value.  One token (or K not a multiple of 8, or W,
 * X not 16-byte aligned) runs the row-blocked vector kernel.  With 16-byte
 * rows, 65 .. 256 tokens with M > 30720 run on the wide row-balanced
 * 16x16x32 MFMA kernel (tile 19 below: W's rows cut evenly over the CUs,
 * each workgroup's rows reused from registers across its tokens); 2 .. 128
 * tokens otherwise on the row-balanced kernel (tile 18) when M >= 16384,
 * or from 33 tokens on for any M; otherwise 2 tokens take the vector
 * kernel, 3 or 4 the 4x4x4 MFMA with W streamed straight into operand
 * registers, up to 64 the 16x16x32 MFMA with W read as whole cache lines and
 * the token block of X staged in LDS (tile 15 below), and beyond that
 * gemm_tn_bf16 on the 256x128 full-line tile while M and K are within the
 * GEMM's limits (MIGEMM_MAX_MN, MIGEMM_MAX_K; larger problems take the
 * vector kernel).  gemv_bf16_ex with a non-zero rows_per_block always runs
 * the vector kernel.  migemm_gemv_plan_for reports the choice.
 */
int gemv_bf16(const uint16_t *W, const uint16_t *X, uint16_t *Y,
              int M, int K, int n, void *stream);

/*
 * attention_decode_bf16 -- decode attention over a paged KV cache (bfloat16).
 *
 * Defined by the DCU decode page (forum.sourcefind.cn db785961): section 6.1
 * gives, per query head, scores = q K^T over the L cached tokens, prob =
 * softmax(scores), out = prob V, and the paged cache layout [block,
 * token_in_block, kv_head, head_dim]; section 6.3 splits the L tokens into
 * contiguous segments, each with a local max, local softmax denominator and
 * local prob V, merged with a numerically stable global reduction (section 7
 * measures 16 vs 32 segments).  Here, one query token per sequence:
 *     out[b][h][:] = softmax(scale * Q[b][h] . K[l], l < seq_lens[b]) V[l]
 * with K[l], V[l] the rows of kv head h / (Hq / Hkv) for token l, found in
 * page block_table[b * max_blocks + l / block_size] at slot l % block_size.
 * FP32 arithmetic, one rounding to bfloat16.
 *   Q, Out:      [B][Hq][D] row-major; Q, Kc, Vc 16-byte aligned.
 *   Kc, Vc:      [num_blocks][block_size][Hkv][D] (device).
 *   block_table: [B][max_blocks] int32 page ids (device); seq_lens: [B]
 *                int32 (device), clamped to max_blocks * block_size.
 *                Tokens on a page id outside [0, num_blocks) are skipped.
 *   D in {64, 128, 256}; Hq / Hkv in {1, 2, 4, 8}.
 *   max_seq_len: host-side upper bound of seq_lens (for the automatic
 *                segment count); num_segments: 0 = automatic
 *                (migemm_attention_segments), else 1 .. 1024.
 *   workspace:   device, 16-byte aligned, at least
 *                migemm_attention_workspace_bytes(B, Hq, D, segments) bytes
 *                (the per-segment FP32 partials); owned by the caller.
 * A sequence with seq_lens[b] == 0 gets zeros.  Errors: MIGEMM_ERR_DIM,
 * _NULL, _ALIGN, _CONFIG (D, group size, segments), _SIZE (workspace too
 * small; B or Hkv above 65535; max_blocks * block_size above 2^30),
 * _OVERLAP (Out or workspace intersecting an input).  B == 0 is a
 * no-op.  Completion as for the GEMM (NULL stream: synchronous).
 */
int attention_decode_bf16(const uint16_t *Q, const uint16_t *Kc, const uint16_t *Vc,
                          const int32_t *block_table, const int32_t *seq_lens,
                          uint16_t *Out, int B, int Hq, int Hkv, int D, int block_size,
                          int max_blocks, int num_blocks, float scale, int max_seq_len,
                          int num_segments, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * attention_decode_bf16_noalloc -- attention_decode_bf16 for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The same arguments
 * without the workspace: the segment partials go to a device array the
 * library holds on each GPU it runs on, MIGEMM_NOALLOC_SCRATCH_BYTES (8 MiB)
 * each, until the process ends.  Returns MIGEMM_ERR_SIZE when
 * migemm_attention_workspace_bytes(B, Hq, D, segments) exceeds it (checked
 * on the host before any HIP call).  Allocates nothing: the array's address
 * is looked up once per device, on the first call with that device current.
 * All calls on one GPU share the array, so calls that run at the same time
 * on one GPU (other streams, other host threads) race: the caller orders
 * them.  Results equal attention_decode_bf16's for the same segment count.
 */
#define MIGEMM_NOALLOC_SCRATCH_BYTES (8 << 20)
int attention_decode_bf16_noalloc(const uint16_t *Q, const uint16_t *Kc, const uint16_t *Vc,
                                  const int32_t *block_table, const int32_t *seq_lens,
                                  uint16_t *Out, int B, int Hq, int Hkv, int D, int block_size,
                                  int max_blocks, int num_blocks, float scale, int max_seq_len,
                                  int num_segments, void *stream);

/* Segments the automatic choice uses (host only): the largest power of two
 * that keeps the segment workgroups (B * Hkv * ceil(Hq / Hkv / 4) per
 * segment) within one round of residency on 256 CUs (512) and at least
 * 128 tokens per segment; 1 when the lengths are short. */
int migemm_attention_segments(int B, int Hq, int Hkv, int max_seq_len);
/* Workspace bytes attention_decode_bf16 needs for that many segments. */
size_t migemm_attention_workspace_bytes(int B, int Hq, int D, int num_segments);

/*
 * 8-bit GEMMs in the k-major ("TN") layout: C(m,n) = C[m + n*M] =
 *     BF16_RNE( scale * sum_k A(m,k) * B(k,n) ),   A(m,k) = At[k + m*K],
 *                                                  B(k,n) = B[k + n*K],
 * i.e. A row-major M x K and B given as its N columns of K contiguous
 * elements (with At = W [M, K] and B = X [N, K] it is Y = X W^T of the DCU
 * decode page, section 6.1, on 8-bit data).  The element types are the
 * 8-bit ones gfx950's matrix cores take for this GEMM (FP8 E4M3 / E5M2 and
 * INT8; OCP FP8 encodings, both operands in the same format): products and
 * sums in FP32 (FP8) or exact INT32 (INT8), then one FP32 multiply by
 * `scale` (the dequantisation factor, e.g. the product of per-tensor
 * scales; for INT8 the INT32 sum is converted to FP32 first), one RNE
 * rounding to bfloat16.  K must be a multiple of 16 and At, B 16-byte
 * aligned (else MIGEMM_ERR_ALIGN); C 2-byte aligned; other checks,
 * ownership and completion as for gemm_f16.  INT8 sums are exact for
 * K * 127 * 128 < 2^31.
 */
int gemm_tn_fp8_e4m3(const uint8_t *At, const uint8_t *B, uint16_t *C,
                     int M, int N, int K, float scale, void *stream);
int gemm_tn_fp8_e5m2(const uint8_t *At, const uint8_t *B, uint16_t *C,
                     int M, int N, int K, float scale, void *stream);
int gemm_tn_i8(const int8_t *At, const int8_t *B, uint16_t *C,
               int M, int N, int K, float scale, void *stream);

/*
 * Split-K GEMM: the product of gemm_ex (a_kmajor 0: A(m,k) = A[m + k*M]) or
 * gemm_tn_ex (a_kmajor 1: A(m,k) = A[k + m*K]), with B(k,n) = B[k + n*K]
 * and C(m,n) = C[m + n*M], for shapes whose output tiles do not fill the
 * 256 CUs: K is cut into `splits` slices (of a multiple of 64 k), each slice
 * summed in FP32 into its own M x N partial in `workspace`, then one kernel
 * adds the partials and rounds once (RNE) to the 16-bit format.  splits 0 =
 * automatic (migemm_splitk_splits); 1 = no split (same as gemm_ex /
 * gemm_tn_ex).  Slices run on the full-line tiles 9, 10 and 13 (tile 0
 * with a split: the automatic rule's tile, below); another explicit tile
 * with splits > 1 is
 * MIGEMM_ERR_CONFIG, and operands without 16-byte rows run unsplit.
 * workspace: device, 16-byte aligned, at least
 * migemm_splitk_workspace_bytes(M, N, slices) bytes where slices =
 * ceil(K / ks), ks = 64 * ceil(ceil(K / splits) / 64) (never more than
 * `splits`), owned by the caller, not overlapping A, B or C; unused (may be
 * NULL) without a split.  Errors as for gemm_ex, plus _NULL / _ALIGN /
 * _SIZE / _OVERLAP for the workspace.  dtype 0 (binary16) or 1 (bfloat16).
 */
int gemm_splitk_ex(int dtype, int a_kmajor, const uint16_t *A, const uint16_t *B,
                   uint16_t *C, int M, int N, int K, int splits, int tile,
                   int group_m, int xcd_remap, void *workspace,
                   size_t workspace_bytes, void *stream);
/* The automatic slice count (host only): the smallest power of two that
 * gives the 256x256 tile (10) >= 256 workgroups, else the 256x128 tile (9)
 * likewise (the automatic tile of gemm_splitk_ex follows), slices of >= 1024
 * k, at most 32; 1 for shapes whose 256x256 tiles fill the chip and for the
 * k-major decode widths (N <= 64), which stream A once anyway. */
int migemm_splitk_splits(int dtype, int a_kmajor, int M, int N, int K);
/* FP32 partial bytes for that many slices (0 when slices <= 1). */
size_t migemm_splitk_workspace_bytes(int M, int N, int splits);

/* ---- explicit-configuration variants (tuning sweeps) --------------------- */

/*
 * Same contract as gemm_f16 / gemm_bf16 with the tile configuration named by
 * the caller instead of chosen by the library:
 *   tile:    0 = automatic (with group_m 0: first an exact-shape table of
 *            measured configurations -- the headline FP16 GEMM, the prefill
 *            GEMM in both layouts, the ragged BF16 GEMM -- then tile 20 when
 *            its 32x32 tiles number at most 768 (512 when A and B have
 *            16-byte rows and K is a multiple of 64) and B has 16-byte rows,
 *            then,
 *            below 128 tiles of 128x128, tile 11 when A and B have 16-byte
 *            rows and K is a multiple of 64 up to 2048 (otherwise tile 12 or
 *            11 for K <= 8192), else the least estimated time over rounds of
 *            workgroups on the 256 CUs among tiles 16, 9 or 2, and 13 or 3,
 *            the full-line 9 and 13 priced lower when A and B have 16-byte
 *            rows and K is a multiple of 64, since they then load through
 *            global addresses); 1 = 256x256 (4 waves as 2x2, 4 LDS stages);
 *            2 = 256x128 (5 stages); 3 = 128x128 (4 stages, two workgroups
 *            per CU); 4 = tile 1 with 5 stages; 5 = 256x256 with the 4 waves
 *            stacked along M; 6 = tile 1 with 3 stages; 7 = 256x256, waves
 *            along M, B loaded as whole 128-byte column lines (64 k) into
 *            its own 3-stage ring, A in a 4-stage ring; 8 = tile 7 with the
 *            waves as 2x2; 9 = 256x128 like tile 7 with a 4-stage B ring;
 *            10 = tile 7 with 8 waves (4 x 2, two per SIMD); skinny tiles for
 *            few columns (decode batches): 11 = 64x32 and 12 = 64x64 (2 waves,
 *            several workgroups per CU), 13 = 128x128 (4 waves as 2x2), all
 *            with tile 7's full-line B ring; 14 = the skinny 4x4x4 MFMA kernel
 *            of gemv_bf16 (gemm_tn_* only, N <= 8); 15 = the batch kernel
 *            of gemv_bf16 (gemm_tn_* only, N <= 128: 64 rows x 16..128
 *            columns per workgroup, 16x16x32 MFMA, A read as whole lines and
 *            re-laid out through LDS, B staged in LDS); 16 = tile 10's
 *            shape, rings and layouts with the ping-pong schedule (the two
 *            waves of each SIMD alternate a load phase and an MFMA phase;
 *            gemm_ex only, not split-K); 17 = the FP8 double-rate tile
 *            (gemm_tn_q_ex only); 18 = the row-balanced batch kernel
 *            (gemm_tn_* only, N <= 256: W's rows spread evenly over the
 *            workgroups, about M / 256 each rounded up to a multiple of 8 and
 *            at most 144, 9 waves of 16 rows, 16..256 columns, K in steps of
 *            64, A read as whole lines through LDS, B staged in LDS); 19 =
 *            the wide row-balanced kernel (gemm_tn_* only, N <= 256: the
 *            same rows per workgroup, 8 waves in two row groups of 7 and 2
 *            row tiles of 16 times four column groups, 128- or 256-column
 *            blocks, K in steps of 64, A and B both staged in LDS by direct
 *            loads); 20 = small problems: a 32x32 tile per workgroup whose 4
 *            waves (8 for at most 256 tiles with K >= 1024) split K,
 *            operands read straight into MFMA registers, the
 *            partial tiles summed in LDS (both layouts; B, and a k-major A,
 *            with 16-byte rows, else MIGEMM_ERR_ALIGN; an m-major A of any M;
 *            at most 65535 32-column blocks, else MIGEMM_ERR_SIZE; not for
 *            8-bit types or split-K).
 *            All step K by 32.  Tiles 1, 2, 4, 5, 6 need 16-byte rows (M and
 *            K multiples of 8, A and B 16-byte aligned); the full-line tiles
 *            7 .. 13 and 16 need 4-byte rows (M and K even, A and B 4-byte
 *            aligned): their k loop stops at K rounded down to a multiple of
 *            8 and one more MFMA step adds the remaining k; tile 3 takes
 *            any alignment (else MIGEMM_ERR_CONFIG);
 *   group_m: width of the grouped tile ordering (FlagGems "Hygon 优化" page,
 *            section "分组调度"), >= 1, or 0 for automatic;
 *   xcd_remap: 1 to place consecutive tiles of the ordering on one XCD's L2,
 *            0 to use the hardware's round-robin dispatch order unchanged.
 * dtype: 0 = binary16, 1 = bfloat16.  MIGEMM_ERR_CONFIG for values out of range.
 */
int gemm_ex(int dtype, const uint16_t *A, const uint16_t *B, uint16_t *C,
            int M, int N, int K, int tile, int group_m, int xcd_remap,
            void *stream);

/*
 * GEMM with A supplied k-major ("TN"): C(m,n) = C[m + n*M] =
 * RNE( sum_k At[k + m*K] * B[k + n*K] ), FP32 accumulation, i.e. C = A x B
 * with A(m,k) = At[k + m*K] (A row-major, M x K).  Called with At = W
 * (row-major [M, K]), B = X (row-major [N, K]) and C = Y it computes the
 * DCU decode page's Y = X W^T (section 6.1) for a batch of N token rows,
 * with Y row-major [N, M] -- the GEMV's own layout.  Same argument checks,
 * ownership and completion rules as gemm_f16 / gemm_bf16.  Runs on the
 * full-line and decode tiles only: tile 0 (automatic, with 16-byte rows:
 * 19 for 65 <= N <= 256 when M > 30720, else 18 for 2 <= N <= 128 when
 * M >= 16384 or N >= 33, else 14 for N <= 4, 15 for N <= 64; beyond that,
 * or with 4-byte rows, the least estimated time among 10, 9 and 13) or
 * 7 .. 15, 18 and 19 (A takes B's 64-k ring layout; MIGEMM_ERR_CONFIG for
 * other tiles, 16 and 17 included, and for 14 with N > 8, 15 with N > 128
 * or 18 and 19 with N > 256).  K even and At, B 4-byte aligned (4-byte
 * rows) for tiles 7 .. 13, K a multiple of 8 and At, B 16-byte aligned for
 * 14, 15, 18 and 19 (which tile 0 then uses); else MIGEMM_ERR_ALIGN.
 */
int gemm_tn_f16(const uint16_t *At, const uint16_t *B, uint16_t *C,
                int M, int N, int K, void *stream);
int gemm_tn_bf16(const uint16_t *At, const uint16_t *B, uint16_t *C,
                 int M, int N, int K, void *stream);
int gemm_tn_ex(int dtype, const uint16_t *At, const uint16_t *B, uint16_t *C,
               int M, int N, int K, int tile, int group_m, int xcd_remap,
               void *stream);

/* The 8-bit GEMMs with an explicit configuration: qtype 2 = FP8 E4M3,
 * 3 = FP8 E5M2, 4 = INT8 (the dtype codes of migemm_gemm_tn_plan_for);
 * tile 0 (automatic: for FP8, 17 when its 256x128 tiles fill the chip;
 * otherwise 10 when the 256x256 tiles fill the chip twice, 9 when 256x128
 * tiles fill it once, else 13), 9, 10, 13, or 17 for FP8 only (256x128, 8
 * waves, the double-rate v_mfma_f32_16x16x128 FP8 instruction on whole
 * 64-byte k steps; MIGEMM_ERR_CONFIG for INT8); group_m and xcd_remap
 * as for gemm_ex.  gemm_tn_ex rejects these dtypes (it has no scale). */
int gemm_tn_q_ex(int qtype, const void *At, const void *B, uint16_t *C,
                 int M, int N, int K, float scale, int tile, int group_m,
                 int xcd_remap, void *stream);

/*
 * Same contract as gemv_bf16 with rows_per_block (output rows of W per
 * workgroup of the vector kernel: 2, 4, 8, 16 or 32), the knob swept on the
 * DCU decode page, section 6.2; 0 = automatic (as gemv_bf16).
 */
int gemv_bf16_ex(const uint16_t *W, const uint16_t *X, uint16_t *Y,
                 int M, int K, int n, int rows_per_block, void *stream);

/* ---- host-only helpers (no GPU work; callable without a GPU) ------------ */

/*
 * The tile scheduler used by the GEMM kernel, evaluated on the host: maps
 * workgroup id `wg` of a grid of num_pid_m x num_pid_n tiles to its tile
 * (*pid_m, *pid_n).  num_xcd > 1 first renumbers ids so that the ids the
 * hardware sends to one XCD form a contiguous range, then applies the grouped
 * ordering with width group_m.  Returns 0, or MIGEMM_ERR_DIM for bad input.
 */
int migemm_tile_coord(int64_t wg, int64_t num_pid_m, int64_t num_pid_n,
                      int64_t group_m, int64_t num_xcd,
                      int64_t *pid_m, int64_t *pid_n);

/* What the library would launch for a GEMM call (for tests and reports). */
typedef struct {
    int tile_m, tile_n, tile_k;   /* workgroup tile (tile_k = K per step)  */
    int waves;                    /* waves per workgroup                  */
    int group_m;                  /* grouped-ordering width               */
    int xcd_remap;                /* 1 if the XCD renumbering is applied  */
    int vec_a, vec_b;             /* elements per global->LDS load of A, B */
    int64_t grid;                 /* workgroups launched                  */
    int lds_bytes;                /* LDS per workgroup                    */
    int tile;                     /* tile configuration id (as gemm_ex's) */
    int a_kmajor;                 /* 1 for gemm_tn_ex's k-major A         */
} migemm_gemm_plan;

/* Fill *plan for gemm_ex's arguments (pointers are inspected for alignment
 * only, never dereferenced).  Returns the code gemm_ex would return for the
 * argument checks (0 if a launch would happen). */
int migemm_gemm_plan_for(int dtype, const uint16_t *A, const uint16_t *B,
                         const uint16_t *C, int M, int N, int K, int tile,
                         int group_m, int xcd_remap, migemm_gemm_plan *plan);
/* The same for gemm_tn_ex, and with dtype 2, 3, 4 for gemm_tn_q_ex (K in
 * elements; tile_k reported in elements). */
int migemm_gemm_tn_plan_for(int dtype, const uint16_t *At, const uint16_t *B,
                            const uint16_t *C, int M, int N, int K, int tile,
                            int group_m, int xcd_remap, migemm_gemm_plan *plan);

/* Which kernel gemv_bf16_ex would run for these arguments (pointers are
 * inspected for alignment only, never dereferenced): writes to *route 0 (no
 * launch: M or n is 0), 1 (the row-blocked vector kernel), 14 (the 4x4x4
 * MFMA kernel), 15 (the batch kernel), 18 (the row-balanced batch kernel),
 * 19 (the wide row-balanced kernel) or 9 (gemm_tn on the 256x128
 * full-line tile; only while M <= MIGEMM_MAX_MN and K <= MIGEMM_MAX_K,
 * larger problems stay on the vector kernel), and returns the code
 * gemv_bf16_ex would return for the argument checks. */
int migemm_gemv_plan_for(const uint16_t *W, const uint16_t *X, const uint16_t *Y,
                         int M, int K, int n, int rows_per_block, int *route);

/* Human-readable text for a return code (static storage). */
const char *migemm_strerror(int code);

/* Library ABI version (bumped when a signature changes). */
int migemm_abi_version(void);

/* ---- measurement --------------------------------------------------------- */

/*
 * Streaming-read bandwidth probe: reads `bytes` bytes from device buffer
 * `buf` once (768 one-wave workgroups, 3 per CU; each wave reads contiguous
 * 8 KiB chunks with eight 16-byte non-temporal loads per lane in flight,
 * the grid size that read fastest when swept) and writes one 32-bit XOR
 * checksum per wave to `sink` (device, migemm_hbm_read_sink_words() words;
 * the XOR of all of them is the XOR of the buffer's 32-bit words).
 * `bytes` must be a multiple of 16 and `buf` 16-byte aligned.  Used to
 * measure the achievable HBM read bandwidth that the GEMV is compared with.
 */
int migemm_hbm_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);
int migemm_hbm_read_sink_words(void);

/*
 * Shader clock probe: `blocks` single-wave workgroups (up to 65535) each
 * read the shader-clock counter and the 100 MHz real-time counter around a
 * chain of `iters` dependent FMAs and write the two elapsed counts to
 * out[2*b] and out[2*b + 1] (device, 8-byte aligned, 2 * blocks words).
 * sum(out[2b]) / sum(out[2b+1]) * 100 MHz is the clock the GPU ran at; run
 * right after a kernel on the same stream it gives the clock that kernel
 * left the chip at.  Used to state measured rates against the measured
 * clock as well as the nominal one.
 */
int migemm_clock_probe(uint64_t *out, int blocks, int iters, void *stream);

/*
 * gemm_ex that also records, for each workgroup, the shader-clock and
 * 100 MHz real-time counts its wave 0 ran for: clocks[2*g] and
 * clocks[2*g + 1] for workgroup g (device, 8-byte aligned, 2 * grid words,
 * grid as migemm_gemm_plan_for reports).  sum(clocks[2g]) /
 * sum(clocks[2g+1]) * 100 MHz is the clock the GEMM itself ran at (the
 * chip lowers it under load within microseconds, so a probe after the
 * kernel would not see it).  Full-line tiles only (MIGEMM_ERR_CONFIG
 * otherwise); C is computed exactly as by gemm_ex.  For measurement.
 */
int migemm_gemm_clocked(int dtype, const uint16_t *A, const uint16_t *B, uint16_t *C, int M, int N,
                        int K, int tile, int group_m, int xcd_remap, uint64_t *clocks, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MIGEMM_H */
