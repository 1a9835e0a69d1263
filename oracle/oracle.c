/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the dense
 * column-major GEMM and the decode GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source with the HIP library.
 *
 * What it follows:
 *  - "MTT S4000 GEMM 优化中的分块、尾处理与并发实战复盘" (blog.mthreads.com,
 *    GEMM03), section 1 (rules table): FP16 inputs, FP32 accumulation, FP16
 *    output, column-major A/B/C, inputs never modified, no skipped work.
 *  - same page, section 2 (GEMM basics): the triple loop over n, m, k, and
 *    the column-major addressing A(m,k) -> A[m + k*M], B(k,n) -> B[k + n*K],
 *    C(m,n) -> C[m + n*M]; the work is 2*M*N*K floating-point operations.
 *  - "DCU decode" forum page (forum.sourcefind.cn, db785961), section 6.1:
 *    the linear layer Y = X W^T with X:[n,k], W:[m,k], Y:[n,m].
 *  - FlagGems "Hygon 优化" page, section "分组调度" (grouped scheduling): the
 *    GROUP_M map from a flat program id to an output tile.
 *  - the 8-bit GEMM (FP8 E4M3 / E5M2, INT8 inputs: the 8-bit element types
 *    of gfx950's matrix instructions) in the k-major layout of the DCU page's
 *    Y = X W^T, with one scale and a BF16 output (see oracle_gemm_tn_q).
 *  - "DCU decode" page, section 6.1 (attention shapes: per query head
 *    scores = Q K^T over the L cached tokens, prob = softmax(scores),
 *    out = prob V; KV cache kept in pages [block, token_in_block, kv_head,
 *    head_dim]) and section 6.3 (the split of K/V along L into contiguous
 *    segments, each with a local max, a local softmax denominator and a
 *    local prob V, merged with a numerically stable global reduction).
 *
 * Arithmetic: every 16-bit input is decoded exactly to double; every product
 * of two decoded inputs is exact in double (11+11 or 8+8 significand bits);
 * the k-sum runs in ascending k in double; the result is rounded ONCE, from
 * double, to the output format with IEEE round-to-nearest-even.  The pages
 * ask for FP32 accumulation but leave the order open, so the double sum is
 * the reference point and the test tolerance covers any FP32 order.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <fenv.h>
#include <omp.h>

#define ORACLE_FP16 0
#define ORACLE_BF16 1

/* ---- IEEE binary16 / bfloat16 codecs (exact decode, RNE encode) -------- */

/* Format parameters: stored mantissa bits, exponent bias, min normal
 * exponent, max finite exponent, exponent-field width. */
typedef struct { int mbits, bias, emin, emax, ebits; } fmt_t;
static const fmt_t FMT[2] = {
    {10, 15, -14, 15, 5},     /* binary16 */
    {7, 127, -126, 127, 8},   /* bfloat16 */
};

double oracle_decode(int fmt, uint16_t h)
{
    const fmt_t f = FMT[fmt];
    int sign = (h >> 15) & 1;
    int e = (h >> f.mbits) & ((1 << f.ebits) - 1);
    int man = h & ((1 << f.mbits) - 1);
    double v;
    if (e == 0) {                       /* zero or subnormal */
        v = ldexp((double)man, f.emin - f.mbits);
    } else if (e == (1 << f.ebits) - 1) {
        v = man ? NAN : INFINITY;
    } else {                            /* normal: (1.man) * 2^(e-bias) */
        v = ldexp((double)((1 << f.mbits) + man), e - f.bias - f.mbits);
    }
    return sign ? -v : v;
}

/* Round a double to the 16-bit format, nearest-even, in one step. */
uint16_t oracle_encode(int fmt, double x)
{
    const fmt_t f = FMT[fmt];
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    uint16_t inf = (uint16_t)(((1 << f.ebits) - 1) << f.mbits);
    if (isnan(x))
        return (uint16_t)(sign | inf | (1 << (f.mbits - 1)));   /* quiet NaN */
    double a = fabs(x);
    if (isinf(a))
        return sign | inf;
    if (a == 0.0)
        return sign;
    int E;
    frexp(a, &E);                       /* a = frac * 2^E, frac in [0.5, 1) */
    int e = E - 1;                      /* a in [2^e, 2^(e+1)) */
    if (e < f.emin)
        e = f.emin;                     /* subnormal range: fixed quantum */
    /* Quantum of the target format in this binade; a/q is exact (power-of-2
     * scaling, far from double's own limits). */
    double r = ldexp(a, f.mbits - e);
    double n = nearbyint(r);            /* default mode: ties to even */
    if (n >= ldexp(1.0, f.mbits + 1)) { /* rounded up into the next binade */
        n = ldexp(n, -1);
        e += 1;
    }
    if (e > f.emax)
        return sign | inf;              /* overflow */
    uint32_t ni = (uint32_t)n;
    if (ni < (1u << f.mbits))           /* still subnormal (only when e==emin) */
        return (uint16_t)(sign | ni);
    return (uint16_t)(sign | ((uint32_t)(e + f.bias) << f.mbits) |
                      (ni - (1u << f.mbits)));
}

void oracle_decode_array(int fmt, const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_decode(fmt, in[i]);
}

void oracle_encode_array(int fmt, const double *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_encode(fmt, in[i]);
}

/* ---- the GEMM: one output entry, straight from the definition ---------- */

/* C(m,n) = sum_k A(m,k) * B(k,n) with A(m,k) = A[m + k*M], B(k,n) = B[k + n*K].
 * Also returns S_abs = sum_k |A(m,k)| * |B(k,n)| (the scale of the error
 * bound).  Adds the number of multiply-adds it performed to *macs. */
static double gemm_entry(int fmt, const uint16_t *A, const uint16_t *B,
                         int64_t M, int64_t K, int64_t m, int64_t n,
                         double *sabs, int64_t *macs)
{
    double s = 0.0, sa = 0.0;
    int64_t cnt = 0;
    for (int64_t k = 0; k < K; ++k) {
        double a = oracle_decode(fmt, A[m + k * M]);
        double b = oracle_decode(fmt, B[k + n * K]);
        s += a * b;
        sa += fabs(a) * fabs(b);
        ++cnt;
    }
    *sabs = sa;
    *macs += cnt;
    return s;
}

/* Full GEMM.  Outputs (each may be NULL): C in the output format, Cx the
 * unrounded double sum, S the S_abs scale; all column-major M x N.
 * Returns the number of multiply-adds performed (must be M*N*K). */
int64_t oracle_gemm(int fmt, const uint16_t *A, const uint16_t *B,
                    uint16_t *C, double *Cx, double *S,
                    int M, int N, int K)
{
    int64_t total = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(+ : total)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double sabs;
            double s = gemm_entry(fmt, A, B, M, K, m, n, &sabs, &total);
            int64_t o = m + n * (int64_t)M;
            if (C) C[o] = oracle_encode(fmt, s);
            if (Cx) Cx[o] = s;
            if (S) S[o] = sabs;
        }
    }
    return total;
}

/* The same quantities at a list of flat column-major output indices
 * idx[i] = m + n*M.  Outputs are indexed by position in the list. */
int64_t oracle_gemm_sampled(int fmt, const uint16_t *A, const uint16_t *B,
                            int M, int N, int K, const int64_t *idx,
                            int64_t count, uint16_t *C, double *Cx, double *S)
{
    (void)N;
    int64_t total = 0;
    #pragma omp parallel for schedule(dynamic, 4) reduction(+ : total)
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = idx[i] % M, n = idx[i] / M;
        double sabs;
        double s = gemm_entry(fmt, A, B, M, K, m, n, &sabs, &total);
        if (C) C[i] = oracle_encode(fmt, s);
        if (Cx) Cx[i] = s;
        if (S) S[i] = sabs;
    }
    return total;
}

/* ---- 8-bit element types ------------------------------------------------
 * OCP 8-bit floating point (gfx950's matrix instructions take FP8 E4M3
 * and E5M2): E4M3 has 1 sign, 4 exponent (bias 7) and 3
 * mantissa bits, no infinities, S.1111.111 is NaN (largest finite 448);
 * E5M2 has 5 exponent bits (bias 15) and 2 mantissa bits with IEEE-style
 * infinities and NaNs (largest finite 57344).  Both have subnormals.
 * INT8 is two's complement. */
#define ORACLE_F8E4M3 2
#define ORACLE_F8E5M2 3
#define ORACLE_I8 4

double oracle_decode8(int fmt, uint8_t v)
{
    if (fmt == ORACLE_I8) return (double)(int8_t)v;
    const int e4 = fmt == ORACLE_F8E4M3;
    const int mbits = e4 ? 3 : 2, bias = e4 ? 7 : 15, emax_field = e4 ? 15 : 31;
    const int sign = v >> 7, e = (v >> mbits) & emax_field, man = v & ((1 << mbits) - 1);
    double x;
    if (e == 0)
        x = ldexp((double)man, 1 - bias - mbits);
    else if (e4 && e == 15 && man == 7)
        x = NAN;
    else if (!e4 && e == 31)
        x = man ? NAN : INFINITY;
    else
        x = ldexp((double)((1 << mbits) + man), e - bias - mbits);
    return sign ? -x : x;
}

void oracle_decode8_array(int fmt, const uint8_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_decode8(fmt, in[i]);
}

/* 8-bit GEMM with A k-major ("TN"): C(m,n) = C[m + n*M], A(m,k) =
 * At[k + m*K], B(k,n) = B[k + n*K]; s = sum_k A(m,k) B(k,n) exactly (every
 * 8-bit value and product is exact in double, and so are these sums).
 * Output: FP8: BF16_RNE(scale * s), rounded once from double; INT8: the sum
 * is an integer, taken to FP32 (RNE), multiplied by scale in FP32 (RNE),
 * then rounded to BF16 -- the FP32 steps that define the INT8 output.
 * Cx = the value before the BF16 rounding, S = |scale| * sum_k |a||b|.
 * All M*N outputs (idx == NULL, column-major) or those at idx[0..count). */
int64_t oracle_gemm_tn_q(int fmt, const uint8_t *At, const uint8_t *B, int M, int N, int K,
                         float scale, const int64_t *idx, int64_t count,
                         uint16_t *C, double *Cx, double *S)
{
    const int64_t total_out = idx ? count : (int64_t)M * N;
    int64_t total = 0;
    #pragma omp parallel for schedule(dynamic, 16) reduction(+ : total)
    for (int64_t i = 0; i < total_out; ++i) {
        const int64_t o = idx ? idx[i] : i;
        const int64_t m = o % M, n = o / M;
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = oracle_decode8(fmt, At[k + m * (int64_t)K]);
            double b = oracle_decode8(fmt, B[k + n * (int64_t)K]);
            s += a * b;
            sa += fabs(a) * fabs(b);
            ++total;
        }
        double v;
        if (fmt == ORACLE_I8) {
            volatile float f = (float)s;          /* FP32, round to nearest even */
            volatile float p = f * scale;         /* one FP32 multiply */
            v = (double)p;
        } else {
            v = (double)scale * s;
        }
        if (C) C[i] = oracle_encode(ORACLE_BF16, v);
        if (Cx) Cx[i] = v;
        if (S) S[i] = fabs((double)scale) * sa;
    }
    return total;
}

/* ---- the decode GEMV: Y = X W^T ---------------------------------------- */

/* W row-major [M,K], X row-major [n,K], Y row-major [n,M]:
 * Y[i*M + j] = sum_k X[i*K + k] * W[j*K + k]. */
int64_t oracle_gemv(int fmt, const uint16_t *W, const uint16_t *X,
                    uint16_t *Y, double *Yx, double *S,
                    int M, int K, int n)
{
    int64_t total = 0;
    #pragma omp parallel for schedule(dynamic, 64) reduction(+ : total)
    for (int64_t j = 0; j < M; ++j) {
        for (int64_t i = 0; i < n; ++i) {
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double x = oracle_decode(fmt, X[i * K + k]);
                double w = oracle_decode(fmt, W[j * K + k]);
                s += x * w;
                sa += fabs(x) * fabs(w);
                ++total;
            }
            int64_t o = i * (int64_t)M + j;
            if (Y) Y[o] = oracle_encode(fmt, s);
            if (Yx) Yx[o] = s;
            if (S) S[o] = sa;
        }
    }
    return total;
}

/* ---- grouped tile ordering (FlagGems Hygon page, grouped scheduling) ---- */

/* The whole grouped ordering, written out by walking the tiles in the order
 * the page's grouping visits them: tile rows taken in groups of group_m (the
 * last group keeps what is left), inside a group every tile column in turn,
 * inside a column the group's rows top to bottom.  Entry p of the arrays is
 * the tile of program id p; both arrays hold num_pid_m * num_pid_n entries. */
void oracle_grouped_order(int64_t num_pid_m, int64_t num_pid_n, int64_t group_m,
                          int64_t *pid_m, int64_t *pid_n)
{
    int64_t p = 0;
    for (int64_t first = 0; first < num_pid_m; first += group_m) {
        int64_t last = first + group_m;
        if (last > num_pid_m) last = num_pid_m;
        for (int64_t col = 0; col < num_pid_n; ++col)
            for (int64_t row = first; row < last; ++row) {
                pid_m[p] = row;
                pid_n[p] = col;
                ++p;
            }
    }
}

/* One program id's tile: the same walk, stopped at that id. */
void oracle_grouped_tile(int64_t pid, int64_t num_pid_m, int64_t num_pid_n,
                         int64_t group_m, int64_t *pid_m, int64_t *pid_n)
{
    int64_t p = 0;
    *pid_m = -1;
    *pid_n = -1;
    for (int64_t first = 0; first < num_pid_m; first += group_m) {
        int64_t last = first + group_m;
        if (last > num_pid_m) last = num_pid_m;
        const int64_t span = (last - first) * num_pid_n;     /* ids of this group */
        if (pid >= p + span) {
            p += span;
            continue;
        }
        for (int64_t col = 0; col < num_pid_n; ++col)
            for (int64_t row = first; row < last; ++row, ++p)
                if (p == pid) {
                    *pid_m = row;
                    *pid_n = col;
                    return;
                }
    }
}

/* ---- decode attention (DCU decode page, sections 6.1 and 6.3) ---------- */

/* Row (b, token l, kv head kvh) of a paged cache laid out
 * [block][token_in_block][kv_head][head_dim]: token l of sequence b sits in
 * page block_table[b * max_blocks + l / block_size] at slot l % block_size. */
static const uint16_t *kv_row(const uint16_t *cache, const int32_t *block_table, int b, int64_t l,
                              int kvh, int Hkv, int D, int block_size, int max_blocks)
{
    int64_t blk = block_table[(int64_t)b * max_blocks + l / block_size];
    int64_t slot = l % block_size;
    return cache + ((blk * block_size + slot) * Hkv + kvh) * (int64_t)D;
}

/* The plain definition, one query token per sequence: for sequence b and
 * query head h (kv head h / (Hq / Hkv)),
 *     s_l = scale * sum_d q_d k_ld          (l < L = seq_lens[b])
 *     out_d = sum_l exp(s_l - max s) v_ld / sum_l exp(s_l - max s)
 * in double; out rounded once.  Also S_d = sum_l p_l |v_ld| (the scale of
 * the terms the tolerance is relative to) and QKabs[b][h] = max_l |scale| *
 * sum_d |q_d k_ld| (what bounds a score's summation error).  L = 0 gives
 * out = 0.  Q, Out: [B][Hq][D].  Returns the multiply-adds (2 per (l, d)). */
int64_t oracle_attention(int fmt, const uint16_t *Q, const uint16_t *Kc, const uint16_t *Vc,
                         const int32_t *block_table, const int32_t *seq_lens, int B, int Hq,
                         int Hkv, int D, int block_size, int max_blocks, double scale,
                         uint16_t *Out, double *Ox, double *S, double *QKabs)
{
    int64_t total = 0;
    const int G = Hq / Hkv;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1) reduction(+ : total)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            const int L = seq_lens[b], kvh = h / G;
            const uint16_t *q = Q + ((int64_t)b * Hq + h) * D;
            double *sc = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
            double mx = -INFINITY, qka = 0.0;
            for (int64_t l = 0; l < L; ++l) {
                const uint16_t *k = kv_row(Kc, block_table, b, l, kvh, Hkv, D, block_size, max_blocks);
                double s = 0.0, sa = 0.0;
                for (int d = 0; d < D; ++d) {
                    const double qd = oracle_decode(fmt, q[d]), kd = oracle_decode(fmt, k[d]);
                    s += qd * kd;
                    sa += fabs(qd * kd);
                }
                sc[l] = scale * s;
                if (sc[l] > mx) mx = sc[l];
                if (fabs(scale) * sa > qka) qka = fabs(scale) * sa;
                total += D;
            }
            if (QKabs) QKabs[(int64_t)b * Hq + h] = qka;
            double z = 0.0;
            for (int64_t l = 0; l < L; ++l) { sc[l] = exp(sc[l] - mx); z += sc[l]; }
            for (int d = 0; d < D; ++d) {
                double o = 0.0, sa = 0.0;
                for (int64_t l = 0; l < L; ++l) {
                    double v = oracle_decode(fmt, kv_row(Vc, block_table, b, l, kvh, Hkv, D, block_size, max_blocks)[d]);
                    o += sc[l] * v;
                    sa += sc[l] * fabs(v);
                }
                total += L;
                const int64_t i = ((int64_t)b * Hq + h) * D + d;
                const double out = L > 0 ? o / z : 0.0;
                if (Out) Out[i] = oracle_encode(fmt, out);
                if (Ox) Ox[i] = out;
                if (S) S[i] = L > 0 ? sa / z : 0.0;
            }
            free(sc);
        }
    }
    return total;
}

/* The page's segmented algorithm (section 6.3), in its own steps: tokens
 * [0, L) split into nseg contiguous segments of ceil(L / nseg) tokens (the
 * last ones shorter or empty).  Segment i keeps its local max m_i, local
 * denominator l_i = sum exp(s - m_i) and local o_i = sum exp(s - m_i) v;
 * the merge takes M = max m_i and out = sum_i o_i e^(m_i - M) /
 * sum_i l_i e^(m_i - M).  Empty segments (m_i = -inf) contribute nothing.
 * Equal to oracle_attention up to double rounding. */
void oracle_attention_segmented(int fmt, const uint16_t *Q, const uint16_t *Kc, const uint16_t *Vc,
                                const int32_t *block_table, const int32_t *seq_lens, int B, int Hq,
                                int Hkv, int D, int block_size, int max_blocks, double scale,
                                int nseg, uint16_t *Out, double *Ox)
{
    const int G = Hq / Hkv;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            const int L = seq_lens[b], kvh = h / G;
            const int64_t seg = (L + nseg - 1) / nseg;
            const uint16_t *q = Q + ((int64_t)b * Hq + h) * D;
            double *m = (double *)malloc(sizeof(double) * nseg);
            double *ls = (double *)malloc(sizeof(double) * nseg);
            double *o = (double *)calloc((size_t)nseg * D, sizeof(double));
            for (int i = 0; i < nseg; ++i) {
                const int64_t l0 = i * seg, l1 = (l0 + seg < L) ? l0 + seg : L;
                m[i] = -INFINITY;
                ls[i] = 0.0;
                for (int64_t l = l0; l < l1; ++l) {
                    const uint16_t *k = kv_row(Kc, block_table, b, l, kvh, Hkv, D, block_size, max_blocks);
                    double s = 0.0;
                    for (int d = 0; d < D; ++d) s += oracle_decode(fmt, q[d]) * oracle_decode(fmt, k[d]);
                    if (scale * s > m[i]) m[i] = scale * s;
                }
                for (int64_t l = l0; l < l1; ++l) {
                    const uint16_t *k = kv_row(Kc, block_table, b, l, kvh, Hkv, D, block_size, max_blocks);
                    const uint16_t *v = kv_row(Vc, block_table, b, l, kvh, Hkv, D, block_size, max_blocks);
                    double s = 0.0;
                    for (int d = 0; d < D; ++d) s += oracle_decode(fmt, q[d]) * oracle_decode(fmt, k[d]);
                    const double p = exp(scale * s - m[i]);
                    ls[i] += p;
                    for (int d = 0; d < D; ++d) o[(int64_t)i * D + d] += p * oracle_decode(fmt, v[d]);
                }
            }
            double M = -INFINITY;
            for (int i = 0; i < nseg; ++i) if (m[i] > M) M = m[i];
            double z = 0.0;
            for (int i = 0; i < nseg; ++i) if (ls[i] > 0.0) z += ls[i] * exp(m[i] - M);
            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int i = 0; i < nseg; ++i) if (ls[i] > 0.0) acc += o[(int64_t)i * D + d] * exp(m[i] - M);
                const int64_t idx = ((int64_t)b * Hq + h) * D + d;
                const double out = z > 0.0 ? acc / z : 0.0;
                if (Out) Out[idx] = oracle_encode(fmt, out);
                if (Ox) Ox[idx] = out;
            }
            free(m); free(ls); free(o);
        }
    }
}

int oracle_abi_version(void) { return 3; }

/* ---- threads ------------------------------------------------------------- */

/* Number of OpenMP threads the oracle's loops use from now on (n >= 1); the
 * result of every function is the same for any count, only its time
 * changes.  Returns the count in force before the call. */
int oracle_set_threads(int n)
{
    const int before = omp_get_max_threads();
    if (n >= 1) omp_set_num_threads(n);
    return before;
}
