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

/* Flat program id -> output tile (pid_m, pid_n).  Consecutive ids walk down
 * a group of up to group_m tile rows before moving to the next tile column,
 * so a group shares one B panel; the last group may hold fewer rows. */
void oracle_grouped_tile(int64_t pid, int64_t num_pid_m, int64_t num_pid_n,
                         int64_t group_m, int64_t *pid_m, int64_t *pid_n)
{
    int64_t per_group = group_m * num_pid_n;     /* programs in one group */
    int64_t group = pid / per_group;
    int64_t first_m = group * group_m;           /* first tile row of group */
    int64_t rows = num_pid_m - first_m;          /* rows in this group */
    if (rows > group_m) rows = group_m;
    int64_t local = pid % per_group;
    *pid_m = first_m + local % rows;
    *pid_n = local / rows;
}

int oracle_abi_version(void) { return 1; }
