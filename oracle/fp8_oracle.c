/*
 * fp8_oracle.c -- CPU oracle for fine-grained FP8 quantization and the
 * block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark load the shared object built from it.
 *
 * It is written to be read against the method's statement, not to be fast:
 * every value is computed the plain way, floating-point work that has an
 * exact definition is done in double precision, and the only liberties are
 * a 256-entry decode table (decode of each byte, computed once) and threads
 * over independent output elements.
 *
 * What the method computes, as the source pages state it:
 *   - all GEMM inputs use E4M3 (4 exponent bits, 3 mantissa bits)
 *     (jp-study.kr page, the passage adopting E4M3 on all tensors);
 *   - activations are grouped and scaled per 1x128 tile (one token, 128
 *     channels); weights per 128x128 block ("Should Fixing Deepseek Take 60
 *     Steps?", Figure 7(a));
 *   - the scale maps each group's maximum absolute value, computed online,
 *     onto the largest finite E4M3 value (why-be.why-be.co.kr page, online
 *     max-abs passage; "Should Fixing Deepseek Take 60 Steps?", max-abs
 *     scaling passage);
 *   - the GEMM consumes the FP8 operands, multiplies each partial result of
 *     a 128-wide K interval by the two block scales and accumulates in FP32
 *     ("promotion", jp-study.kr page, Figure 7(b)); outputs are BF16 or FP32
 *     ("Should Fixing Deepseek Take 60 Steps?", GEMM passage).
 *
 * Readings where the pages are silent (each is also listed in the design
 * notes of the repository):
 *   - E4M3 is the OCP "E4M3FN" encoding: bias 7, no infinities, NaN only at
 *     S.1111.111, largest finite magnitude 448.
 *   - Encoding rounds to nearest, ties to even mantissa, and saturates at
 *     +-448; the sign of zero is kept.
 *   - The stored scale is the dequantization factor s = fl32(amax / 448);
 *     quantization multiplies by inv = min(fl32(448 / amax), FLT_MAX), both
 *     IEEE single-precision divisions, then encodes fl32(x * inv).
 *   - The GEMM reference is the exact per-K-block sum: the fp64 value of
 *     sum_kb (sa*sb) * sum_{k in kb} dec(a)*dec(b).  Each per-block sum of
 *     products of two E4M3 values is exact in fp64, so the only roundings
 *     are the scale product times partial and the running sum over blocks.
 *
 * A second scale rule serves the hardware-scaled variant: the scale is the
 * power of two 2^e (smallest e with amax <= 448 * 2^e, e in [-127, 127]),
 * the value an E8M0 exponent carries, so that the matrix instruction can
 * apply it.  The pages ask for hardware that applies group scales inside
 * the matrix multiply (why-be.why-be.co.kr page, hardware-design passage).
 *
 * Parity pins: every function here is checked by the CPU test-suite against
 * closed forms, a brute-force nearest-value encoder, PyTorch's own E4M3 cast,
 * exact rational arithmetic and integer matmul (tests/test_oracle_*.py).
 */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* E4M3 (OCP E4M3FN) decode and encode                                       */
/* ------------------------------------------------------------------------ */

/* Byte layout s eeee mmm.  e == 0: subnormal m * 2^-9.  Otherwise
 * (1 + m/8) * 2^(e-7), except e == 15 && m == 7 which is NaN. */
OR_EXPORT double or_e4m3_decode(uint8_t b) {
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(8.0 + (double)m, e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

static double g_dec[256];        /* decode of every byte                   */
static double g_pos[127];        /* magnitudes of codes 0x00 .. 0x7E        */
static pthread_once_t g_once = PTHREAD_ONCE_INIT;

static void init_tables(void) {
    for (int b = 0; b < 256; ++b) g_dec[b] = or_e4m3_decode((uint8_t)b);
    for (int c = 0; c <= 0x7E; ++c) g_pos[c] = g_dec[c];
}

static void ensure_tables(void) { pthread_once(&g_once, init_tables); }

/* Round-to-nearest-even, saturating encode of one FP32 value.
 * The positive codes 0x00..0x7E are strictly increasing in magnitude, so the
 * two neighbours of |v| are codes c and c+1.  |v| is compared against the
 * exact midpoint of the two (a value representable in fp64, as is |v|). */
OR_EXPORT uint8_t or_e4m3_encode(float v) {
    ensure_tables();
    uint8_t sgn = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(0x7F | sgn);
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(0x7E | sgn);
    /* largest c in [0, 0x7D] with g_pos[c] <= a (binary search) */
    int lo = 0, hi = 0x7E; /* invariant: g_pos[lo] <= a < g_pos[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (g_pos[mid] <= a) lo = mid; else hi = mid;
    }
    double midpoint = 0.5 * (g_pos[lo] + g_pos[hi]);
    int c;
    if (a < midpoint) c = lo;
    else if (a > midpoint) c = hi;
    else c = (lo % 2 == 0) ? lo : hi; /* tie: even mantissa LSB */
    return (uint8_t)(c | sgn);
}

OR_EXPORT void or_e4m3_encode_array(const float* v, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_e4m3_encode(v[i]);
}

OR_EXPORT void or_e4m3_decode_array(const uint8_t* b, double* out, int64_t n) {
    ensure_tables();
    for (int64_t i = 0; i < n; ++i) out[i] = g_dec[b[i]];
}

/* ------------------------------------------------------------------------ */
/* Group quantization                                                        */
/* ------------------------------------------------------------------------ */

enum { OR_F32 = 0, OR_BF16 = 1 };

/* Element (i) of a tensor given as FP32 or as BF16 bit patterns; widening
 * BF16 to FP32 is exact (append 16 zero bits). */
static float load_elem(const void* x, int dtype, int64_t idx) {
    if (dtype == OR_F32) return ((const float*)x)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)x)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Scale rule for one group with maximum absolute value amax. */
OR_EXPORT void or_group_scale(float amax, float* s, float* inv) {
    volatile float a = amax;            /* keep the divisions in FP32 */
    float sc = a / 448.0f;
    float iv = 448.0f / a;              /* +inf when amax == 0          */
    if (!(iv <= FLT_MAX)) iv = FLT_MAX; /* clamp +inf to FLT_MAX         */
    *s = sc;
    *inv = iv;
}

/* Power-of-two scale rule (the scale an E8M0 exponent can carry): s = 2^e
 * with e the smallest integer such that amax <= 448 * 2^e, clamped to the
 * E8M0 range [-127, 127] (amax == 0 gives e = -127); inv = 2^-e.  Found by
 * direct search in fp64, where 448 * 2^e and amax are exact. */
OR_EXPORT void or_group_scale_pow2(float amax, float* s, float* inv) {
    int e = -127;
    if (amax > 0.0f) {
        double a = (double)amax;
        e = 0;
        while (ldexp(448.0, e) < a) ++e;
        while (ldexp(448.0, e - 1) >= a) --e;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
    }
    *s = ldexpf(1.0f, e);
    *inv = ldexpf(1.0f, -e);
}

enum { OR_RULE_FP32 = 0, OR_RULE_POW2 = 1 };

static void group_scale_rule(int rule, float amax, float* s, float* inv) {
    if (rule == OR_RULE_POW2) or_group_scale_pow2(amax, s, inv);
    else or_group_scale(amax, s, inv);
}

static uint8_t quant_one(float x, float inv) {
    volatile float p = x * inv;         /* one FP32 product, RNE */
    return or_e4m3_encode(p);
}

/* 1x128 groups along the column index of a logical [rows, cols] matrix whose
 * element (r, c) sits at x[r*xs_r + c*xs_c].  Writes q[r*ldq + c] and
 * s[g*lds + r] for g < ceil(cols/128).  A partial last group covers the
 * columns present. */
typedef struct {
    const void* x; int dtype; int64_t rows, cols, xs_r, xs_c;
    uint8_t* q; int64_t ldq; float* s; int64_t lds;
    int64_t r0, r1;
    int rule;
} q1x128_job;

static void* q1x128_worker(void* p) {
    q1x128_job* j = (q1x128_job*)p;
    int64_t groups = (j->cols + 127) / 128;
    for (int64_t r = j->r0; r < j->r1; ++r) {
        for (int64_t g = 0; g < groups; ++g) {
            int64_t c0 = g * 128, c1 = c0 + 128 < j->cols ? c0 + 128 : j->cols;
            float amax = 0.0f;
            for (int64_t c = c0; c < c1; ++c) {
                float v = fabsf(load_elem(j->x, j->dtype, r * j->xs_r + c * j->xs_c));
                if (v > amax) amax = v;
            }
            float s, inv;
            group_scale_rule(j->rule, amax, &s, &inv);
            j->s[g * j->lds + r] = s;
            for (int64_t c = c0; c < c1; ++c)
                j->q[r * j->ldq + c] =
                    quant_one(load_elem(j->x, j->dtype, r * j->xs_r + c * j->xs_c), inv);
        }
    }
    return NULL;
}

static int clamp_threads(int nthreads, int64_t work) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (work < nthreads) nthreads = work > 0 ? (int)work : 1;
    return nthreads;
}

OR_EXPORT void or_quant_1x128_rule(const void* x, int dtype, int64_t rows, int64_t cols,
                                   int64_t xs_r, int64_t xs_c, uint8_t* q, int64_t ldq,
                                   float* s, int64_t lds, int nthreads, int rule) {
    ensure_tables();
    nthreads = clamp_threads(nthreads, rows);
    pthread_t th[256];
    q1x128_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        q1x128_job j = {x, dtype, rows, cols, xs_r, xs_c, q, ldq, s, lds,
                        rows * t / nthreads, rows * (t + 1) / nthreads, rule};
        jobs[t] = j;
        pthread_create(&th[t], NULL, q1x128_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

OR_EXPORT void or_quant_1x128(const void* x, int dtype, int64_t rows, int64_t cols,
                              int64_t xs_r, int64_t xs_c, uint8_t* q, int64_t ldq,
                              float* s, int64_t lds, int nthreads) {
    or_quant_1x128_rule(x, dtype, rows, cols, xs_r, xs_c, q, ldq, s, lds, nthreads,
                        OR_RULE_FP32);
}

/* 128x128 blocks of a row-major [rows, cols] matrix with leading dimension
 * ldw.  Writes q[r*ldq + c], s[(r/128)*ceil(cols/128) + c/128] and, when
 * q_t is not NULL, the transposed codes q_t[c*ldqt + r]. */
typedef struct {
    const void* w; int dtype; int64_t rows, cols, ldw;
    uint8_t* q; int64_t ldq; float* s; uint8_t* q_t; int64_t ldqt;
    int64_t b0, b1; /* block-row range */
    int rule;
} q128_job;

static void* q128_worker(void* p) {
    q128_job* j = (q128_job*)p;
    int64_t gc = (j->cols + 127) / 128;
    for (int64_t bi = j->b0; bi < j->b1; ++bi) {
        for (int64_t bj = 0; bj < gc; ++bj) {
            int64_t r0 = bi * 128, r1 = r0 + 128 < j->rows ? r0 + 128 : j->rows;
            int64_t c0 = bj * 128, c1 = c0 + 128 < j->cols ? c0 + 128 : j->cols;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float v = fabsf(load_elem(j->w, j->dtype, r * j->ldw + c));
                    if (v > amax) amax = v;
                }
            float s, inv;
            group_scale_rule(j->rule, amax, &s, &inv);
            j->s[bi * gc + bj] = s;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    uint8_t code = quant_one(load_elem(j->w, j->dtype, r * j->ldw + c), inv);
                    j->q[r * j->ldq + c] = code;
                    if (j->q_t) j->q_t[c * j->ldqt + r] = code;
                }
        }
    }
    return NULL;
}

OR_EXPORT void or_quant_128x128_rule(const void* w, int dtype, int64_t rows, int64_t cols,
                                     int64_t ldw, uint8_t* q, int64_t ldq, float* s,
                                     uint8_t* q_t, int64_t ldqt, int nthreads, int rule) {
    ensure_tables();
    int64_t gr = (rows + 127) / 128;
    nthreads = clamp_threads(nthreads, gr);
    pthread_t th[256];
    q128_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        q128_job j = {w, dtype, rows, cols, ldw, q, ldq, s, q_t, ldqt,
                      gr * t / nthreads, gr * (t + 1) / nthreads, rule};
        jobs[t] = j;
        pthread_create(&th[t], NULL, q128_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

OR_EXPORT void or_quant_128x128(const void* w, int dtype, int64_t rows, int64_t cols,
                                int64_t ldw, uint8_t* q, int64_t ldq, float* s,
                                uint8_t* q_t, int64_t ldqt, int nthreads) {
    or_quant_128x128_rule(w, dtype, rows, cols, ldw, q, ldq, s, q_t, ldqt, nthreads,
                          OR_RULE_FP32);
}

/* ------------------------------------------------------------------------ */
/* Block-scaled GEMM, exact per 128-wide K block                             */
/* ------------------------------------------------------------------------ */

enum { OR_SCALE_BLOCK128 = 0, OR_SCALE_ROW128 = 1 };

/* C*[m,n] = sum_kb (sa[m,kb] * sb[n,kb]) * sum_{k in kb} dec(a[m,k]) dec(b[n,k])
 * and the error denominator
 * S[m,n]  = sum_kb |sa*sb| * sum_{k in kb} |dec(a[m,k]) dec(b[n,k])|.
 * sa[kb*ldsa + m].  BLOCK128: sb[(n/128)*sbs0 + kb*sbs1].  ROW128:
 * sb[kb*sbs0 + n]. */
static void gemm_elem(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                      const uint8_t* b, int64_t ldb, const float* sb, int mode,
                      int64_t sbs0, int64_t sbs1, int64_t K, int64_t m, int64_t n,
                      double* c_out, double* s_out) {
    double acc = 0.0, den = 0.0;
    int64_t nkb = K / 128;
    const uint8_t* arow = a + m * lda;
    const uint8_t* brow = b + n * ldb;
    for (int64_t kb = 0; kb < nkb; ++kb) {
        double part = 0.0, part_abs = 0.0;
        for (int64_t k = kb * 128; k < kb * 128 + 128; ++k) {
            double prod = g_dec[arow[k]] * g_dec[brow[k]]; /* exact */
            part += prod;                                  /* exact */
            part_abs += fabs(prod);                        /* exact */
        }
        double sav = (double)sa[kb * ldsa + m];
        double sbv = (mode == OR_SCALE_BLOCK128) ? (double)sb[(n / 128) * sbs0 + kb * sbs1]
                                                 : (double)sb[kb * sbs0 + n];
        double sab = sav * sbv; /* exact: 24-bit x 24-bit */
        acc += sab * part;
        den += fabs(sab) * part_abs;
    }
    *c_out = acc;
    *s_out = den;
}

typedef struct {
    const uint8_t* a; int64_t lda; const float* sa; int64_t ldsa;
    const uint8_t* b; int64_t ldb; const float* sb; int mode; int64_t sbs0, sbs1;
    int64_t K;
    const int64_t* mi; const int64_t* ni; int64_t count; /* element list      */
    int64_t N;                                           /* full mode: cols   */
    double* c; double* s;
    int64_t e0, e1;
    /* grouped mode */
    const int32_t* offsets; int64_t num_groups; int64_t gstride_b; int64_t gstride_sb;
} gemm_job;

static int64_t find_group(const int32_t* off, int64_t G, int64_t m) {
    /* largest g with off[g] <= m, among groups that are non-empty at m */
    int64_t lo = 0, hi = G; /* off[lo] <= m < off[hi] */
    while (hi - lo > 1) {
        int64_t mid = (lo + hi) / 2;
        if ((int64_t)off[mid] <= m) lo = mid; else hi = mid;
    }
    return lo;
}

static void* gemm_worker(void* p) {
    gemm_job* j = (gemm_job*)p;
    for (int64_t e = j->e0; e < j->e1; ++e) {
        int64_t m, n;
        if (j->mi) { m = j->mi[e]; n = j->ni[e]; }
        else { m = e / j->N; n = e % j->N; }
        const uint8_t* b = j->b;
        const float* sb = j->sb;
        if (j->offsets) {
            int64_t g = find_group(j->offsets, j->num_groups, m);
            b += g * j->gstride_b;
            sb += g * j->gstride_sb;
        }
        gemm_elem(j->a, j->lda, j->sa, j->ldsa, b, j->ldb, sb, j->mode, j->sbs0, j->sbs1,
                  j->K, m, n, &j->c[e], &j->s[e]);
    }
    return NULL;
}

static void run_gemm_jobs(gemm_job proto, int64_t total, int nthreads) {
    ensure_tables();
    nthreads = clamp_threads(nthreads, total);
    pthread_t th[256];
    gemm_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].e0 = total * t / nthreads;
        jobs[t].e1 = total * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, gemm_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* Full M x N output: c[m*N + n], s[m*N + n]. */
OR_EXPORT void or_gemm_exact(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                             const uint8_t* b, int64_t ldb, const float* sb, int mode,
                             int64_t sbs0, int64_t sbs1, int64_t M, int64_t N, int64_t K,
                             double* c, double* s, int nthreads) {
    gemm_job j;
    memset(&j, 0, sizeof j);
    j.a = a; j.lda = lda; j.sa = sa; j.ldsa = ldsa; j.b = b; j.ldb = ldb; j.sb = sb;
    j.mode = mode; j.sbs0 = sbs0; j.sbs1 = sbs1; j.K = K; j.N = N; j.c = c; j.s = s;
    run_gemm_jobs(j, M * N, nthreads);
}

/* Listed elements (mi[e], ni[e]) only: c[e], s[e]. */
OR_EXPORT void or_gemm_exact_elems(const uint8_t* a, int64_t lda, const float* sa,
                                   int64_t ldsa, const uint8_t* b, int64_t ldb,
                                   const float* sb, int mode, int64_t sbs0, int64_t sbs1,
                                   int64_t K, const int64_t* mi, const int64_t* ni,
                                   int64_t count, double* c, double* s, int nthreads) {
    gemm_job j;
    memset(&j, 0, sizeof j);
    j.a = a; j.lda = lda; j.sa = sa; j.ldsa = ldsa; j.b = b; j.ldb = ldb; j.sb = sb;
    j.mode = mode; j.sbs0 = sbs0; j.sbs1 = sbs1; j.K = K; j.mi = mi; j.ni = ni;
    j.count = count; j.c = c; j.s = s;
    run_gemm_jobs(j, count, nthreads);
}

/* Grouped (MoE) GEMM on listed elements.  Row m belongs to the group g with
 * offsets[g] <= m < offsets[g+1]; that group uses B_g = b + g*N*ldb and the
 * 128x128 block scales sb_g = sb + g*ceil(N/128)*(K/128), laid out
 * [n/128][kb]. */
OR_EXPORT void or_grouped_gemm_exact_elems(const uint8_t* a, int64_t lda, const float* sa,
                                           int64_t ldsa, const uint8_t* b, int64_t ldb,
                                           const float* sb, const int32_t* offsets,
                                           int64_t num_groups, int64_t N, int64_t K,
                                           const int64_t* mi, const int64_t* ni,
                                           int64_t count, double* c, double* s,
                                           int nthreads) {
    gemm_job j;
    memset(&j, 0, sizeof j);
    int64_t kb = K / 128, gn = (N + 127) / 128;
    j.a = a; j.lda = lda; j.sa = sa; j.ldsa = ldsa; j.b = b; j.ldb = ldb; j.sb = sb;
    j.mode = OR_SCALE_BLOCK128; j.sbs0 = kb; j.sbs1 = 1; j.K = K; j.mi = mi; j.ni = ni;
    j.count = count; j.c = c; j.s = s;
    j.offsets = offsets; j.num_groups = num_groups;
    j.gstride_b = N * ldb; j.gstride_sb = gn * kb;
    run_gemm_jobs(j, count, nthreads);
}
