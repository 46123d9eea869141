/*
 * CPU oracle for the block-scaled variant of C = ReLU(A . B): A and B hold
 * 8-bit (E4M3, E5M2) or 4-bit (E2M1) floating-point codes, every 32
 * consecutive elements along K share one power-of-two scale (an E8M0 byte),
 * and C is float16.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it. The product library never
 * links, loads or calls it. It shares no source, header, table or helper with
 * the GPU path (nor with the float16 oracle next to it).
 *
 * Where this comes from. The project page "TileLang: a tile-level DSL for
 * writing GPU kernels in Python" (hysenlabs.com, "Three backends under one
 * language dialect") names FP4 E2M1 matrix cores on CDNA4 (gfx950) and a
 * block-scaled MMA path; the forum post "TileLang: Writing Near-Hardware-
 * Limit GPU Kernels in 70 Lines of Python" (zhichai.net, "Key Technical
 * Milestones") names MXFP8 grouped GEMM with block scaling and a
 * transposed B. Neither page defines the element codes or the scale
 * semantics; the plainest reading is the OCP Microscaling (MX) formats,
 * which both names refer to:
 *   - a block is 32 consecutive elements along K of one row of A (or of one
 *     column of B, i.e. one row of B given transposed, N x K);
 *   - a block's scale is an E8M0 byte e: the value 2^(e - 127); e = 255 is NaN;
 *   - elements are E4M3 (bias 7, no infinities, S.1111.111 is NaN), E5M2
 *     (bias 15, IEEE-style infinities and NaNs) or E2M1 (bias 1, no
 *     infinities or NaNs), each with subnormals;
 *   - C[i][j] = ReLU( sum over blocks b of 2^(sa[i][b]-127) * 2^(sb[j][b]-127)
 *                     * sum over k in block b of a[i][k] * b[j][k] ),
 *     then the float16 copy-out, as in the quick-start kernel's epilogue.
 * The sum is evaluated in binary64, blocks in ascending order and k
 * ascending inside a block; every product of two decoded elements times two
 * power-of-two scales is exact in binary64, and a block's E4M3 or E2M1 sum
 * is exact as well. The result is rounded once, binary64 -> binary16,
 * to nearest with ties to even (subnormals kept, overflow to infinity).
 * ReLU maps x > 0 to x and everything else (-0, NaN) to +0.
 *
 * Storage: row-major, leading dimensions in elements. 8-bit codes are one
 * byte each; 4-bit codes are packed two per byte, element 2t in the low
 * nibble and element 2t+1 in the high nibble of byte t of the row (so a
 * row's leading dimension is even). Scales are M x K/32 (A) and N x K/32 (B)
 * bytes with their own row strides. K must be a multiple of 32.
 *
 * Build with -ffp-contract=off and without -ffast-math.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* element formats (same numbering as the Python wrapper) */
enum { MX_E4M3 = 1, MX_E5M2 = 2, MX_E2M1 = 3 };

/* ---------- element codes -> binary64, from the format definitions ---------- */

/* A code with `eb` exponent bits (bias `bias`) and `mb` fraction bits, sign in
 * the top bit: normal values (1 + f/2^mb) * 2^(e - bias), subnormal values
 * (e == 0) f/2^mb * 2^(1 - bias). Special codes are handled by the callers. */
static double minifloat(uint32_t code, int eb, int mb, int bias) {
    uint32_t sign = (code >> (eb + mb)) & 1u;
    uint32_t e = (code >> mb) & ((1u << eb) - 1u);
    uint32_t f = code & ((1u << mb) - 1u);
    double v;
    if (e == 0)
        v = ldexp((double)f, 1 - bias - mb);
    else
        v = ldexp((double)((1u << mb) + f), (int)e - bias - mb);
    return sign ? -v : v;
}

double oracle_mx_decode(int fmt, uint32_t code) {
    switch (fmt) {
    case MX_E4M3:
        code &= 0xffu;
        if ((code & 0x7fu) == 0x7fu) return NAN; /* S.1111.111 */
        return minifloat(code, 4, 3, 7);
    case MX_E5M2:
        code &= 0xffu;
        if (((code >> 2) & 0x1fu) == 0x1fu) { /* exponent all ones */
            if ((code & 3u) == 0) return (code & 0x80u) ? -INFINITY : INFINITY;
            return NAN;
        }
        return minifloat(code, 5, 2, 15);
    case MX_E2M1:
        return minifloat(code & 0xfu, 2, 1, 1);
    default:
        return NAN;
    }
}

/* E8M0 scale byte: 2^(e - 127); 255 is NaN. */
double oracle_mx_scale(uint32_t e) {
    e &= 0xffu;
    if (e == 255u) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* ---------- binary64 -> binary16, round to nearest, ties to even ---------- */

uint16_t oracle_f64_to_f16(double x) {
    uint64_t u;
    memcpy(&u, &x, sizeof u);
    uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    uint32_t exp = (uint32_t)((u >> 52) & 0x7ffu);
    uint64_t frac = u & 0xfffffffffffffull;
    if (exp == 0x7ffu) return (uint16_t)(sign | (frac ? 0x7e00u : 0x7c00u));
    if (exp == 0) return sign; /* zero or binary64 subnormal: rounds to zero */
    int e = (int)exp - 1023;                    /* value = sig * 2^(e - 52) */
    uint64_t sig = frac | (1ull << 52);         /* 53-bit significand */
    if (e > 15) return (uint16_t)(sign | 0x7c00u);
    /* keep 11 significant bits in the normal range (e >= -14), else a
     * multiple of the subnormal quantum 2^-24 */
    int shift = (e >= -14) ? 42 : (28 - e);
    if (shift > 53) return sign; /* below 2^-25: rounds to zero */
    uint64_t q = sig >> shift;
    uint64_t rem = sig & ((1ull << shift) - 1ull);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1ull))) q += 1ull;
    if (e >= -14) {
        uint32_t bits = ((uint32_t)(e + 15) << 10) + (uint32_t)(q - 1024ull);
        if (bits >= 0x7c00u) bits = 0x7c00u;
        return (uint16_t)(sign | bits);
    }
    return (uint16_t)(sign | (uint32_t)q);
}

static double relu64(double x) { return (x > 0.0) ? x : 0.0; }

uint16_t oracle_mx_relu_to_f16(double acc) { return oracle_f64_to_f16(relu64(acc)); }

/* ---------- element access ---------- */

static uint32_t code_at(int fmt, const uint8_t *X, int64_t ld, int64_t r, int64_t k) {
    if (fmt == MX_E2M1) {
        uint8_t byte = X[(r * ld + k) / 2];
        return ((r * ld + k) % 2 == 0) ? (byte & 0xfu) : (byte >> 4);
    }
    return X[r * ld + k];
}

/* ---------- the definition, one element at a time ---------- */

static double mx_dot(int fmt, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *SA, int64_t ldsa,
                     const uint8_t *B, int64_t ldb, const uint8_t *SB, int64_t ldsb, int64_t i, int64_t j) {
    double acc = 0.0;
    for (int64_t b = 0; b < K / 32; b++) {
        double block = 0.0;
        for (int64_t k = 32 * b; k < 32 * b + 32; k++)
            block = block + oracle_mx_decode(fmt, code_at(fmt, A, lda, i, k)) *
                                oracle_mx_decode(fmt, code_at(fmt, B, ldb, j, k));
        acc = acc + oracle_mx_scale(SA[i * ldsa + b]) * oracle_mx_scale(SB[j * ldsb + b]) * block;
    }
    return acc;
}

static int args_ok(int fmt, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    if (fmt != MX_E4M3 && fmt != MX_E5M2 && fmt != MX_E2M1) return 0;
    if (M < 0 || N < 0 || K < 0 || K % 32) return 0;
    if (fmt == MX_E2M1 && (lda % 2 || ldb % 2)) return 0;
    return 1;
}

/* C[ii[t]][jj[t]] for each t. Returns 0, or -1 on bad arguments. */
int oracle_gemm_relu_mx_elems(int fmt, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *SA, int64_t ldsa,
                              const uint8_t *B, int64_t ldb, const uint8_t *SB, int64_t ldsb, int64_t count,
                              const int64_t *ii, const int64_t *jj, uint16_t *out) {
    if (!args_ok(fmt, 0, 0, K, lda, ldb)) return -1;
    for (int64_t t = 0; t < count; t++)
        out[t] = oracle_mx_relu_to_f16(mx_dot(fmt, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, ii[t], jj[t]));
    return 0;
}

/* ---------- the whole output, rows split between threads ---------- */

typedef struct {
    int fmt;
    int64_t i0, i1, N, K;
    const uint8_t *A;
    int64_t lda;
    const uint8_t *SA;
    int64_t ldsa;
    const uint8_t *B;
    int64_t ldb;
    const uint8_t *SB;
    int64_t ldsb;
    uint16_t *C;
    int64_t ldc;
} mx_job;

static void *mx_worker(void *arg) {
    const mx_job *jb = (const mx_job *)arg;
    for (int64_t i = jb->i0; i < jb->i1; i++)
        for (int64_t j = 0; j < jb->N; j++)
            jb->C[i * jb->ldc + j] = oracle_mx_relu_to_f16(
                mx_dot(jb->fmt, jb->K, jb->A, jb->lda, jb->SA, jb->ldsa, jb->B, jb->ldb, jb->SB, jb->ldsb, i, j));
    return NULL;
}

static int default_threads(void) {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof set, &set) == 0) {
        int n = CPU_COUNT(&set);
        if (n > 0) return n;
    }
    return 1;
}

/* Returns 0 on success, -1 on bad arguments, -2 if threads fail. */
int oracle_gemm_relu_mx(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *SA,
                        int64_t ldsa, const uint8_t *B, int64_t ldb, const uint8_t *SB, int64_t ldsb, uint16_t *C,
                        int64_t ldc, int threads) {
    if (!args_ok(fmt, M, N, K, lda, ldb)) return -1;
    if (M == 0 || N == 0) return 0;
    if (threads <= 0) threads = default_threads();
    if (threads > M) threads = (int)M;
    mx_job *jobs = (mx_job *)calloc((size_t)threads, sizeof(mx_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    int rc = 0;
    if (!jobs || !tids) {
        rc = -2;
    } else {
        int started = 0;
        for (int t = 0; t < threads; t++) {
            jobs[t] = (mx_job){fmt, M * t / threads, M * (t + 1) / threads, N, K, A, lda, SA, ldsa,
                               B, ldb, SB, ldsb, C, ldc};
            if (pthread_create(&tids[t], NULL, mx_worker, &jobs[t]) != 0) {
                rc = -2;
                break;
            }
            started++;
        }
        for (int t = 0; t < started; t++) pthread_join(tids[t], NULL);
    }
    free(jobs);
    free(tids);
    return rc;
}
