/*
 * CPU oracle for C = ReLU(A . B), fp16 inputs, fp32 accumulation, fp16 output.
 *
 * TEST INFRASTRUCTURE ONLY. This file defines what a correct result is. Only
 * the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * may load it. The product library never links, loads or calls it. It shares
 * no source, header, table or helper with the GPU path.
 *
 * What is computed follows the quick-start kernel `matmul_relu` printed in the
 * "Programming model" section of the TileLang article (aiwiki.ai/wiki/tilelang):
 *   - A is an (M, K) float16 tensor and B a (K, N) float16 tensor;
 *   - the accumulator fragment C_local is float32 and is cleared first;
 *   - the tile GEMM adds A.B into the accumulator over the whole K range;
 *   - ReLU is applied elementwise on the float32 accumulator (max with 0);
 *   - the accumulator is then copied out into the float16 output C (M, N).
 * The tile sizes, stage count and thread count in that kernel are a schedule
 * and do not change the mathematics (same section: the scheduling annotations
 * are layered on top of the dataflow).
 *
 * Readings taken where the article is silent (each is listed with its reason
 * in the design notes of the repository):
 *   - accumulation is sequential in ascending k, one fp32 rounding per step;
 *   - ReLU maps acc > 0 to acc and everything else (including -0 and NaN)
 *     to +0;
 *   - the fp32 -> fp16 copy rounds to nearest, ties to even, keeps
 *     subnormals and overflows to infinity;
 *   - strides are in elements, row-major: A[i][k] is at A[i*lda + k];
 *   - M == 0 or N == 0 computes nothing; K == 0 gives the empty sum +0.
 *
 * Conversions are written from the IEEE-754 binary16/binary32 definitions.
 * Build with -ffp-contract=off and without -ffast-math: the accumulation must
 * never be reassociated. (An fp16 x fp16 product is exact in fp32, so fused
 * and unfused multiply-add would give the same bits anyway.)
 */
#define _GNU_SOURCE
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------- IEEE-754 conversions ---------- */

static float bits_to_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* binary16 -> binary32, exact for every input (binary32 has a wider exponent
 * range and a longer significand). Layout of binary16: 1 sign bit, 5 exponent
 * bits with bias 15, 10 fraction bits. */
float oracle_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t exp = (h >> 10) & 0x1fu;
    uint32_t frac = h & 0x3ffu;
    if (exp == 0x1fu) {
        /* infinity (frac == 0) or NaN (payload moved to the top fraction bits) */
        return bits_to_f32(sign | 0x7f800000u | (frac << 13));
    }
    if (exp == 0) {
        if (frac == 0) return bits_to_f32(sign); /* signed zero */
        /* subnormal: value = frac * 2^-24. Normalise: shift the fraction left
         * until its leading one reaches the hidden-bit position (bit 10). */
        int e = -14;
        while ((frac & 0x400u) == 0) {
            frac <<= 1;
            e -= 1;
        }
        frac &= 0x3ffu;
        return bits_to_f32(sign | ((uint32_t)(e + 127) << 23) | (frac << 13));
    }
    /* normal: rebias the exponent from 15 to 127, widen the fraction */
    return bits_to_f32(sign | ((exp - 15u + 127u) << 23) | (frac << 13));
}

/* binary32 -> binary16, round to nearest with ties to even. Values too large
 * round to infinity, values too small become subnormal or zero (gradual
 * underflow). NaN stays NaN (quiet bit set, sign kept). */
uint16_t oracle_f32_to_f16(float f) {
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t exp = (u >> 23) & 0xffu;
    uint32_t frac = u & 0x7fffffu;
    if (exp == 0xffu) {
        if (frac == 0) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | 0x7e00u | (frac >> 13));
    }
    if (exp == 0) {
        /* zero or binary32 subnormal: magnitude below 2^-126, far under half
         * of the smallest binary16 subnormal (2^-25), so it rounds to zero */
        return sign;
    }
    int e = (int)exp - 127;          /* value = sig * 2^(e - 23) */
    uint32_t sig = frac | 0x800000u; /* 24-bit significand with hidden one */
    if (e > 15) return (uint16_t)(sign | 0x7c00u); /* at least 2^16: overflow */
    /* Number of low significand bits to drop. In the normal binary16 range
     * (e >= -14) the result keeps 11 significant bits; below it, the result
     * is a multiple of 2^-24 (the subnormal quantum). */
    int shift = (e >= -14) ? 13 : (-1 - e);
    if (shift > 24) return sign; /* below 2^-25: rounds to zero */
    uint32_t q = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
    if (e >= -14) {
        /* q is in [1024, 2048]; the carry out of the fraction (q == 2048)
         * moves into the exponent, and exponent 31 is infinity */
        uint32_t bits = ((uint32_t)(e + 15) << 10) + (q - 1024u);
        if (bits >= 0x7c00u) bits = 0x7c00u;
        return (uint16_t)(sign | bits);
    }
    /* subnormal result: q is in [0, 1024]; q == 1024 is the smallest normal */
    return (uint16_t)(sign | q);
}

void oracle_f16_to_f32_array(const uint16_t *in, float *out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_f16_to_f32(in[i]);
}

void oracle_f32_to_f16_array(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_f32_to_f16(in[i]);
}

/* ---------- the epilogue: ReLU on fp32, then the fp16 copy-out ---------- */

static float relu_f32(float acc) { return (acc > 0.0f) ? acc : 0.0f; }

uint16_t oracle_relu_to_f16(float acc) { return oracle_f32_to_f16(relu_f32(acc)); }

/* ---------- the definition, one element at a time ---------- */

/* C[i][j] for each requested (i, j): the literal definition, k ascending. */
void oracle_gemm_relu_f16_elems(int64_t K, const uint16_t *A, int64_t lda,
                                const uint16_t *B, int64_t ldb, int64_t count,
                                const int64_t *ii, const int64_t *jj,
                                uint16_t *out) {
    for (int64_t t = 0; t < count; t++) {
        int64_t i = ii[t], j = jj[t];
        float acc = 0.0f;
        for (int64_t k = 0; k < K; k++)
            acc = acc + oracle_f16_to_f32(A[i * lda + k]) * oracle_f16_to_f32(B[k * ldb + j]);
        out[t] = oracle_relu_to_f16(acc);
    }
}

/* The literal i -> j -> k triple loop over the whole output. */
void oracle_gemm_relu_f16_ijk(int64_t M, int64_t N, int64_t K,
                              const uint16_t *A, int64_t lda,
                              const uint16_t *B, int64_t ldb,
                              uint16_t *C, int64_t ldc) {
    for (int64_t i = 0; i < M; i++)
        for (int64_t j = 0; j < N; j++) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; k++)
                acc = acc + oracle_f16_to_f32(A[i * lda + k]) * oracle_f16_to_f32(B[k * ldb + j]);
            C[i * ldc + j] = oracle_relu_to_f16(acc);
        }
}

/* ---------- the same definition, row-parallel, loop order i -> k -> j ----------
 *
 * Every C[i][j] still receives exactly the sequence acc = acc + A[i][k]*B[k][j]
 * for k = 0, 1, ..., K-1 in that order, so the bits equal the literal loop
 * above. Only independent elements are interleaved (the j loop), and rows are
 * split between threads. B is widened to fp32 once, up front. */

typedef struct {
    int64_t i0, i1, N, K;
    const uint16_t *A;
    int64_t lda;
    const float *Bf; /* K x N, packed */
    uint16_t *C;
    int64_t ldc;
} row_job;

static void *row_worker(void *arg) {
    row_job *jb = (row_job *)arg;
    float *acc = (float *)malloc((size_t)(jb->N > 0 ? jb->N : 1) * sizeof(float));
    if (!acc) return (void *)1;
    for (int64_t i = jb->i0; i < jb->i1; i++) {
        for (int64_t j = 0; j < jb->N; j++) acc[j] = 0.0f;
        for (int64_t k = 0; k < jb->K; k++) {
            float a = oracle_f16_to_f32(jb->A[i * jb->lda + k]);
            const float *brow = jb->Bf + k * jb->N;
            for (int64_t j = 0; j < jb->N; j++) acc[j] = acc[j] + a * brow[j];
        }
        for (int64_t j = 0; j < jb->N; j++) jb->C[i * jb->ldc + j] = oracle_relu_to_f16(acc[j]);
    }
    free(acc);
    return NULL;
}

int oracle_default_threads(void) {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof set, &set) == 0) {
        int n = CPU_COUNT(&set);
        if (n > 0) return n;
    }
    return 1;
}

/* Returns 0 on success, -1 on bad arguments, -2 if memory or threads fail. */
int oracle_gemm_relu_f16(int64_t M, int64_t N, int64_t K,
                         const uint16_t *A, int64_t lda,
                         const uint16_t *B, int64_t ldb,
                         uint16_t *C, int64_t ldc, int threads) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (threads <= 0) threads = oracle_default_threads();
    if (threads > M) threads = (int)M;
    float *Bf = (float *)malloc((size_t)(K * N > 0 ? K * N : 1) * sizeof(float));
    if (!Bf) return -2;
    for (int64_t k = 0; k < K; k++)
        for (int64_t j = 0; j < N; j++) Bf[k * N + j] = oracle_f16_to_f32(B[k * ldb + j]);
    row_job *jobs = (row_job *)calloc((size_t)threads, sizeof(row_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
    int rc = 0;
    if (!jobs || !tids) {
        rc = -2;
    } else {
        int started = 0;
        for (int t = 0; t < threads; t++) {
            jobs[t] = (row_job){M * t / threads, M * (t + 1) / threads, N, K, A, lda, Bf, C, ldc};
            if (pthread_create(&tids[t], NULL, row_worker, &jobs[t]) != 0) {
                rc = -2;
                break;
            }
            started++;
        }
        for (int t = 0; t < started; t++) {
            void *ret = NULL;
            pthread_join(tids[t], &ret);
            if (ret != NULL) rc = -2;
        }
    }
    free(jobs);
    free(tids);
    free(Bf);
    return rc;
}
