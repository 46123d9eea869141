/*
 * Sanitizer driver for the CPU oracles (test infrastructure): built together
 * with oracle/oracle.c and oracle/oracle_mx.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer, it calls every exported oracle function on
 * small random problems (random fp16 bit patterns including NaN, infinity and
 * subnormals, padded leading dimensions, one and several threads, the
 * element-wise and literal-loop forms), and on every fp16 pattern and a
 * sample of fp32 patterns for the conversions. It checks that the forms of
 * the fp16 oracle agree bit for bit and exits 0; any out-of-bounds access,
 * leak, overflow or other undefined behaviour is reported by the sanitizers,
 * which then make the process fail.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float f);
uint16_t oracle_relu_to_f16(float acc);
void oracle_f16_to_f32_array(const uint16_t *in, float *out, int64_t n);
void oracle_f32_to_f16_array(const float *in, uint16_t *out, int64_t n);
void oracle_gemm_relu_f16_elems(int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                                int64_t count, const int64_t *ii, const int64_t *jj, uint16_t *out);
void oracle_gemm_relu_f16_ijk(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                              int64_t ldb, uint16_t *C, int64_t ldc);
int oracle_gemm_relu_f16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B,
                         int64_t ldb, uint16_t *C, int64_t ldc, int threads);
int oracle_default_threads(void);
double oracle_mx_decode(int fmt, uint32_t code);
double oracle_mx_scale(uint32_t e);
uint16_t oracle_f64_to_f16(double x);
uint16_t oracle_mx_relu_to_f16(double acc);
int oracle_gemm_relu_mx_elems(int fmt, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *SA, int64_t ldsa,
                              const uint8_t *B, int64_t ldb, const uint8_t *SB, int64_t ldsb, int64_t count,
                              const int64_t *ii, const int64_t *jj, uint16_t *out);
int oracle_gemm_relu_mx(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t *A, int64_t lda, const uint8_t *SA,
                        int64_t ldsa, const uint8_t *B, int64_t ldb, const uint8_t *SB, int64_t ldsb, uint16_t *C,
                        int64_t ldc, int threads);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t rnd(void) { /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 2685821657736338717ull;
}
static int64_t rnd_in(int64_t lo, int64_t hi) { return lo + (int64_t)(rnd() % (uint64_t)(hi - lo + 1)); }

static int fail(const char *what, int64_t a, int64_t b, int64_t c) {
    fprintf(stderr, "oracle_driver: %s (%lld %lld %lld)\n", what, (long long)a, (long long)b, (long long)c);
    return 1;
}

static int fp16_cases(void) {
    float *f = malloc(65536 * sizeof(float));
    uint16_t *h = malloc(65536 * sizeof(uint16_t)), *back = malloc(65536 * sizeof(uint16_t));
    for (int i = 0; i < 65536; i++) h[i] = (uint16_t)i;
    oracle_f16_to_f32_array(h, f, 65536);
    oracle_f32_to_f16_array(f, back, 65536);
    int bad = 0;
    for (int i = 0; i < 65536; i++) {
        const int nan = ((i & 0x7c00) == 0x7c00) && (i & 0x3ff);
        if (!nan && back[i] != h[i]) bad = 1; /* widening then narrowing is the identity on non-NaN */
        (void)oracle_relu_to_f16(f[i]);
    }
    for (int t = 0; t < 1 << 20; t++) {
        uint32_t u = (uint32_t)rnd();
        float x;
        memcpy(&x, &u, sizeof x);
        (void)oracle_f32_to_f16(x);
        (void)oracle_relu_to_f16(x);
    }
    free(f);
    free(h);
    free(back);
    return bad ? fail("fp16 round trip", 0, 0, 0) : 0;
}

static uint16_t rnd_f16(int kind) {
    if (kind == 0) return (uint16_t)rnd();                 /* any pattern: NaN, inf, subnormal */
    int v = (int)rnd_in(-2, 2);                            /* small integers */
    return oracle_f32_to_f16((float)v);
}

static int fp16_gemm_cases(void) {
    for (int t = 0; t < 300; t++) {
        const int64_t M = rnd_in(0, 23), N = rnd_in(0, 29), K = rnd_in(0, 40);
        const int64_t lda = (K > 0 ? K : 1) + rnd_in(0, 5), ldb = (N > 0 ? N : 1) + rnd_in(0, 5);
        const int64_t ldc = (N > 0 ? N : 1) + rnd_in(0, 3);
        const int kind = (int)(t % 2);
        uint16_t *A = malloc((size_t)((M > 0 ? M : 1) * lda) * 2), *B = malloc((size_t)((K > 0 ? K : 1) * ldb) * 2);
        uint16_t *C1 = calloc((size_t)((M > 0 ? M : 1) * ldc), 2), *C2 = calloc((size_t)((M > 0 ? M : 1) * ldc), 2);
        uint16_t *C3 = calloc((size_t)((M > 0 ? M : 1) * ldc), 2);
        for (int64_t i = 0; i < M * lda; i++) A[i] = rnd_f16(kind);
        for (int64_t i = 0; i < K * ldb; i++) B[i] = rnd_f16(kind);
        if (oracle_gemm_relu_f16(M, N, K, A, lda, B, ldb, C1, ldc, 1) != 0) return fail("gemm 1 thread", M, N, K);
        if (oracle_gemm_relu_f16(M, N, K, A, lda, B, ldb, C2, ldc, 3) != 0) return fail("gemm 3 threads", M, N, K);
        oracle_gemm_relu_f16_ijk(M, N, K, A, lda, B, ldb, C3, ldc);
        for (int64_t i = 0; i < M; i++)
            for (int64_t j = 0; j < N; j++) {
                const uint16_t a = C1[i * ldc + j], b = C2[i * ldc + j], c = C3[i * ldc + j];
                if (a != b || a != c) return fail("forms differ", i, j, K);
            }
        if (M > 0 && N > 0) {
            int64_t ii[16], jj[16];
            uint16_t out[16];
            for (int s = 0; s < 16; s++) {
                ii[s] = rnd_in(0, M - 1);
                jj[s] = rnd_in(0, N - 1);
            }
            oracle_gemm_relu_f16_elems(K, A, lda, B, ldb, 16, ii, jj, out);
            for (int s = 0; s < 16; s++)
                if (out[s] != C1[ii[s] * ldc + jj[s]]) return fail("elements differ", ii[s], jj[s], K);
        }
        free(A);
        free(B);
        free(C1);
        free(C2);
        free(C3);
    }
    if (oracle_gemm_relu_f16(-1, 1, 1, NULL, 1, NULL, 1, NULL, 1, 1) != -1) return fail("negative M", 0, 0, 0);
    return oracle_default_threads() >= 1 ? 0 : fail("threads", 0, 0, 0);
}

static int mx_cases(void) {
    for (uint32_t c = 0; c < 256; c++) {
        (void)oracle_mx_decode(1, c);
        (void)oracle_mx_decode(2, c);
        (void)oracle_mx_decode(3, c & 0xf);
        (void)oracle_mx_scale(c);
    }
    for (int t = 0; t < 1 << 16; t++) {
        uint64_t u = rnd();
        double x;
        memcpy(&x, &u, sizeof x);
        (void)oracle_f64_to_f16(x);
        (void)oracle_mx_relu_to_f16(x);
    }
    for (int t = 0; t < 120; t++) {
        const int fmt = 1 + t % 3, per = fmt == 3 ? 2 : 1;
        const int64_t M = rnd_in(0, 9), N = rnd_in(0, 11), K = 32 * rnd_in(0, 4);
        const int64_t lda = (K > 0 ? K : 2) + 2 * rnd_in(0, 8), ldb = (K > 0 ? K : 2) + 2 * rnd_in(0, 8);
        const int64_t kb = K / 32, ldsa = (kb > 0 ? kb : 1) + rnd_in(0, 2), ldsb = (kb > 0 ? kb : 1) + rnd_in(0, 2);
        const int64_t ldc = (N > 0 ? N : 1) + rnd_in(0, 2);
        const size_t abytes = (size_t)((M > 0 ? M : 1) * lda / per), bbytes = (size_t)((N > 0 ? N : 1) * ldb / per);
        uint8_t *A = malloc(abytes), *B = malloc(bbytes);
        uint8_t *SA = malloc((size_t)((M > 0 ? M : 1) * ldsa)), *SB = malloc((size_t)((N > 0 ? N : 1) * ldsb));
        uint16_t *C1 = calloc((size_t)((M > 0 ? M : 1) * ldc), 2), *C2 = calloc((size_t)((M > 0 ? M : 1) * ldc), 2);
        for (size_t i = 0; i < abytes; i++) A[i] = (uint8_t)rnd();
        for (size_t i = 0; i < bbytes; i++) B[i] = (uint8_t)rnd();
        for (int64_t i = 0; i < (M > 0 ? M : 1) * ldsa; i++) SA[i] = (uint8_t)rnd_in(100, 150);
        for (int64_t i = 0; i < (N > 0 ? N : 1) * ldsb; i++) SB[i] = (uint8_t)rnd_in(100, 150);
        if (oracle_gemm_relu_mx(fmt, M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, C1, ldc, 1) != 0)
            return fail("mx gemm", M, N, K);
        if (oracle_gemm_relu_mx(fmt, M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, C2, ldc, 2) != 0)
            return fail("mx gemm 2 threads", M, N, K);
        for (int64_t i = 0; i < M * ldc; i++)
            if (C1[i] != C2[i]) return fail("mx threads differ", i, 0, K);
        if (M > 0 && N > 0) {
            int64_t ii[8], jj[8];
            uint16_t out[8];
            for (int s = 0; s < 8; s++) {
                ii[s] = rnd_in(0, M - 1);
                jj[s] = rnd_in(0, N - 1);
            }
            if (oracle_gemm_relu_mx_elems(fmt, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, 8, ii, jj, out) != 0)
                return fail("mx elems", M, N, K);
            for (int s = 0; s < 8; s++)
                if (out[s] != C1[ii[s] * ldc + jj[s]]) return fail("mx elements differ", ii[s], jj[s], K);
        }
        free(A);
        free(B);
        free(SA);
        free(SB);
        free(C1);
        free(C2);
    }
    if (oracle_gemm_relu_mx(1, 1, 1, 33, NULL, 33, NULL, 1, NULL, 33, NULL, 1, NULL, 1, 1) != -1)
        return fail("mx K not whole blocks", 0, 0, 0);
    return 0;
}

int main(void) {
    if (fp16_cases() || fp16_gemm_cases() || mx_cases()) return 1;
    printf("oracle_driver: ok\n");
    return 0;
}
