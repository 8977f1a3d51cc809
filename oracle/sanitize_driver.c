/*
 * Driver for the sanitizer build of the oracle (TEST INFRASTRUCTURE ONLY):
 * compiled together with oracle.c under -fsanitize=address,undefined by
 * tests/test_oracle_sanitize.py and run as a program.  It calls every
 * exported oracle function on exactly sized heap buffers -- empty, one-element,
 * ragged and strided shapes, every input type, both B layouts, every
 * epilogue, more threads than rows, every block format -- so that an
 * out-of-bounds access, a use after free, a leak or undefined behaviour in
 * the oracle stops the run.  A few results are also checked against sums
 * written out here, so the calls cannot be optimised away.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16_to_f64(uint16_t h);
double oracle_bf16_to_f64(uint16_t h);
double oracle_f32_to_f64(uint32_t w);
uint16_t oracle_f64_to_f16(double x);
uint16_t oracle_f64_to_bf16(double x);
uint32_t oracle_f64_to_f32(double x);
void oracle_decode(int type, int64_t n, const void* src, double* dst);
void oracle_encode(int type, int64_t n, const double* src, void* dst);
double oracle_gelu_tanh(double t);
int oracle_gemm(int64_t M, int64_t N, int64_t K, double alpha, int a_type, const void* A,
                int64_t lda, int b_type, const void* B, int64_t ldb, int trans_b, double beta,
                const double* Cin, int64_t ldcin, int epi, const double* bias, double* out,
                double* U, int nthreads);
int oracle_dequant_q4(const uint8_t* q, int64_t rows, int64_t cols, uint16_t* out, int64_t ldo);
int oracle_dequant_q6_k(const uint8_t* q, int64_t rows, int64_t cols, int64_t stride,
                        uint16_t* out, int64_t ldo);
int oracle_dequant_q4_k(const uint8_t* q, int64_t rows, int64_t cols, uint16_t* out,
                        int64_t ldo);

static uint64_t rng = 88172645463325252ull;
static uint32_t next_u32(void) {  /* xorshift64 */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 11);
}

static int failures = 0;
#define CHECK(c)                                                       \
    do {                                                               \
        if (!(c)) {                                                    \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                \
        }                                                              \
    } while (0)

/* small integers in [-4, 4] stored in the given type */
static void* int_matrix(int type, int64_t n, int64_t* vals) {
    size_t es = type == 2 ? 4 : 2;
    unsigned char* p = (unsigned char*)malloc(es * (size_t)(n > 0 ? n : 1));
    double* d = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        vals[i] = (int64_t)(next_u32() % 9) - 4;
        d[i] = (double)vals[i];
    }
    oracle_encode(type, n, d, p);
    free(d);
    return p;
}

static void gemm_case(int type, int64_t M, int64_t N, int64_t K, int trans_b, int epi,
                      int threads, double beta) {
    int64_t* av = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M * K > 0 ? M * K : 1));
    int64_t* bv = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N * K > 0 ? N * K : 1));
    void* A = int_matrix(type, M * K, av);
    void* B = int_matrix(type, N * K, bv);
    double* cin = (double*)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
    double* bias = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* out = (double*)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
    double* U = (double*)malloc(sizeof(double) * (size_t)(M * N > 0 ? M * N : 1));
    for (int64_t i = 0; i < M * N; ++i) cin[i] = (double)((int)(next_u32() % 7) - 3);
    for (int64_t j = 0; j < N; ++j) bias[j] = (double)((int)(next_u32() % 5) - 2);
    CHECK(oracle_gemm(M, N, K, 1.0, type, A, K, type, B, trans_b ? K : N, trans_b, beta,
                      beta != 0.0 ? cin : NULL, N, epi, epi ? bias : NULL, out, U, threads) == 0);
    if (epi != 2) {
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                int64_t s = 0;
                for (int64_t k = 0; k < K; ++k)
                    s += av[i * K + k] * (trans_b ? bv[j * K + k] : bv[k * N + j]);
                double want = (double)s + (beta != 0.0 ? beta * cin[i * N + j] : 0.0) +
                              (epi ? bias[j] : 0.0);
                CHECK(out[i * N + j] == want);
            }
    }
    free(av); free(bv); free(A); free(B); free(cin); free(bias); free(out); free(U);
}

int main(void) {
    /* conversions: every 16-bit pattern both ways, random binary32 patterns */
    for (uint32_t h = 0; h < 65536; ++h) {
        double x = oracle_f16_to_f64((uint16_t)h), y = oracle_bf16_to_f64((uint16_t)h);
        if (!isnan(x)) CHECK(oracle_f64_to_f16(x) == h);
        if (!isnan(y)) CHECK(oracle_f64_to_bf16(y) == h);
    }
    for (int i = 0; i < 100000; ++i) {
        uint32_t w = next_u32() ^ (next_u32() << 21);
        double x = oracle_f32_to_f64(w);
        if (!isnan(x)) CHECK(oracle_f64_to_f32(x) == w);
    }
    for (int i = -50; i <= 50; ++i) (void)oracle_gelu_tanh(i * 0.37);

    /* GEMM: empty, single-element, ragged, strided, threads > rows */
    int shapes[][3] = {{0, 5, 3}, {5, 0, 3}, {3, 4, 0}, {1, 1, 1}, {7, 3, 33}, {33, 70, 17},
                       {2, 9, 64}};
    for (int s = 0; s < 7; ++s)
        for (int type = 0; type < 3; ++type)
            for (int tb = 0; tb < 2; ++tb)
                for (int epi = 0; epi < 3; ++epi)
                    gemm_case(type, shapes[s][0], shapes[s][1], shapes[s][2], tb, epi,
                              1 + (s % 3) * 7, (epi == 1) ? 2.0 : 0.0);

    /* q4 dequant: exact buffers, ragged rows, padded output */
    for (int64_t rows = 1; rows <= 5; rows += 2)
        for (int64_t cols = 32; cols <= 96; cols += 32) {
            size_t nq = (size_t)(rows * (cols / 32) * 18);
            uint8_t* q = (uint8_t*)malloc(nq);
            for (size_t i = 0; i < nq; ++i) q[i] = (uint8_t)next_u32();
            uint16_t* out = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(rows * (cols + 3)));
            CHECK(oracle_dequant_q4(q, rows, cols, out, cols + 3) == 0);
            CHECK(oracle_dequant_q4(q, rows, cols + 1, out, cols + 3) == -1);
            free(q);
            free(out);
        }
    /* K-quant formats: q6_K at both strides, q4_K */
    for (int64_t rows = 1; rows <= 3; ++rows)
        for (int64_t cols = 256; cols <= 512; cols += 256) {
            int64_t nsb = rows * (cols / 256);
            int64_t strides[2] = {210, 224};
            for (int si = 0; si < 2; ++si) {
                uint8_t* q = (uint8_t*)malloc((size_t)(nsb * strides[si]));
                for (int64_t i = 0; i < nsb * strides[si]; ++i) q[i] = (uint8_t)next_u32();
                uint16_t* out = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(rows * cols));
                CHECK(oracle_dequant_q6_k(q, rows, cols, strides[si], out, cols) == 0);
                free(q);
                free(out);
            }
            uint8_t* q = (uint8_t*)malloc((size_t)(nsb * 144));
            for (int64_t i = 0; i < nsb * 144; ++i) q[i] = (uint8_t)next_u32();
            uint16_t* out = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(rows * cols));
            CHECK(oracle_dequant_q4_k(q, rows, cols, out, cols) == 0);
            free(q);
            free(out);
        }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("sanitizer run clean\n");
    return 0;
}
