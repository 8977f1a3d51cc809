/*
 * Dense-GEMM oracle: a plain, slow, obviously correct CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library: every conversion and every
 * formula below is written out here from its definition.
 *
 * What it computes, and where each definition comes from:
 *
 *  - GEMM.  C_ij = sum_k A_ik B_kj, 2MNK FLOPs ("Matrix Multiplication: The
 *    Operation Behind Modern AI", section "The operation everything is made
 *    of").  Inputs are decoded exactly to binary64 from their raw bits and the
 *    sum is accumulated in binary64 in ascending k, i-k-j loop order, so the
 *    summation order of every element is fixed and threads cannot change it.
 *    B_kj is B[k*ldb + j] for a K x N row-major B, or B[j*ldb + k] for an
 *    N x K weight ("02 · 8m/8m② — Tiled wmma f16 prefill GEMM", §3.2: the
 *    prefill product is C[nt,od] = A[nt,id] · B[od,id]^T).
 *    The same loop also accumulates U_ij = sum_k |A_ik||B_kj|, the scale of
 *    the elementwise error bound.
 *
 *  - Epilogue.  t = alpha*S + beta*C_old (C_old not read when beta == 0),
 *    then t += bias_j (one value per output column), then optionally the
 *    tanh form of GELU, 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3)))
 *    (Hendrycks & Gimpel, "Gaussian Error Linear Units").  All in binary64.
 *
 *  - q4 dequantisation ("02 · 8m/8m② — Tiled wmma f16 prefill GEMM", §2.3
 *    and the q4_0 dequant kernel of §3.2).  A row of `cols` weights is
 *    cols/32 blocks of 18 bytes: a little-endian binary16 scale d, then 16
 *    code bytes.  Byte i holds element i in its low nibble and element i+16 in
 *    its high nibble; a code q in 0..15 stands for d*(q-8).  The product is
 *    exact in binary64 and is rounded once, to nearest-even, to binary16.
 *
 *  - K-quant dequantisation (same page, §3.2: one dequant kernel per weight
 *    type; float arithmetic, then one conversion to binary16).  256 weights
 *    per super-block:
 *      q6_K, 210 bytes (or the same 210 bytes padded to a 224-byte stride,
 *        the two layouts the page's q6_K kernel takes through its block
 *        stride): ql[128] low 4 bits, qh[64] high 2 bits, 16 int8
 *        sub-block scales sc[16] at byte 192, binary16 d at byte 208; weight
 *        = d * sc * (q - 32) with q = low | high << 4.  The page names the
 *        interleaved addressing (half, quarter tt, 16-group) without printing
 *        it; the reading taken, which matches every field it does show (low
 *        nibble for tt < 2, high nibble otherwise, high bits qh >> 2 tt):
 *        weight e = 128 h + 32 tt + l (l < 32) takes ql[64 h + 32 (tt & 1) +
 *        l], qh[32 h + l] and sc[8 h + 2 tt + l / 16].  d * sc * (q - 32)
 *        has at most 24 significant bits, so it is exact and rounds once.
 *      q4_K, 144 bytes (the pages name the type and its dmin but print no
 *        layout; the reading taken is the K-quant layout): binary16 d and
 *        dmin, 12 bytes packing a 6-bit scale sc_j and 6-bit min m_j for 8
 *        sub-blocks of 32, then qs[128]; sub-blocks 2p and 2p + 1 take the
 *        low and high nibbles of qs[32 p .. 32 p + 31]; weight =
 *        RNE16(RNE32(d sc_j q - dmin m_j)): d sc_j q and dmin m_j are exact
 *        in binary32, the difference is rounded to binary32 as the page's
 *        float arithmetic does, then once more to binary16.
 *
 *  - Rounding.  binary64 -> binary16 / bfloat16 / binary32, round to nearest,
 *    ties to even, with gradual underflow and overflow to infinity.
 *
 * Every function here but one is pinned by the CPU test suite against brute
 * force, closed forms and library routines (numpy's float16 cast, exact
 * rational arithmetic).  The exception: oracle_dequant_q4_k is PARITY
 * UNPINNED.  The pages name the q4_K type but print no layout, so its 6-bit
 * scale/min packing and nibble order are a reading from outside them; its
 * golden blocks and the test's packer follow that same reading, and no
 * importable library decodes the format, so a wrong reading of the layout
 * would pass every test.  Its arithmetic (two exact binary32 products, one
 * binary32 difference, one binary16 rounding) is pinned; its layout is not.
 *
 * Built with -O2 -ffp-contract=off and no fast-math, so `acc += a*b` is a
 * rounded multiply followed by a rounded add, as written.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1, ORACLE_F32 = 2 };
enum { ORACLE_EPI_NONE = 0, ORACLE_EPI_BIAS = 1, ORACLE_EPI_BIAS_GELU = 2 };

/* ---------------------------------------------------------------- decoding */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent field 0 is zero/subnormal (f * 2^-24); 31 is inf/NaN. */
double oracle_f16_to_f64(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return s ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t h) {
    int s = (h >> 15) & 1, e = (h >> 7) & 255, f = h & 127;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);
    return s ? -v : v;
}

/* IEEE 754 binary32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits. */
double oracle_f32_to_f64(uint32_t w) {
    int s = (w >> 31) & 1, e = (w >> 23) & 255;
    uint32_t f = w & 0x7fffffu;
    double v;
    if (e == 0)
        v = ldexp((double)f, -149);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(0x800000u + f), e - 150);
    return s ? -v : v;
}

/* ---------------------------------------------------------------- encoding */

/* Round |x| to a format with `p` significand bits (hidden bit included),
 * minimum normal exponent emin and maximum exponent emax; returns the
 * unsigned encoding.  nearbyint() rounds to nearest, ties to even, in the
 * default rounding mode; ldexp() is exact. */
static uint64_t round_magnitude(double a, int p, int emin, int emax, int frac_bits) {
    uint64_t inf_code = ((uint64_t)(emax - emin + 2) << frac_bits);
    if (isinf(a)) return inf_code;
    if (a == 0.0) return 0;
    int e2;
    (void)frexp(a, &e2);
    int E = e2 - 1; /* a = 1.f * 2^E */
    if (E < emin) {
        /* gradual underflow: a multiple of 2^(emin - (p-1)) */
        double k = nearbyint(ldexp(a, (p - 1) - emin));
        return (uint64_t)k; /* k == 2^(p-1) lands exactly on the smallest normal */
    }
    double k = nearbyint(ldexp(a, (p - 1) - E)); /* in [2^(p-1), 2^p] */
    if (k == ldexp(1.0, p)) {
        k = ldexp(1.0, p - 1);
        E += 1;
    }
    if (E > emax) return inf_code;
    return ((uint64_t)(E - emin + 1) << frac_bits) | ((uint64_t)k - ((uint64_t)1 << (p - 1)));
}

uint16_t oracle_f64_to_f16(double x) {
    if (isnan(x)) return 0x7e00;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    return (uint16_t)(s | round_magnitude(fabs(x), 11, -14, 15, 10));
}

uint16_t oracle_f64_to_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    uint16_t s = signbit(x) ? 0x8000 : 0;
    return (uint16_t)(s | round_magnitude(fabs(x), 8, -126, 127, 7));
}

uint32_t oracle_f64_to_f32(double x) {
    if (isnan(x)) return 0x7fc00000u;
    uint32_t s = signbit(x) ? 0x80000000u : 0;
    return (uint32_t)(s | round_magnitude(fabs(x), 24, -126, 127, 23));
}

/* Vector forms used by the Python wrapper. */
void oracle_decode(int type, int64_t n, const void* src, double* dst) {
    for (int64_t i = 0; i < n; ++i) {
        if (type == ORACLE_F16)
            dst[i] = oracle_f16_to_f64(((const uint16_t*)src)[i]);
        else if (type == ORACLE_BF16)
            dst[i] = oracle_bf16_to_f64(((const uint16_t*)src)[i]);
        else
            dst[i] = oracle_f32_to_f64(((const uint32_t*)src)[i]);
    }
}

void oracle_encode(int type, int64_t n, const double* src, void* dst) {
    for (int64_t i = 0; i < n; ++i) {
        if (type == ORACLE_F16)
            ((uint16_t*)dst)[i] = oracle_f64_to_f16(src[i]);
        else if (type == ORACLE_BF16)
            ((uint16_t*)dst)[i] = oracle_f64_to_bf16(src[i]);
        else
            ((uint32_t*)dst)[i] = oracle_f64_to_f32(src[i]);
    }
}

static double decode_one(int type, const void* base, int64_t idx) {
    if (type == ORACLE_F16) return oracle_f16_to_f64(((const uint16_t*)base)[idx]);
    if (type == ORACLE_BF16) return oracle_bf16_to_f64(((const uint16_t*)base)[idx]);
    return oracle_f32_to_f64(((const uint32_t*)base)[idx]);
}

/* ---------------------------------------------------------------- epilogue */

double oracle_gelu_tanh(double t) {
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * t * (1.0 + tanh(c * (t + 0.044715 * t * t * t)));
}

/* ---------------------------------------------------------------- GEMM */

typedef struct {
    int64_t M, N, K;
    double alpha, beta;
    int a_type;
    const void* A;
    int64_t lda;
    const double* Bd; /* B decoded to binary64, K x N row-major */
    const double* Cin;
    int64_t ldcin;
    int epi;
    const double* bias;
    double* out;
    double* U;
    int64_t row0, row1;
} gemm_job;

static void* gemm_rows(void* arg) {
    gemm_job* j = (gemm_job*)arg;
    const int64_t N = j->N, K = j->K;
    double* acc = (double*)malloc(sizeof(double) * (size_t)(N ? N : 1));
    double* aacc = (double*)malloc(sizeof(double) * (size_t)(N ? N : 1));
    for (int64_t i = j->row0; i < j->row1; ++i) {
        for (int64_t c = 0; c < N; ++c) {
            acc[c] = 0.0;
            aacc[c] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
            const double a = decode_one(j->a_type, j->A, i * j->lda + k);
            const double aa = fabs(a);
            const double* brow = j->Bd + k * N;
            for (int64_t c = 0; c < N; ++c) {
                acc[c] += a * brow[c];
                aacc[c] += aa * fabs(brow[c]);
            }
        }
        for (int64_t c = 0; c < N; ++c) {
            double t = j->alpha * acc[c];
            if (j->beta != 0.0) t += j->beta * j->Cin[i * j->ldcin + c];
            if (j->epi == ORACLE_EPI_BIAS || j->epi == ORACLE_EPI_BIAS_GELU) t += j->bias[c];
            if (j->epi == ORACLE_EPI_BIAS_GELU) t = oracle_gelu_tanh(t);
            j->out[i * N + c] = t;
            if (j->U) j->U[i * N + c] = aacc[c];
        }
    }
    free(acc);
    free(aacc);
    return NULL;
}

/*
 * out[M x N] = epilogue(alpha * A B + beta * Cin), all binary64.
 *   A: M x K row-major, raw bits of a_type, leading dimension lda.
 *   B: K x N row-major (trans_b = 0, ldb >= N) or N x K (trans_b = 1,
 *      ldb >= K), raw bits of b_type.
 *   Cin: binary64 values of the old C, M x N with leading dimension ldcin;
 *      only read when beta != 0.
 *   bias: binary64, N values; only read for the bias epilogues.
 *   U (optional): sum_k |A_ik||B_kj|.
 *   nthreads: rows are split in contiguous ranges; every element's value is
 *      independent of the split.
 * Returns 0, or -1 on an allocation failure.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K, double alpha, int a_type, const void* A,
                int64_t lda, int b_type, const void* B, int64_t ldb, int trans_b, double beta,
                const double* Cin, int64_t ldcin, int epi, const double* bias, double* out,
                double* U, int nthreads) {
    if (M <= 0 || N <= 0) return 0;
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K * N : 1));
    if (!Bd) return -1;
    for (int64_t k = 0; k < K; ++k)
        for (int64_t c = 0; c < N; ++c)
            Bd[k * N + c] = decode_one(b_type, B, trans_b ? c * ldb + k : k * ldb + c);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > M) nthreads = (int)M;
    gemm_job* jobs = (gemm_job*)calloc((size_t)nthreads, sizeof(gemm_job));
    pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tids) {
        free(Bd);
        free(jobs);
        free(tids);
        return -1;
    }
    for (int t = 0; t < nthreads; ++t) {
        gemm_job* j = &jobs[t];
        j->M = M; j->N = N; j->K = K;
        j->alpha = alpha; j->beta = beta;
        j->a_type = a_type; j->A = A; j->lda = lda;
        j->Bd = Bd; j->Cin = Cin; j->ldcin = ldcin;
        j->epi = epi; j->bias = bias; j->out = out; j->U = U;
        j->row0 = M * t / nthreads;
        j->row1 = M * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&tids[t], NULL, gemm_rows, &jobs[t]);
    gemm_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(tids[t], NULL);
    free(jobs);
    free(tids);
    free(Bd);
    return 0;
}

/* ---------------------------------------------------------------- q4 dequant */

/*
 * out (binary16 bits, rows x cols, leading dimension ldo) from `rows` rows of
 * cols/32 blocks of 18 bytes each.  Returns -1 if cols is not a multiple of 32.
 */
int oracle_dequant_q4(const uint8_t* q, int64_t rows, int64_t cols, uint16_t* out, int64_t ldo) {
    if (cols % 32 != 0) return -1;
    const int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = q + 18 * (r * nb + b);
            const double d = oracle_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
            for (int i = 0; i < 16; ++i) {
                const int lo = blk[2 + i] & 15, hi = blk[2 + i] >> 4;
                out[r * ldo + 32 * b + i] = oracle_f64_to_f16(d * (double)(lo - 8));
                out[r * ldo + 32 * b + 16 + i] = oracle_f64_to_f16(d * (double)(hi - 8));
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------- K-quant dequant */

/* q6_K: rows x cols weights (cols % 256 == 0), super-blocks of 210 bytes
 * placed every `stride` bytes (210, or 224 for the padded layout the same
 * page's q6_K kernel also accepts; the bytes past 210 are ignored),
 * row-major by (row, super-block).  Returns -1 for a bad shape or stride. */
int oracle_dequant_q6_k(const uint8_t* q, int64_t rows, int64_t cols, int64_t stride,
                        uint16_t* out, int64_t ldo) {
    if (cols % 256 != 0 || stride < 210) return -1;
    const int64_t nsb = cols / 256;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nsb; ++b) {
            const uint8_t* blk = q + stride * (r * nsb + b);
            const uint8_t* ql = blk;
            const uint8_t* qh = blk + 128;
            const int8_t* sc = (const int8_t*)(blk + 192);
            const double d = oracle_f16_to_f64((uint16_t)(blk[208] | (blk[209] << 8)));
            for (int e = 0; e < 256; ++e) {
                const int h = e / 128, tt = (e % 128) / 32, l = e % 32;
                const int byte = ql[64 * h + 32 * (tt & 1) + l];
                const int low = tt < 2 ? (byte & 15) : (byte >> 4);
                const int high = (qh[32 * h + l] >> (2 * tt)) & 3;
                const int code = (low | (high << 4)) - 32;
                const double v = d * (double)sc[8 * h + 2 * tt + l / 16] * (double)code;
                out[r * ldo + 256 * b + e] = oracle_f64_to_f16(v);
            }
        }
    }
    return 0;
}

/* The 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes:
 * sub-blocks 0..3 keep their scale and min in the low 6 bits of bytes j and
 * j + 4; sub-blocks 4..7 keep the low 4 bits of each in byte j + 4 (scale in
 * the low nibble, min in the high one) and the top 2 bits in the top 2 bits
 * of bytes j - 4 (scale) and j (min). */
static void q4_k_scale_min(const uint8_t* s12, int j, int* sc, int* m) {
    if (j < 4) {
        *sc = s12[j] & 63;
        *m = s12[j + 4] & 63;
    } else {
        *sc = (s12[j + 4] & 15) | ((s12[j - 4] >> 6) << 4);
        *m = (s12[j + 4] >> 4) | ((s12[j] >> 6) << 4);
    }
}

/* q4_K: rows x cols weights (cols % 256 == 0), super-blocks of 144 bytes. */
int oracle_dequant_q4_k(const uint8_t* q, int64_t rows, int64_t cols, uint16_t* out,
                        int64_t ldo) {
    if (cols % 256 != 0) return -1;
    const int64_t nsb = cols / 256;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nsb; ++b) {
            const uint8_t* blk = q + 144 * (r * nsb + b);
            const double d = oracle_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
            const double dmin = oracle_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
            const uint8_t* qs = blk + 16;
            for (int e = 0; e < 256; ++e) {
                const int p = e / 64, w = e % 64;
                const int j = 2 * p + (w >= 32);
                const int byte = qs[32 * p + w % 32];
                const int code = w < 32 ? (byte & 15) : (byte >> 4);
                int sc, m;
                q4_k_scale_min(blk + 4, j, &sc, &m);
                const double t = d * (double)sc * (double)code; /* <= 21 bits: exact */
                const double u = dmin * (double)m;              /* <= 17 bits: exact */
                /* t - u in binary64 is exact when the operands are within 2^29 of
                 * each other; otherwise the smaller is below half a binary32 ulp of
                 * the larger (an exact binary32 value) and both this difference and
                 * the exact one round to the larger in binary32. */
                const double f32 = oracle_f32_to_f64(oracle_f64_to_f32(t - u));
                out[r * ldo + 256 * b + e] = oracle_f64_to_f16(f32);
            }
        }
    }
    return 0;
}
