/*
 * Oracle for the tiled dense GEMM D = alpha * A * B with optional ReLU.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this code.  It shares no
 * code, header, table or helper with the GPU library and must never be used
 * as a fallback for it.
 *
 * What it computes (Tylo.jl manual, "Walk through GEMM", opening paragraph
 * and section 5 "Apply the epilogue and store by ownership"; cuTile.jl
 * tutorial "Matrix Multiplication", Step 3 "Looping over K"):
 *
 *   S[m,n]   = sum over k < K of a[m,k] * b[k,n]      (fp64, k ascending)
 *   ref[m,n] = relu ? max(alpha * S[m,n], 0) : alpha * S[m,n]
 *   mag[m,n] = sum over k < K of |alpha * a[m,k] * b[k,n]|
 *
 * The scalar epilogue applies alpha first and then clamps at zero (Tylo
 * manual section 5).  K = 0 gives the empty sum, so ref = 0 (the pages are
 * silent on this; the plain reading of an empty sum is taken).
 *
 * Storage (Tylo manual section 2 "Bind runtime global arrays"; coordinates
 * are zero-based): a[m,k] lives at element m*lda + k of A (K-contiguous),
 * b[k,n] at element k + n*ldb of B (K-contiguous).  The result is written to
 * ref[(n - n0)*ldr + m], i.e. M-contiguous like the product's own output.
 *
 * Element decoding is written here from the format definitions:
 *   bf16: the 16 stored bits are the upper half of an IEEE binary32;
 *   fp16: IEEE binary16 (1 sign, 5 exponent bits with bias 15, 10 fraction
 *         bits), subnormals decoded exactly as fraction * 2^-24;
 *   fp32: IEEE binary32 as stored.
 *   e4m3: 8-bit float, 1 sign, 4 exponent bits with bias 7, 3 fraction
 *         bits; exponent 0 holds zero and subnormals (fraction * 2^-9);
 *         exponent 15 with fraction 7 is NaN, every other code is finite
 *         (largest 448); there is no infinity;
 *   e5m2: 8-bit float, 1 sign, 5 exponent bits with bias 15, 2 fraction
 *         bits; subnormals fraction * 2^-16; exponent 31 is infinity
 *         (fraction 0) or NaN, as in the IEEE formats.
 *   e2m1: 4-bit float (the MX FP4 element), 1 sign, 2 exponent bits with
 *         bias 1, 1 fraction bit; exponent 0 holds zero and the subnormal
 *         0.5 (fraction * 2^-1); every code is finite (largest 6);
 *   e2m3: 6-bit float (MX FP6, E2M3), 1 sign, 2 exponent bits with bias 1,
 *         3 fraction bits; subnormals fraction * 2^-3; all finite (largest
 *         7.5);
 *   e3m2: 6-bit float (MX FP6, E3M2), 1 sign, 3 exponent bits with bias 3,
 *         2 fraction bits; subnormals fraction * 2^-4; all finite (largest
 *         28).
 * The pages name FP4 among the block-scaled matmul formats without defining
 * it; the plain reading is the OCP microscaling (MX) element formats above.
 * Every decoded value is exactly representable in fp64.
 *
 * Packing of the 4- and 6-bit formats: element i of a stored array occupies
 * bits [w*i, w*i + w) of the array read as one little-endian bit string (bit
 * j of byte x is bit 8x + j), w = 4 or 6: two fp4 elements per byte, low
 * nibble first, and four fp6 elements in every three bytes.  Element indices
 * (m*lda + k, k + n*ldb) count elements, not bytes.
 *
 * Block scales (8-, 6- and 4-bit operands; the pages name block-scaled 8-bit
 * and 4-bit matmuls but do not define them, so the plain reading of the MX
 * formats is taken): an optional unsigned 8-bit exponent per 32 consecutive k of every
 * A row and every B column, value 2^(e - 127), e = 255 meaning NaN.  With
 * scales, a[m,k] stands for decode(a[m,k]) * 2^(sa[m, k/32] - 127), and b
 * likewise with sb[n, k/32]; the scale of A row m for k-block j is byte
 * m*lds_a + j, that of B column n is byte n*lds_b + j.
 *
 * Built with plain -O2 (no fast-math), so the k order of each sum is kept.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 1, ORACLE_F16 = 2, ORACLE_F32 = 3, ORACLE_E4M3 = 4, ORACLE_E5M2 = 5,
       ORACLE_E2M1 = 6, ORACLE_E2M3 = 7, ORACLE_E3M2 = 8 };

double oracle_decode_bf16(uint16_t bits) {
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

double oracle_decode_f16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 31;
    int frac = bits & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);            /* zero and subnormals */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

double oracle_decode_f32(uint32_t bits) {
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

double oracle_decode_e4m3(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int expo = (bits >> 3) & 15;
    int frac = bits & 7;
    double v;
    if (expo == 15 && frac == 7)
        v = NAN;
    else if (expo == 0)
        v = ldexp((double)frac, -9);              /* zero and subnormals */
    else
        v = ldexp((double)(8 + frac), expo - 10); /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

double oracle_decode_e5m2(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int expo = (bits >> 2) & 31;
    int frac = bits & 3;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -16);             /* zero and subnormals */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(4 + frac), expo - 17); /* (1 + f/4) * 2^(e-15) */
    return sign ? -v : v;
}

double oracle_decode_e2m1(uint8_t bits) {
    int sign = (bits >> 3) & 1;
    int expo = (bits >> 1) & 3;
    int frac = bits & 1;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -1);              /* zero and the subnormal 0.5 */
    else
        v = ldexp((double)(2 + frac), expo - 2);  /* (1 + f/2) * 2^(e-1) */
    return sign ? -v : v;
}

double oracle_decode_e2m3(uint8_t bits) {
    int sign = (bits >> 5) & 1;
    int expo = (bits >> 3) & 3;
    int frac = bits & 7;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -3);              /* zero and subnormals */
    else
        v = ldexp((double)(8 + frac), expo - 4);  /* (1 + f/8) * 2^(e-1) */
    return sign ? -v : v;
}

double oracle_decode_e3m2(uint8_t bits) {
    int sign = (bits >> 5) & 1;
    int expo = (bits >> 2) & 7;
    int frac = bits & 3;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -4);              /* zero and subnormals */
    else
        v = ldexp((double)(4 + frac), expo - 5);  /* (1 + f/4) * 2^(e-3) */
    return sign ? -v : v;
}

/* The w-bit code of element idx of a packed array (w = 4 or 6): bits
 * [w*idx, w*idx + w) of the little-endian bit string.  Only the bytes that
 * hold those bits are read. */
static uint8_t packed_code(const uint8_t* base, int w, int64_t idx) {
    const int64_t bit = (int64_t)w * idx;
    const int64_t byte = bit >> 3;
    const int sh = (int)(bit & 7);
    unsigned v = base[byte] >> sh;
    if (sh + w > 8) v |= (unsigned)base[byte + 1] << (8 - sh);
    return (uint8_t)(v & ((1u << w) - 1u));
}

/* Block scale: 2^(e - 127), e = 255 is NaN. */
double oracle_decode_e8m0(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* Bits per stored element (0: unknown dtype). */
static int elem_bits(int dtype) {
    switch (dtype) {
        case ORACLE_F32: return 32;
        case ORACLE_BF16:
        case ORACLE_F16: return 16;
        case ORACLE_E4M3:
        case ORACLE_E5M2: return 8;
        case ORACLE_E2M3:
        case ORACLE_E3M2: return 6;
        case ORACLE_E2M1: return 4;
        default: return 0;
    }
}

static double decode_at(const void* base, int dtype, int64_t idx) {
    switch (dtype) {
        case ORACLE_BF16: return oracle_decode_bf16(((const uint16_t*)base)[idx]);
        case ORACLE_F16: return oracle_decode_f16(((const uint16_t*)base)[idx]);
        case ORACLE_E4M3: return oracle_decode_e4m3(((const uint8_t*)base)[idx]);
        case ORACLE_E5M2: return oracle_decode_e5m2(((const uint8_t*)base)[idx]);
        case ORACLE_E2M1: return oracle_decode_e2m1(packed_code((const uint8_t*)base, 4, idx));
        case ORACLE_E2M3: return oracle_decode_e2m3(packed_code((const uint8_t*)base, 6, idx));
        case ORACLE_E3M2: return oracle_decode_e3m2(packed_code((const uint8_t*)base, 6, idx));
        default: return oracle_decode_f32(((const uint32_t*)base)[idx]);
    }
}

/* Element k of a row or column stored at base + rowoff, with its block scale
 * (scales NULL: no scale). */
static double scaled_at(const void* base, int dtype, int64_t rowoff, int64_t k, const uint8_t* scales,
                        int64_t scale_off) {
    double v = decode_at(base, dtype, rowoff + k);
    if (scales) v *= oracle_decode_e8m0(scales[scale_off + k / 32]);
    return v;
}

/* Decode `count` stored elements into fp64 (used by tests of the decoders). */
int oracle_decode(const void* src, int dtype, int64_t count, double* dst) {
    if (!elem_bits(dtype)) return -5;
    for (int64_t i = 0; i < count; ++i) dst[i] = decode_at(src, dtype, i);
    return 0;
}

/*
 * Round x to the nearest value of the 16-bit format `dtype` (ties to the even
 * significand) and return its bits; used to predict low-precision outputs
 * (cuTile.jl tutorial "Matrix Multiplication", Step 4: the fp32 accumulator is
 * converted on the way out).  Formats, from their definitions:
 *   bf16: 8 significant bits, normal exponents -126..127 (bias 127),
 *         subnormal spacing 2^-133;
 *   fp16: 11 significant bits, normal exponents -14..15 (bias 15),
 *         subnormal spacing 2^-24, largest finite 65504.
 * A rounded magnitude above the largest finite value becomes infinity; NaN
 * becomes the quiet NaN with the input's sign.  The rounding works on the
 * exact fp64 value (scaling by powers of two is exact), so there is no double
 * rounding.
 */
static uint16_t encode16(double x, int p, int emin, int emax, int mant_bits) {
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    const uint16_t exp_all = (uint16_t)(((1u << (15 - mant_bits)) - 1u) << mant_bits);
    if (isnan(x)) return (uint16_t)(sign | exp_all | (1u << (mant_bits - 1)));
    const double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | exp_all);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                      /* a = f * 2^e, f in [0.5, 1) */
    int E = e - 1;                     /* floor(log2 a) */
    if (E < emin) E = emin;            /* subnormal range: fixed spacing */
    const double ulp = ldexp(1.0, E - (p - 1));
    const double v = nearbyint(a / ulp) * ulp;  /* default mode: ties to even */
    const double maxf = ldexp(2.0 - ldexp(1.0, -(p - 1)), emax);
    if (v > maxf) return (uint16_t)(sign | exp_all);
    int ev;
    frexp(v, &ev);
    const int Ev = ev - 1;
    if (v == 0.0 || Ev < emin)         /* subnormal (or rounded to zero) */
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, emin - (p - 1))));
    const int bias = emax;
    const uint16_t frac = (uint16_t)((v / ldexp(1.0, Ev) - 1.0) * (double)(1u << mant_bits));
    return (uint16_t)(sign | (uint16_t)((Ev + bias) << mant_bits) | frac);
}

/* Encode `count` fp64 values to bf16 or fp16 bits (round to nearest even). */
int oracle_encode(const double* src, int dtype, int64_t count, uint16_t* dst) {
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F16) return -5;
    for (int64_t i = 0; i < count; ++i)
        dst[i] = dtype == ORACLE_BF16 ? encode16(src[i], 8, -126, 127, 7) : encode16(src[i], 11, -14, 15, 10);
    return 0;
}

/* One output element, straight from the definition. */
static void one_entry(int64_t m, int64_t n, int64_t K, double alpha, int relu,
                      const double* arow, const double* bcol, double* out, double* mag) {
    double s = 0.0, t = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = arow[k] * bcol[k];
        s += p;
        t += fabs(p);
    }
    (void)m; (void)n;
    double r = alpha * s;
    if (relu && r < 0.0) r = 0.0;
    *out = r;
    *mag = fabs(alpha) * t;
}

typedef struct {
    int64_t M, N, K, lda, ldb, n0, n1, ldr;
    double alpha;
    int relu, dtype, nthreads, tid;
    const double* a;   /* decoded A, row m at a + m*K (NULL when M*K == 0) */
    const void* B;
    double* ref;
    double* mag;
    /* sampled-entry mode */
    int64_t count;
    const int64_t* ms;
    const int64_t* ns;
    const void* A;
    const uint8_t* sa;  /* block scales (NULL: none) */
    const uint8_t* sb;
    int64_t lds_a, lds_b;
} job_t;

static void* full_worker(void* arg) {
    job_t* j = (job_t*)arg;
    double* bcol = (double*)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
    if (!bcol) return (void*)1;
    /* columns n0 + tid, n0 + tid + nthreads, ...: loop order n -> m -> k */
    for (int64_t n = j->n0 + j->tid; n < j->n1; n += j->nthreads) {
        for (int64_t k = 0; k < j->K; ++k) bcol[k] = scaled_at(j->B, j->dtype, n * j->ldb, k, j->sb, n * j->lds_b);
        for (int64_t m = 0; m < j->M; ++m) {
            int64_t o = (n - j->n0) * j->ldr + m;
            one_entry(m, n, j->K, j->alpha, j->relu, j->a + m * j->K, bcol, &j->ref[o], &j->mag[o]);
        }
    }
    free(bcol);
    return NULL;
}

static void* entry_worker(void* arg) {
    job_t* j = (job_t*)arg;
    size_t kk = (size_t)(j->K > 0 ? j->K : 1);
    double* arow = (double*)malloc(sizeof(double) * kk);
    double* bcol = (double*)malloc(sizeof(double) * kk);
    if (!arow || !bcol) { free(arow); free(bcol); return (void*)1; }
    for (int64_t i = j->tid; i < j->count; i += j->nthreads) {
        int64_t m = j->ms[i], n = j->ns[i];
        for (int64_t k = 0; k < j->K; ++k) {
            arow[k] = scaled_at(j->A, j->dtype, m * j->lda, k, j->sa, m * j->lds_a);
            bcol[k] = scaled_at(j->B, j->dtype, n * j->ldb, k, j->sb, n * j->lds_b);
        }
        one_entry(m, n, j->K, j->alpha, j->relu, arow, bcol, &j->ref[i], &j->mag[i]);
    }
    free(arow);
    free(bcol);
    return NULL;
}

static int check_args(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                      const void* B, int64_t ldb, int dtype) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (lda < (K > 1 ? K : 1) || ldb < (K > 1 ? K : 1)) return -2;
    const int w = elem_bits(dtype);
    if (!w) return -5;
    /* packed formats: every row and column starts on a byte boundary */
    if (w < 8 && (((lda * w) & 7) || ((ldb * w) & 7))) return -2;
    if (K > 0 && ((M > 0 && !A) || (N > 0 && !B))) return -3;
    return 0;
}

/* Scales are for the 8-, 6- and 4-bit formats only; each row holds
 * ceil(K/32) of them. */
static int check_scales(int64_t K, int dtype, const uint8_t* sa, int64_t lds_a, const uint8_t* sb,
                        int64_t lds_b) {
    if (!sa && !sb) return 0;
    if (elem_bits(dtype) > 8) return -5;
    const int64_t blocks = (K + 31) / 32;
    if ((sa && lds_a < blocks) || (sb && lds_b < blocks)) return -2;
    return 0;
}

static int run_threads(job_t* proto, int nthreads, void* (*fn)(void*)) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    job_t jobs[256];
    pthread_t th[256];
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].nthreads = nthreads;
        jobs[t].tid = t;
    }
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, fn, &jobs[t]) != 0) { rc = -9; break; }
        ++started;
    }
    for (int t = 0; t < started; ++t) {
        void* ret = NULL;
        pthread_join(th[t], &ret);
        if (ret) rc = -9;
    }
    return rc;
}

/*
 * Full columns n in [n0, n1) of the result, every m < M.
 * ref and mag are (n1 - n0) columns of ldr >= M doubles each.
 * Returns 0, or a negative code for bad arguments / allocation failure.
 */
int oracle_gemm_scaled(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                       const void* A, int64_t lda, const void* B, int64_t ldb, int dtype,
                       const uint8_t* sa, int64_t lds_a, const uint8_t* sb, int64_t lds_b,
                       int64_t n0, int64_t n1, double* ref, double* mag, int64_t ldr, int nthreads) {
    int rc = check_args(M, N, K, A, lda, B, ldb, dtype);
    if (!rc) rc = check_scales(K, dtype, sa, lds_a, sb, lds_b);
    if (rc) return rc;
    if (n0 < 0 || n1 > N || n0 > n1 || ldr < M) return -2;
    if (M == 0 || n1 == n0) return 0;
    double* a = NULL;
    if (K > 0) {
        a = (double*)malloc(sizeof(double) * (size_t)M * (size_t)K);
        if (!a) return -9;
        for (int64_t m = 0; m < M; ++m)
            for (int64_t k = 0; k < K; ++k) a[m * K + k] = scaled_at(A, dtype, m * lda, k, sa, m * lds_a);
    }
    job_t p;
    memset(&p, 0, sizeof p);
    p.M = M; p.N = N; p.K = K; p.lda = lda; p.ldb = ldb; p.n0 = n0; p.n1 = n1; p.ldr = ldr;
    p.alpha = (double)alpha; p.relu = relu; p.dtype = dtype;
    p.a = a; p.B = B; p.ref = ref; p.mag = mag;
    p.sb = sb; p.lds_b = lds_b;
    int64_t cols = n1 - n0;
    rc = run_threads(&p, nthreads > cols ? (int)cols : nthreads, full_worker);
    free(a);
    return rc;
}

int oracle_gemm(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                const void* A, int64_t lda, const void* B, int64_t ldb, int dtype,
                int64_t n0, int64_t n1, double* ref, double* mag, int64_t ldr, int nthreads) {
    return oracle_gemm_scaled(M, N, K, alpha, relu, A, lda, B, ldb, dtype, NULL, 0, NULL, 0, n0, n1, ref, mag, ldr,
                              nthreads);
}

/* Sampled entries (ms[i], ns[i]), i < count, into ref[i] and mag[i]. */
int oracle_gemm_entries_scaled(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                               const void* A, int64_t lda, const void* B, int64_t ldb, int dtype,
                               const uint8_t* sa, int64_t lds_a, const uint8_t* sb, int64_t lds_b,
                               int64_t count, const int64_t* ms, const int64_t* ns,
                               double* ref, double* mag, int nthreads) {
    int rc = check_args(M, N, K, A, lda, B, ldb, dtype);
    if (!rc) rc = check_scales(K, dtype, sa, lds_a, sb, lds_b);
    if (rc) return rc;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
    if (count == 0) return 0;
    job_t p;
    memset(&p, 0, sizeof p);
    p.M = M; p.N = N; p.K = K; p.lda = lda; p.ldb = ldb;
    p.alpha = (double)alpha; p.relu = relu; p.dtype = dtype;
    p.A = A; p.B = B; p.ref = ref; p.mag = mag;
    p.count = count; p.ms = ms; p.ns = ns;
    p.sa = sa; p.lds_a = lds_a; p.sb = sb; p.lds_b = lds_b;
    return run_threads(&p, nthreads > count ? (int)count : nthreads, entry_worker);
}

int oracle_gemm_entries(int64_t M, int64_t N, int64_t K, float alpha, int relu,
                        const void* A, int64_t lda, const void* B, int64_t ldb, int dtype,
                        int64_t count, const int64_t* ms, const int64_t* ns,
                        double* ref, double* mag, int nthreads) {
    return oracle_gemm_entries_scaled(M, N, K, alpha, relu, A, lda, B, ldb, dtype, NULL, 0, NULL, 0, count, ms, ns,
                                      ref, mag, nthreads);
}
