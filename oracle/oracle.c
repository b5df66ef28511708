/*
 * CPU oracle for the fp16 NT matrix product, its split-K fp32 form and GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source, header, table or helper with the
 * HIP library, and it never reads a value the GPU produced.
 *
 * What it computes (the plain definition, written out):
 *
 *   GEMM   C[i][j] = round_f16( sum_{k=0}^{K-1} A[i][k] * B[j][k] )
 *          A is M x K, B is N x K, both row-major fp16, C is M x N fp16.
 *          Source: "TileLang FP16 matrix-multiply autotune benchmark" page,
 *          section 1 (the product is C = A B^T with fp16 operands and fp32
 *          accumulation) and section 2 (signature A(M,K), B(N,K), C(M,N) with
 *          transpose_B); the autotune tutorial page's reference() function
 *          (multiply in fp32, cast back to fp16).
 *   SPLITK C32[i][j] = round_f32( same sum ).  Source: the "basic GEMM to
 *          SplitK" page, SplitK section: K is cut into slices, each slice is
 *          multiplied on its own and the slice results are added into a C of
 *          out_dtype float32.  Cutting K regroups one sum, so the oracle does
 *          not cut.
 *   GEMV   y[n] = round_f16( sum_k W[n][k] * x[k] ).  Source: the "TileLang
 *          GEMV optimisation" page, problem statement (GEMV is the (1,k)x(k,n)
 *          degenerate GEMM) and its kernels' signature A(K,), B(N,K), C(N,),
 *          accumulated in float; here x = A, W = B, y = C.
 *   2:4    Structured sparsity of A.  Source: the "TileLang FP16 matmul
 *          autotune benchmark" page, section 6 (further reading): A is
 *          compressed 2:4-style into A_sparse of shape (M, K/2) plus mask
 *          metadata E of shape (M, K/e_factor), and the sparse product is
 *          the GEMM above taken with the A that these two describe.  The page
 *          fixes neither the choice of the two kept entries nor the bit
 *          layout of E; the readings taken here:
 *            - K is cut into groups of 4 consecutive entries; a group keeps
 *              the two entries of largest magnitude, ties going to the lower
 *              index (so a group with at most two nonzeros loses nothing).
 *              Magnitude is compared on the fp16 bit pattern without its
 *              sign, which orders every non-NaN value by |x| and puts NaN
 *              above infinity.
 *            - A_sparse holds the two kept values of group g at positions
 *              2g, 2g+1, lower index first.
 *            - E holds 4 bits per group, i0 | i1 << 2 (i0 < i1 the kept
 *              indices within the group), packed from the least significant
 *              bit up in group order into 16-bit words: group g sits at bits
 *              4 (g % 4) of word g / 4, so E is (M, K/16) for e_dtype int16
 *              (e_factor 16); read as bytes (int8) or 32-bit words (int32) on
 *              a little-endian machine the same memory is the e_factor 8 and
 *              32 forms.
 *          K must be a multiple of 16 (whole metadata words).
 *          SPARSE GEMM C = round_f16( decompress(A_sparse, E) . B^T ).
 *
 * Arithmetic: every input is decoded exactly to double, every sum runs over
 * ascending k starting from +0.0, and the result is rounded once.  A product
 * of two fp16 values has at most 22 significant bits, so each product is
 * exact in double; only the running sum may round (relative 2^-53 per add).
 *
 * Rounding to fp16 is round-to-nearest, ties-to-even, written from the IEEE
 * 754 binary16 definition (1 sign bit, 5 exponent bits with bias 15, 10
 * fraction bits; subnormals step by 2^-24; the largest finite value is 65504,
 * and any magnitude at or above the halfway point 65520 overflows to inf).
 * The pages only show casts and name no rounding mode; round-to-nearest-even
 * is the reading taken.  Rounding to fp32 is the C conversion (float)d, which
 * under the default rounding mode is IEEE round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- binary16 <-> double -------------------------------------------- */

double oracle_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0x1f)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24 */
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

uint16_t oracle_f16_from_double(double v)
{
    if (isnan(v))
        return 0x7e00;                           /* quiet NaN */
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a >= 65520.0)
        return sign | 0x7c00;                    /* overflow to infinity */
    if (a == 0.0)
        return sign;

    /* quantum q of the binade that holds a (2^-24 below the normal range) */
    int ex;
    frexp(a, &ex);                               /* a = m * 2^ex, m in [0.5,1) */
    int e = ex - 1;                              /* floor(log2 a) */
    int qexp = (e < -14 ? -14 : e) - 10;
    double n = ldexp(a, -qexp);                  /* exact: scaling by 2^-qexp */
    double fl = floor(n);
    double r = n - fl;                           /* exact */
    double nr;
    if (r > 0.5)
        nr = fl + 1.0;
    else if (r < 0.5)
        nr = fl;
    else
        nr = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;   /* tie: to even */
    double val = ldexp(nr, qexp);                /* the rounded magnitude */

    if (val < ldexp(1.0, -14))                   /* subnormal (or 0) */
        return sign | (uint16_t)nr;
    frexp(val, &ex);
    e = ex - 1;
    uint16_t frac = (uint16_t)(ldexp(val, 10 - e) - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | frac;
}

float oracle_f32_from_double(double v) { return (float)v; }

/* ---- helpers that only decode inputs --------------------------------- */

static double* decode(const uint16_t* src, int64_t count)
{
    double* d = (double*)malloc((size_t)(count > 0 ? count : 1) * sizeof(double));
    if (!d)
        return NULL;
    for (int64_t t = 0; t < count; ++t)
        d[t] = oracle_f16_to_double(src[t]);
    return d;
}

static double dot(const double* a, const double* b, int K)
{
    double s = 0.0;
    for (int k = 0; k < K; ++k)
        s += a[k] * b[k];
    return s;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the parallel loops that follow (n >= 1); timing only. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---- GEMM, fp16 out: rows [row_begin, row_end) of C ------------------ */
int oracle_gemm_nt_f16_rows(const uint16_t* A, const uint16_t* B, uint16_t* C,
                            int M, int N, int K, int row_begin, int row_end)
{
    if (M < 0 || N < 0 || K < 0 || row_begin < 0 || row_end > M || row_begin > row_end)
        return 1;
    int rows = row_end - row_begin;
    double* a = decode(A + (int64_t)row_begin * K, (int64_t)rows * K);
    double* b = decode(B, (int64_t)N * K);
    if (!a || !b) { free(a); free(b); return 2; }
#pragma omp parallel for schedule(static)
    for (int i = 0; i < rows; ++i)
        for (int j = 0; j < N; ++j)
            C[(int64_t)i * N + j] =
                oracle_f16_from_double(dot(a + (int64_t)i * K, b + (int64_t)j * K, K));
    free(a);
    free(b);
    return 0;
}

int oracle_gemm_nt_f16(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K)
{
    return oracle_gemm_nt_f16_rows(A, B, C, M, N, K, 0, M);
}

/* ---- split-K GEMM, fp32 out ------------------------------------------ */
int oracle_gemm_nt_f32(const uint16_t* A, const uint16_t* B, float* C, int M, int N, int K)
{
    if (M < 0 || N < 0 || K < 0)
        return 1;
    double* a = decode(A, (int64_t)M * K);
    double* b = decode(B, (int64_t)N * K);
    if (!a || !b) { free(a); free(b); return 2; }
#pragma omp parallel for schedule(static)
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < N; ++j)
            C[(int64_t)i * N + j] =
                oracle_f32_from_double(dot(a + (int64_t)i * K, b + (int64_t)j * K, K));
    free(a);
    free(b);
    return 0;
}

/* ---- single entries (i, j) of C, for sampled checks at full size ------- */
/* out16 (fp16 rounding) and out32 (fp32 rounding) may each be NULL. */
int oracle_gemm_nt_entries(const uint16_t* A, const uint16_t* B, int M, int N, int K,
                           const int64_t* ij, int64_t count, uint16_t* out16, float* out32)
{
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return 1;
    for (int64_t t = 0; t < count; ++t)
        if (ij[2 * t] < 0 || ij[2 * t] >= M || ij[2 * t + 1] < 0 || ij[2 * t + 1] >= N)
            return 1;
#pragma omp parallel
    {
        double* a = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
        double* b = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < count; ++t) {
            int64_t i = ij[2 * t], j = ij[2 * t + 1];
            for (int k = 0; k < K; ++k) {
                a[k] = oracle_f16_to_double(A[i * K + k]);
                b[k] = oracle_f16_to_double(B[j * K + k]);
            }
            double s = dot(a, b, K);
            if (out16) out16[t] = oracle_f16_from_double(s);
            if (out32) out32[t] = oracle_f32_from_double(s);
        }
        free(a);
        free(b);
    }
    return 0;
}

/* ---- GEMV, fp16 out --------------------------------------------------- */
int oracle_gemv_f16(const uint16_t* W, const uint16_t* x, uint16_t* y, int N, int K)
{
    if (N < 0 || K < 0)
        return 1;
    double* xd = decode(x, K);
    if (!xd) return 2;
#pragma omp parallel
    {
        double* w = (double*)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
#pragma omp for schedule(static)
        for (int n = 0; n < N; ++n) {
            for (int k = 0; k < K; ++k)
                w[k] = oracle_f16_to_double(W[(int64_t)n * K + k]);
            y[n] = oracle_f16_from_double(dot(w, xd, K));
        }
        free(w);
    }
    free(xd);
    return 0;
}

/* ---- array forms of the two conversions (used by the self-tests) ------ */
void oracle_f16_encode_array(const double* v, uint16_t* out, int64_t n)
{
    for (int64_t t = 0; t < n; ++t)
        out[t] = oracle_f16_from_double(v[t]);
}

void oracle_f16_decode_array(const uint16_t* h, double* out, int64_t n)
{
    for (int64_t t = 0; t < n; ++t)
        out[t] = oracle_f16_to_double(h[t]);
}

/* ---- 2:4 structured sparsity ------------------------------------------ */

/* Sign-free bit pattern: orders fp16 values by magnitude (NaN above inf). */
static unsigned magnitude_key(uint16_t h) { return h & 0x7fffu; }

/* A (M x K) -> A_sparse (M x K/2) and E (M x K/16 16-bit words). */
int oracle_sp24_compress(const uint16_t* A, uint16_t* Asp, uint16_t* E, int M, int K)
{
    if (M < 0 || K < 0 || K % 16 != 0)
        return 1;
    const int groups = K / 4;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < M; ++i) {
        const uint16_t* a = A + (int64_t)i * K;
        uint16_t* v = Asp + (int64_t)i * (K / 2);
        uint16_t* e = E + (int64_t)i * (K / 16);
        for (int w = 0; w < K / 16; ++w)
            e[w] = 0;
        for (int g = 0; g < groups; ++g) {
            const uint16_t* x = a + 4 * g;
            /* largest magnitude, first occurrence */
            int first = 0;
            for (int t = 1; t < 4; ++t)
                if (magnitude_key(x[t]) > magnitude_key(x[first]))
                    first = t;
            /* largest of the other three, first occurrence */
            int second = -1;
            for (int t = 0; t < 4; ++t) {
                if (t == first)
                    continue;
                if (second < 0 || magnitude_key(x[t]) > magnitude_key(x[second]))
                    second = t;
            }
            const int i0 = first < second ? first : second;
            const int i1 = first < second ? second : first;
            v[2 * g] = x[i0];
            v[2 * g + 1] = x[i1];
            e[g / 4] |= (uint16_t)((i0 | (i1 << 2)) << (4 * (g % 4)));
        }
    }
    return 0;
}

/* A_sparse and E -> the dense A they describe (zeros elsewhere).  Returns 3
 * if a group's field does not name two indices in increasing order. */
int oracle_sp24_decompress(const uint16_t* Asp, const uint16_t* E, uint16_t* A, int M, int K)
{
    if (M < 0 || K < 0 || K % 16 != 0)
        return 1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int i = 0; i < M; ++i) {
        const uint16_t* v = Asp + (int64_t)i * (K / 2);
        const uint16_t* e = E + (int64_t)i * (K / 16);
        uint16_t* a = A + (int64_t)i * K;
        for (int k = 0; k < K; ++k)
            a[k] = 0;
        for (int g = 0; g < K / 4; ++g) {
            const int field = (e[g / 4] >> (4 * (g % 4))) & 0xf;
            const int i0 = field & 3, i1 = field >> 2;
            if (i0 >= i1) {
                bad = 1;
                continue;
            }
            a[4 * g + i0] = v[2 * g];
            a[4 * g + i1] = v[2 * g + 1];
        }
    }
    return bad ? 3 : 0;
}

