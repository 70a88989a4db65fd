/*
 * CPU oracle for the fused GEMM + ReLU:  C = ReLU(A @ B).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this code.  The HIP library
 * never includes, links or calls it, and it includes nothing from the HIP
 * side: the two implementations share no code.
 *
 * What it computes follows the GEMM + ReLU example of "Writing
 * High-Performance Kernels in TileLang" (atlascloud.ai, section "Let's write
 * a GEMM", also the Korean edition and the devpress.csdn.net TileLang
 * introduction's matrix-multiply example):
 *   A is (M, K), B is (K, N), C is (M, N), all row-major in one 16-bit dtype;
 *   products are summed into a wider accumulator that starts at zero; every
 *   accumulator element is replaced by max(value, 0); the result is cast to
 *   the dtype of C and stored.
 *
 * The oracle writes that definition out plainly:
 *   1. decode every 16-bit input to its exact real value (fp64 holds every
 *      fp16 and bf16 value exactly, subnormals included);
 *   2. s[i][j] = sum over k = 0 .. K-1, ascending, of a[i][k] * b[k][j], in
 *      fp64 (each product is exact in fp64; only the sums round);
 *   3. r = s if s > 0, else +0.0;
 *   4. C[i][j] = r rounded to the output dtype, IEEE round-to-nearest-even,
 *      overflow to +inf.
 * No blocking, no SIMD, no BLAS.  The only parallelism is independent rows
 * of C handed to OpenMP threads; each element's sum order is fixed.
 *
 * Readings of points the pages leave open (ReLU gives +0.0 for every s <= 0;
 * RNE for the cast; K = 0 gives all +0.0) are stated at the functions that
 * take them.
 *
 * The codec (decode/encode) is written from the IEEE 754 binary16 layout and
 * the bfloat16 layout (the upper half of an IEEE binary32); it uses only
 * frexp/ldexp/rint from libm.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

/* ---------------------------------------------------------------- decode */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1.f) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);              /* subnormal: f * 2^-133 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);   /* (1.f) * 2^(e-127) */
    return sign ? -v : v;
}

/* ---------------------------------------------------------------- encode */

/*
 * Round a finite or infinite double to a 16-bit float with `frac_bits`
 * stored fraction bits, exponent bias `bias` and all-ones exponent `emax_field`
 * reserved for inf/NaN.  Round to nearest, ties to even; overflow to inf.
 *
 * Method: a finite value x != 0 lies in a binade [2^e, 2^(e+1)).  The
 * representable values near x are the multiples of the quantum
 * q = 2^(e - frac_bits), or of the subnormal quantum 2^(1 - bias - frac_bits)
 * once e falls below the smallest normal exponent.  x / q is an exact double
 * (scaling by a power of two); rint() rounds it to the nearest integer with
 * ties to even (the default FE_TONEAREST mode).  An integer that carries into
 * the next binade is still correct: the encoding below absorbs the carry.
 */
static uint16_t encode_rne(double x, int frac_bits, int bias, int emax_field)
{
    uint16_t sign = signbit(x) ? 1 : 0;
    uint16_t sign_bit = (uint16_t)(sign << 15);
    uint16_t inf_bits = (uint16_t)(emax_field << frac_bits);
    if (isnan(x))
        return (uint16_t)(sign_bit | inf_bits | (1u << (frac_bits - 1)));
    double ax = fabs(x);
    if (isinf(ax))
        return (uint16_t)(sign_bit | inf_bits);
    if (ax == 0.0)
        return sign_bit;

    int e2;
    frexp(ax, &e2);             /* ax = m * 2^e2, m in [0.5, 1)  =>  binade e = e2 - 1 */
    int e = e2 - 1;
    int emin = 1 - bias;        /* exponent of the smallest normal */
    if (e < emin)
        e = emin;               /* subnormal range: fixed quantum */
    double n = rint(ldexp(ax, frac_bits - e));   /* ax / 2^(e - frac_bits), rounded RNE */
    /* n is in [0, 2^(frac_bits+1)]; n == 2^(frac_bits+1) means a carry into the next binade. */
    if (n >= ldexp(1.0, frac_bits + 1)) {
        n = ldexp(1.0, frac_bits);
        e += 1;
    }
    uint32_t field;
    uint32_t frac;
    if (n < ldexp(1.0, frac_bits)) {
        /* subnormal (only possible when e == emin); n == 0 is a signed zero */
        field = 0;
        frac = (uint32_t)n;
    } else {
        field = (uint32_t)(e + bias);
        frac = (uint32_t)n - (1u << frac_bits);
    }
    if (field >= (uint32_t)emax_field)
        return (uint16_t)(sign_bit | inf_bits);
    return (uint16_t)(sign_bit | (field << frac_bits) | frac);
}

uint16_t oracle_f64_to_f16(double x) { return encode_rne(x, 10, 15, 31); }
uint16_t oracle_f64_to_bf16(double x) { return encode_rne(x, 7, 127, 255); }

/* Bulk forms for the tests. */
void oracle_decode(const uint16_t* src, double* dst, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = dtype == ORACLE_BF16 ? oracle_bf16_to_f64(src[i]) : oracle_f16_to_f64(src[i]);
}

void oracle_encode(const double* src, uint16_t* dst, int64_t n, int dtype)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = dtype == ORACLE_BF16 ? oracle_f64_to_bf16(src[i]) : oracle_f64_to_f16(src[i]);
}

/* ------------------------------------------------------------ GEMM + ReLU */

/* ReLU on the fp64 sum, then the cast.  s <= 0 (including -0.0) gives +0.0. */
static uint16_t relu_then_cast(double s, int dtype)
{
    double r = s > 0.0 ? s : 0.0;
    return dtype == ORACLE_BF16 ? oracle_f64_to_bf16(r) : oracle_f64_to_f16(r);
}

static int bad_args(const void* A, const void* B, const void* C,
                    int64_t M, int64_t N, int64_t K, int dtype)
{
    if (M < 0 || N < 0 || K < 0) return 1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return 1;
    if (M > 0 && N > 0 && !C) return 1;
    if (M > 0 && K > 0 && !A) return 1;
    if (K > 0 && N > 0 && !B) return 1;
    return 0;
}

/*
 * Rows [row0, row1) of C = ReLU(A @ B).  A is the full (M, K) matrix, B the
 * full (K, N) matrix, C the full (M, N) output; only the selected rows of C
 * are written.  threads <= 0 means "OpenMP default".  Returns 0, or -1 on bad
 * arguments or allocation failure (then C is untouched).
 */
int oracle_gemm_relu_rows(const uint16_t* A, const uint16_t* B, uint16_t* C,
                          int64_t M, int64_t N, int64_t K,
                          int64_t row0, int64_t row1, int dtype, int threads)
{
    if (bad_args(A, B, C, M, N, K, dtype)) return -1;
    if (row0 < 0 || row1 > M || row0 > row1) return -1;
    if (row0 == row1 || N == 0) return 0;

    /* B decoded once to exact fp64 values. */
    double* Bd = NULL;
    if (K > 0) {
        Bd = (double*)malloc((size_t)K * (size_t)N * sizeof(double));
        if (!Bd) return -1;
        oracle_decode(B, Bd, K * N, dtype);
    }
    int failed = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)N * sizeof(double));
        if (!acc) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = row0; i < row1; ++i) {
                for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
                /* k ascending for every j: the textbook i-j-k sum order; the
                   k-outer loop order only changes memory access, not any sum */
                for (int64_t k = 0; k < K; ++k) {
                    uint16_t abits = A[i * K + k];
                    double a = dtype == ORACLE_BF16 ? oracle_bf16_to_f64(abits)
                                                    : oracle_f16_to_f64(abits);
                    const double* brow = Bd + k * N;
                    for (int64_t j = 0; j < N; ++j) acc[j] += a * brow[j];
                }
                for (int64_t j = 0; j < N; ++j) C[i * N + j] = relu_then_cast(acc[j], dtype);
            }
            free(acc);
        }
    }
    free(Bd);
    return failed ? -1 : 0;
}

/* The whole of C = ReLU(A @ B). */
int oracle_gemm_relu(const uint16_t* A, const uint16_t* B, uint16_t* C,
                     int64_t M, int64_t N, int64_t K, int dtype, int threads)
{
    return oracle_gemm_relu_rows(A, B, C, M, N, K, 0, M, dtype, threads);
}

/*
 * Selected elements: out[t] = C[ii[t]][jj[t]] for t < count, each computed as
 * its own k-ascending fp64 dot product.  Used to check outputs of shapes too
 * large for the full oracle.  Returns 0, or -1 on a bad argument or index.
 */
int oracle_gemm_relu_entries(const uint16_t* A, const uint16_t* B,
                             int64_t M, int64_t N, int64_t K,
                             const int64_t* ii, const int64_t* jj, int64_t count,
                             uint16_t* out, int dtype)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    if (dtype != ORACLE_F16 && dtype != ORACLE_BF16) return -1;
    for (int64_t t = 0; t < count; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        int64_t i = ii[t], j = jj[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            uint16_t ab = A[i * K + k], bb = B[k * N + j];
            double a = dtype == ORACLE_BF16 ? oracle_bf16_to_f64(ab) : oracle_f16_to_f64(ab);
            double b = dtype == ORACLE_BF16 ? oracle_bf16_to_f64(bb) : oracle_f16_to_f64(bb);
            s += a * b;
        }
        out[t] = relu_then_cast(s, dtype);
    }
    return 0;
}

/* Number of threads an OpenMP parallel region would use (for reports). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
