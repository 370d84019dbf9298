/*
 * oracle_gemm.c -- plain, slow CPU reference for C = A * B.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or table with the HIP
 * library, and it includes no HIP, torch or kernel header.
 *
 * What it computes (the plain definition of the matrix product):
 *   C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]
 * as written out in "Part 4 -- Pipelining and Occupancy" (gpucourse.com),
 * section 4.3 "Register reuse", both the triple loop with a local accumulator
 * and the outer-product (k-outer) form; the GEMM the "CUDA Kernel Study:
 * Pipelining" README benchmarks in "Example Code" is the same C = A x B.
 * Software pipelining only reorders loads and leaves the arithmetic alone
 * ("pipeline-gpu-kernel", step 5), so the oracle for every pipelined variant
 * is this one definition.
 *
 * Arithmetic:
 *  - int8 inputs: exact products accumulated in int64, then reduced modulo
 *    2^32 into a two's-complement int32.  This is the uint32_t wrap-around
 *    reference that closes section 4.3 of the gpucourse page; for every shape
 *    whose |C| < 2^31 it is simply the exact sum.
 *  - fp16 / bf16 / fp32 inputs: each element is decoded exactly to double
 *    from its bit pattern (IEEE-754 binary16, bfloat16 = the upper half of a
 *    binary32, binary32), products are formed and summed in double, in
 *    increasing k, one term at a time.  The result is returned in double;
 *    callers round it as they need.
 *
 * Layouts (element (r, c) of an R x Cc matrix with leading dimension ld):
 *   A is row-major M x K:           A(i,k) = A[i*lda + k]
 *   layout 0 ("RR"): B row-major K x N:  B(k,j) = B[k*ldb + j]
 *   layout 1 ("RC"): B column-major:     B(k,j) = B[j*ldb + k]
 *   C is row-major M x N:           C(i,j) = C[i*ldc + j]
 *
 * Loop order: layout RR uses the k-outer outer-product form restricted to one
 * row of C (acc[j] += a_ik * B(k,j)), layout RC the inner-product form
 * (sum over k of A(i,k) * B(k,j) with both operands contiguous in k).  Each
 * C element is accumulated in increasing k in both forms, so the result does
 * not depend on the form, nor on how rows are spread over OpenMP threads.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

enum { OR_I8 = 0, OR_F16 = 1, OR_BF16 = 2, OR_F32 = 3 };
enum { OR_RR = 0, OR_RC = 1 };

/* ---- exact decoders, written from the bit-level definitions ---------- */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 is zero/subnormal (fraction * 2^-24); exponent 31 is
 * infinity (fraction 0) or NaN. */
double oracle_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bfloat16 is the upper 16 bits of an IEEE-754 binary32. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_f(int dtype, const void *p, int64_t idx)
{
    switch (dtype) {
    case OR_F16:  return oracle_f16_to_double(((const uint16_t *)p)[idx]);
    case OR_BF16: return oracle_bf16_to_double(((const uint16_t *)p)[idx]);
    default:      return (double)((const float *)p)[idx];
    }
}

static int64_t b_index(int layout, int64_t k, int64_t j, int64_t ldb)
{
    return layout == OR_RR ? k * ldb + j : j * ldb + k;
}

static int32_t wrap_i32(int64_t s)
{
    /* reduce modulo 2^32, then reinterpret as two's complement */
    uint32_t u = (uint32_t)((uint64_t)s & 0xffffffffu);
    int32_t r;
    memcpy(&r, &u, sizeof r);
    return r;
}

static int check_args(int dtype, int layout, int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda, const void *B, int64_t ldb)
{
    if (dtype < OR_I8 || dtype > OR_F32) return -1;
    if (layout != OR_RR && layout != OR_RC) return -1;
    if (M < 0 || N < 0 || K < 0) return -1;
    if ((M > 0 && K > 0) && (!A || lda < K)) return -1;
    if (N > 0 && K > 0) {
        if (!B) return -1;
        if (layout == OR_RR && ldb < N) return -1;
        if (layout == OR_RC && ldb < K) return -1;
    }
    return 0;
}

/* ---- one C element, accumulated in increasing k ----------------------- */

static int32_t dot_i8(int layout, int64_t i, int64_t j, int64_t K,
                      const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb)
{
    int64_t s = 0;
    for (int64_t k = 0; k < K; ++k)
        s += (int64_t)A[i * lda + k] * (int64_t)B[b_index(layout, k, j, ldb)];
    return wrap_i32(s);
}

static double dot_f(int dtype, int layout, int64_t i, int64_t j, int64_t K,
                    const void *A, int64_t lda, const void *B, int64_t ldb)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += load_f(dtype, A, i * lda + k) * load_f(dtype, B, b_index(layout, k, j, ldb));
    return s;
}

/*
 * Full product.  C points at int32 (dtype int8) or double (fp16, bf16, fp32)
 * storage with leading dimension ldc >= N.  Returns 0, or -1 on bad
 * arguments (nothing is written then).
 */
int oracle_gemm(int dtype, int layout, int64_t M, int64_t N, int64_t K,
                const void *A, int64_t lda, const void *B, int64_t ldb,
                void *C, int64_t ldc)
{
    if (check_args(dtype, layout, M, N, K, A, lda, B, ldb)) return -1;
    if (M > 0 && N > 0 && (!C || ldc < N)) return -1;

    if (dtype == OR_I8) {
        const int8_t *a = (const int8_t *)A, *b = (const int8_t *)B;
        int32_t *c = (int32_t *)C;
        if (layout == OR_RC) {
            #pragma omp parallel for schedule(static)
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = 0; j < N; ++j)
                    c[i * ldc + j] = dot_i8(layout, i, j, K, a, lda, b, ldb);
        } else {
            #pragma omp parallel
            {
                int64_t *acc = (int64_t *)malloc((size_t)(N > 0 ? N : 1) * sizeof(int64_t));
                #pragma omp for schedule(static)
                for (int64_t i = 0; i < M; ++i) {
                    for (int64_t j = 0; j < N; ++j) acc[j] = 0;
                    for (int64_t k = 0; k < K; ++k) {
                        int64_t aik = a[i * lda + k];
                        const int8_t *brow = b + k * ldb;
                        for (int64_t j = 0; j < N; ++j) acc[j] += aik * (int64_t)brow[j];
                    }
                    for (int64_t j = 0; j < N; ++j) c[i * ldc + j] = wrap_i32(acc[j]);
                }
                free(acc);
            }
        }
        return 0;
    }

    double *c = (double *)C;
    if (layout == OR_RC) {
        #pragma omp parallel
        {
            /* decode one row of A once; B columns are decoded on the fly */
            double *arow = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
            #pragma omp for schedule(static)
            for (int64_t i = 0; i < M; ++i) {
                for (int64_t k = 0; k < K; ++k) arow[k] = load_f(dtype, A, i * lda + k);
                for (int64_t j = 0; j < N; ++j) {
                    double s = 0.0;
                    for (int64_t k = 0; k < K; ++k)
                        s += arow[k] * load_f(dtype, B, j * ldb + k);
                    c[i * ldc + j] = s;
                }
            }
            free(arow);
        }
    } else {
        #pragma omp parallel
        {
            double *acc = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
            #pragma omp for schedule(static)
            for (int64_t i = 0; i < M; ++i) {
                for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double aik = load_f(dtype, A, i * lda + k);
                    for (int64_t j = 0; j < N; ++j)
                        acc[j] += aik * load_f(dtype, B, k * ldb + j);
                }
                for (int64_t j = 0; j < N; ++j) c[i * ldc + j] = acc[j];
            }
            free(acc);
        }
    }
    return 0;
}

/*
 * Selected entries only: out[t] = C(rows[t], cols[t]) for t < count, in the
 * same arithmetic as oracle_gemm.  out is int32 for int8 inputs, double
 * otherwise.  Used where the full product is too large for the CPU.
 */
int oracle_gemm_entries(int dtype, int layout, int64_t M, int64_t N, int64_t K,
                        const void *A, int64_t lda, const void *B, int64_t ldb,
                        int64_t count, const int64_t *rows, const int64_t *cols,
                        void *out)
{
    if (check_args(dtype, layout, M, N, K, A, lda, B, ldb)) return -1;
    if (count < 0 || (count > 0 && (!rows || !cols || !out))) return -1;
    for (int64_t t = 0; t < count; ++t)
        if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;

    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t) {
        if (dtype == OR_I8)
            ((int32_t *)out)[t] = dot_i8(layout, rows[t], cols[t], K,
                                         (const int8_t *)A, lda, (const int8_t *)B, ldb);
        else
            ((double *)out)[t] = dot_f(dtype, layout, rows[t], cols[t], K, A, lda, B, ldb);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_num_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
