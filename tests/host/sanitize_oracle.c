/*
 * Runs the CPU oracle (oracle/oracle_gemm.c, compiled into this program)
 * under AddressSanitizer and UndefinedBehaviorSanitizer: every dtype and
 * layout, shapes from empty to ragged, padded leading dimensions, output
 * rows wider than N, and the argument errors.  Buffers are sized exactly to
 * the matrices they hold, so any read or write past them is reported.
 * Checks: full and entry-wise results agree bit for bit, and C's padding
 * columns are never written.  Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm(int dtype, int layout, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                const void *B, int64_t ldb, void *C, int64_t ldc);
int oracle_gemm_entries(int dtype, int layout, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                        const void *B, int64_t ldb, int64_t count, const int64_t *rows, const int64_t *cols,
                        void *out);

static int esize(int dt) { return dt == 0 ? 1 : dt == 3 ? 4 : 2; }

/* Small finite values of each type from a counter. */
static void fill(int dt, void *p, int64_t n, unsigned seed) {
    for (int64_t i = 0; i < n; ++i) {
        unsigned v = (unsigned)(i * 2654435761u + seed * 40503u) >> 7;
        if (dt == 0) ((int8_t *)p)[i] = (int8_t)(v & 0xff);
        else if (dt == 1) ((uint16_t *)p)[i] = (uint16_t)(0x3000 | (v & 0x3ff) | ((v & 0x400) << 5)); /* |x| < 1 */
        else if (dt == 2) ((uint16_t *)p)[i] = (uint16_t)(0x3e00 | (v & 0x7f) | ((v & 0x80) << 8));
        else { float f = (float)((int)(v % 2001) - 1000) / 1000.0f; memcpy((char *)p + 4 * i, &f, 4); }
    }
}

int main(void) {
    static const int64_t shapes[][3] = {{0, 0, 0}, {1, 1, 1}, {0, 5, 3}, {4, 0, 3}, {3, 4, 0},
                                        {3, 5, 7}, {17, 9, 33}, {33, 31, 70}};
    int fails = 0;
    for (int dt = 0; dt < 4; ++dt)
        for (int lay = 0; lay < 2; ++lay)
            for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
                const int64_t M = shapes[s][0], N = shapes[s][1], K = shapes[s][2];
                const int64_t lda = K + 3, ldb = (lay == 0 ? N : K) + 2, ldc = N + 1;
                const int64_t brows = lay == 0 ? K : N, bcols = lay == 0 ? N : K;
                const int64_t na = M > 0 ? (M - 1) * lda + K : 0, nb = brows > 0 ? (brows - 1) * ldb + bcols : 0;
                const int64_t nc = M > 0 ? (M - 1) * ldc + N + 1 : 1;   /* one padding column after each row */
                const int osz = dt == 0 ? 4 : 8;
                void *A = malloc((size_t)(na > 0 ? na : 1) * esize(dt));
                void *B = malloc((size_t)(nb > 0 ? nb : 1) * esize(dt));
                unsigned char *C = malloc((size_t)nc * osz);
                fill(dt, A, na, 1 + (unsigned)s);
                fill(dt, B, nb, 7 + (unsigned)s);
                memset(C, 0xA5, (size_t)nc * osz);
                if (oracle_gemm(dt, lay, M, N, K, na ? A : NULL, lda, nb ? B : NULL, ldb, C, ldc) != 0) {
                    printf("oracle_gemm refused dt=%d lay=%d shape %ld %ld %ld\n", dt, lay, (long)M, (long)N, (long)K);
                    ++fails;
                }
                for (int64_t i = 0; i < M; ++i)   /* C(i, N) and beyond up to ldc stay untouched */
                    for (int64_t j = N; j < ldc && i * ldc + j < nc; ++j)
                        for (int b = 0; b < osz; ++b)
                            if (C[(i * ldc + j) * osz + b] != 0xA5) { ++fails; printf("wrote padding\n"); i = M; j = ldc; break; }
                if (M > 0 && N > 0) {
                    const int64_t cnt = M * N < 50 ? M * N : 50;
                    int64_t *rows = malloc((size_t)cnt * 8), *cols = malloc((size_t)cnt * 8);
                    unsigned char *out = malloc((size_t)cnt * osz);
                    for (int64_t t = 0; t < cnt; ++t) { rows[t] = (t * 7) % M; cols[t] = (t * 5) % N; }
                    if (oracle_gemm_entries(dt, lay, M, N, K, A, lda, B, ldb, cnt, rows, cols, out) != 0) ++fails;
                    for (int64_t t = 0; t < cnt; ++t)
                        if (memcmp(out + t * osz, C + (rows[t] * ldc + cols[t]) * osz, (size_t)osz) != 0) {
                            ++fails; printf("entry differs dt=%d lay=%d\n", dt, lay); break;
                        }
                    free(rows); free(cols); free(out);
                }
                free(A); free(B); free(C);
            }
    /* argument errors: nothing is read or written */
    int8_t a = 1, b = 1; int32_t c = 0;
    if (oracle_gemm(0, 1, 1, 1, 1, &a, 0, &b, 1, &c, 1) == 0) ++fails;      /* lda < K */
    if (oracle_gemm(0, 1, -1, 1, 1, &a, 1, &b, 1, &c, 1) == 0) ++fails;     /* negative size */
    if (oracle_gemm(9, 1, 1, 1, 1, &a, 1, &b, 1, &c, 1) == 0) ++fails;      /* bad dtype */
    if (oracle_gemm(0, 1, 1, 1, 1, &a, 1, &b, 1, NULL, 1) == 0) ++fails;    /* no C */
    printf(fails ? "FAIL (%d)\n" : "oracle under ASan/UBSan: OK\n", fails);
    return fails ? 1 : 0;
}
