/*
 * Sanitizer driver for the CPU oracle (a test, built with
 * -fsanitize=address,undefined by tests/test_sanitizers.py).  Every input is
 * a heap buffer of exactly the size the operation defines -- ceil(n/2)
 * packed bytes, ceil(n/blocksize) codes, ceil(blocks/256) absmax values --
 * so a read one element past the end is reported.  Inputs are filled from a
 * linear congruential sequence; nothing here computes the method.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int dq4o_dequant_range(const uint8_t *, const uint8_t *, const float *, const float *,
                       const float *, float, int64_t, int64_t, int32_t, int32_t, int32_t, void *);
int dq4o_dequant_rows(const uint8_t *, const uint8_t *, const float *, const float *,
                      const float *, float, int64_t, int64_t, int64_t, int64_t, int32_t, int32_t,
                      int32_t, void *);
int dq4o_int8_prep(const uint16_t *, int64_t, int64_t, const int8_t *, const float *, int64_t,
                   const int64_t *, int64_t, uint16_t *, uint16_t *);

static uint32_t state = 12345u;
static uint32_t next(void) { state = state * 1664525u + 1013904223u; return state >> 8; }

static void *exact(size_t n) { return malloc(n ? n : 1); }

static int run_dequant(int64_t n, int32_t bs, int32_t dtype)
{
    const int64_t nb = (n + bs - 1) / bs, ng = (nb + 255) / 256;
    uint8_t *packed = exact((size_t)((n + 1) / 2));
    uint8_t *codes = exact((size_t)nb);
    float *absmax = exact((size_t)ng * 4);
    float *scb = exact(256 * 4), *cb4 = exact(16 * 4);
    for (int64_t i = 0; i < (n + 1) / 2; ++i) packed[i] = (uint8_t)next();
    for (int64_t i = 0; i < nb; ++i) codes[i] = (uint8_t)next();
    for (int64_t i = 0; i < ng; ++i) absmax[i] = (float)(next() % 1000) / 997.0f;
    for (int i = 0; i < 256; ++i) scb[i] = (float)((int)(next() % 2001) - 1000) / 1000.0f;
    for (int i = 0; i < 16; ++i) cb4[i] = (float)((int)(next() % 2001) - 1000) / 1000.0f;
    const size_t ebytes = dtype == 0 ? 4 : 2;
    void *out = exact((size_t)n * ebytes);
    int rc = dq4o_dequant_range(packed, codes, absmax, scb, cb4, 0.03f, 0, n, bs, 256, dtype, out);
    /* a row window that starts mid-byte and mid-block, ending at the last element */
    if (rc == 0 && n >= 7) {
        const int64_t cols = 7, rows = n / cols, r0 = rows / 2;
        void *win = exact((size_t)(rows - r0) * cols * ebytes);
        rc = dq4o_dequant_rows(packed, codes, absmax, scb, cb4, -0.1f, rows, cols, r0, rows - r0,
                               bs, 256, dtype, win);
        free(win);
    }
    free(packed); free(codes); free(absmax); free(scb); free(cb4); free(out);
    return rc;
}

static int run_int8(int64_t M, int64_t K, int64_t N, int64_t L)
{
    uint16_t *A = exact((size_t)(M * K) * 2);
    int8_t *CB = exact((size_t)(N * K));
    float *SCB = exact((size_t)N * 4);
    int64_t *cols = exact((size_t)L * 8);
    uint16_t *subA = exact((size_t)(M * L) * 2), *subB = exact((size_t)(L * N) * 2);
    for (int64_t i = 0; i < M * K; ++i) A[i] = (uint16_t)next();
    for (int64_t i = 0; i < N * K; ++i) CB[i] = (int8_t)next();
    for (int64_t i = 0; i < N; ++i) SCB[i] = (float)(next() % 100000) / 7.0f;
    for (int64_t i = 0; i < L; ++i) cols[i] = (int64_t)(next() % (uint32_t)K);
    cols[0] = K - 1;
    const int rc = dq4o_int8_prep(A, M, K, CB, SCB, N, cols, L, subA, subB);
    free(A); free(CB); free(SCB); free(cols); free(subA); free(subB);
    return rc;
}

int main(void)
{
    static const int32_t sizes[] = {32, 64, 256, 4096};
    int failures = 0;
    for (int s = 0; s < 4; ++s) {
        const int64_t B = sizes[s];
        const int64_t lengths[] = {1, 2, 3, B - 1, B, B + 1, 256 * B - 1, 256 * B + 1,
                                   256 * B + B + 1};
        for (int k = 0; k < 9; ++k)
            for (int32_t dt = 0; dt < 3; ++dt)
                if (run_dequant(lengths[k], (int32_t)B, dt) != 0) {
                    printf("dequant n=%lld bs=%lld dtype=%d failed\n", (long long)lengths[k],
                           (long long)B, dt);
                    ++failures;
                }
    }
    if (run_int8(3, 100, 5, 4) != 0 || run_int8(1, 1, 1, 1) != 0 || run_int8(2, 64, 0, 3) != 0)
        ++failures;
    printf("oracle sanitizer driver: %d failures\n", failures);
    return failures != 0;
}
