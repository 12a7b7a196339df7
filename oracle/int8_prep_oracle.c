/*
 * int8_prep_oracle.c -- plain CPU oracle for the LLM.int8 correction-operand
 * preparation.
 *
 * TEST INFRASTRUCTURE ONLY (see dq4_oracle.c): used by the tests, the smoke
 * check and the benchmark's CPU baseline, never by the product path, and it
 * shares no code with the HIP library.
 *
 * What it computes (bitsandbytes issue "Fuse LLM.int8 correction operand
 * preparation into one CUDA kernel", sections "Summary", "Bounded method" and
 * "Exact correctness oracle"):
 *   subA[r][l] = A[r][cols[l]]                     a raw 16-bit copy, r < M, l < L
 *   subB[l][n] = fp16(fl32(fl32(CB[n][cols[l]] * SCB[n]) * R127))        n < N
 * i.e. the eager chain gather -> int8 row-scale dequantization (an FP32
 * multiply by the row scale, then a separately rounded FP32 multiply by the
 * reciprocal-127 constant) -> FP16 conversion -> transpose.
 * Readings: R127 is the FP32 value nearest to 1/127 (the page names "the
 * existing reciprocal-127 constant" but prints no digits); A and subA are
 * 16-bit values copied bit for bit; cols may repeat and appear in any order.
 * Compile with -ffp-contract=off (no fused multiplies).
 */
#include <stdint.h>
#include <string.h>

uint16_t dq4o_f32_to_f16(float x); /* dq4_oracle.c: IEEE RNE conversion */

int dq4o_int8_prep(const uint16_t *A, int64_t M, int64_t K, const int8_t *CB,
                   const float *SCB, int64_t N, const int64_t *cols, int64_t L,
                   uint16_t *subA, uint16_t *subB)
{
    if (M < 0 || K < 0 || N < 0 || L < 0)
        return 1;
    const float r127 = (float)(1.0 / 127.0);
    for (int64_t l = 0; l < L; ++l)
        if (cols[l] < 0 || cols[l] >= K)
            return 1;

    /* the activation gather */
    for (int64_t r = 0; r < M; ++r)
        for (int64_t l = 0; l < L; ++l)
            subA[r * L + l] = A[r * K + cols[l]];

    /* the weight gather, dequantization, conversion and transpose */
    for (int64_t l = 0; l < L; ++l) {
        for (int64_t n = 0; n < N; ++n) {
            const float code = (float)CB[n * K + cols[l]];
            const float scaled = code * SCB[n];
            const float v = scaled * r127;
            subB[l * N + n] = dq4o_f32_to_f16(v);
        }
    }
    return 0;
}
