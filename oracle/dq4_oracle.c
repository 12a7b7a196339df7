/*
 * dq4_oracle.c -- plain CPU oracle for nested (double-quantized) block-wise
 * 4-bit dequantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code with the HIP library.
 *
 * What it computes (bitsandbytes issue "Fuse nested scale reconstruction
 * into SM103 4-bit dequantization", sections "Problem" and "Proposed
 * experiment"): the existing three-step nested dequantization, whose result
 * the fused kernel must reproduce bit for bit:
 *   1. each uint8 scale code becomes an FP32 value
 *        t = scale_codebook[code] * nested_absmax[group]        (FP32 multiply)
 *   2. the nested offset is added in a separate FP32 operation
 *        s = t + offset                                         (FP32 add)
 *   3. each packed 4-bit value is decoded through its 16-entry table and
 *      multiplied by its block's scale
 *        v = codebook4[nibble] * s                              (FP32 multiply)
 *      then written as FP32, FP16 or BF16.
 * The section "Correctness requirements" fixes that the multiply and the add
 * are rounded separately (no contraction).  This file must be compiled with
 * -ffp-contract=off and without -ffast-math; on x86-64 float arithmetic is
 * SSE single precision (FLT_EVAL_METHOD 0), so each operation above is one
 * IEEE binary32 round-to-nearest-even step.
 *
 * Readings taken where the pages are silent:
 *   - element i of the flat row-major tensor sits in byte i/2, low nibble for
 *     even i, high nibble for odd i;
 *   - outer block b = i / blocksize, nested group g = b / nested_blocksize
 *     (the nested group counts outer blocks; the pages' default is 256);
 *   - the last block and the last group may be partial; for odd n the high
 *     nibble of the last byte is padding and is never written;
 *   - FP16 and BF16 outputs are IEEE round-to-nearest-even conversions of the
 *     FP32 value, subnormals kept;
 *   - a row window [r0, r0 + rows) of an n_rows x n_cols weight (llama.cpp
 *     PR "out_prod dequantizes a 2D weight in row blocks", section "What")
 *     is the same computation restricted to global elements
 *     [r0*n_cols, (r0+rows)*n_cols), written from output index 0, with the
 *     block and group indices taken from the global element index.
 */
#include <stdint.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* ---------------------------------------------------------------------------
 * IEEE-754 round-to-nearest-even conversion of a binary32 value to a narrower
 * binary format, written from the definition of the formats:
 *   a finite nonzero binary32 value is m * 2^e with an integer m < 2^24;
 *   the narrow format with `frac_bits` stored fraction bits represents
 *   q * 2^k with integer q < 2^(frac_bits+1), where the quantum exponent is
 *   k = max(kmin, floor(log2 |x|) - frac_bits) and kmin is the quantum of its
 *   subnormals.  Its encoding is ((k - kmin) << frac_bits) + q, which covers
 *   both subnormals (k == kmin, q below the hidden bit) and normals, and a
 *   rounding carry into the next binade.  Encodings at or above the all-ones
 *   exponent overflow to infinity.
 * ------------------------------------------------------------------------- */
static uint32_t f32_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return u;
}

static int floor_log2_u32(uint32_t m) /* m > 0 */
{
    return 31 - __builtin_clz(m);
}

static uint32_t round_binary32_to_narrow(float x, int frac_bits, int kmin,
                                         uint32_t exp_all_ones, uint32_t quiet_nan)
{
    const uint32_t u = f32_bits(x);
    const uint32_t sign = u >> 31;
    const uint32_t biased = (u >> 23) & 0xFFu;
    const uint32_t fraction = u & 0x7FFFFFu;
    const uint32_t sign_bit = sign << 15; /* both narrow formats are 16 bits wide */
    const uint32_t inf_bits = exp_all_ones << frac_bits;

    if (biased == 0xFFu)
        return sign_bit | (fraction ? quiet_nan : inf_bits);

    uint32_t m;
    int e;
    if (biased == 0) { /* zero or binary32 subnormal */
        m = fraction;
        e = -149;
    } else {
        m = fraction | 0x800000u;
        e = (int)biased - 150;
    }
    if (m == 0)
        return sign_bit;

    int k = floor_log2_u32(m) + e - frac_bits;
    if (k < kmin)
        k = kmin;

    uint64_t q;
    const int shift = k - e; /* value / 2^k = m * 2^(e-k) */
    if (shift <= 0) {
        q = (uint64_t)m << (-shift);
    } else if (shift > 40) {
        q = 0; /* far below half a quantum */
    } else {
        const uint64_t mm = m;
        q = mm >> shift;
        const uint64_t rem = mm & ((1ull << shift) - 1);
        const uint64_t half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (q & 1)))
            q += 1;
    }
    uint64_t enc = ((uint64_t)(k - kmin) << frac_bits) + q;
    if (enc >= inf_bits)
        enc = inf_bits;
    return sign_bit | (uint32_t)enc;
}

uint16_t dq4o_f32_to_f16(float x)
{
    /* binary16: 10 fraction bits, subnormal quantum 2^-24, exponent field 31 */
    return (uint16_t)round_binary32_to_narrow(x, 10, -24, 0x1Fu, 0x200u | 0x7C00u);
}

uint16_t dq4o_f32_to_bf16(float x)
{
    /* bfloat16: 7 fraction bits, subnormal quantum 2^-133, exponent field 255 */
    return (uint16_t)round_binary32_to_narrow(x, 7, -133, 0xFFu, 0x40u | 0x7F80u);
}

/* Bulk forms over raw binary32 bit patterns (used by the exhaustive checks). */
void dq4o_f32_to_f16_array(const uint32_t *in, uint16_t *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) {
        float x;
        memcpy(&x, &in[i], sizeof x);
        out[i] = dq4o_f32_to_f16(x);
    }
}

void dq4o_f32_to_bf16_array(const uint32_t *in, uint16_t *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) {
        float x;
        memcpy(&x, &in[i], sizeof x);
        out[i] = dq4o_f32_to_bf16(x);
    }
}

/* ---------------------------------------------------------------------------
 * The dequantization itself, one element at a time, in element order.
 * Elements [first, first + count) of the flat tensor are produced; output
 * index 0 holds element `first`.  The scale is recomputed for every element:
 * that is the same value for every element of a block and keeps this code a
 * direct transcription of the definition.
 * ------------------------------------------------------------------------- */
int dq4o_dequant_range(const uint8_t *packed, const uint8_t *scale_codes,
                       const float *nested_absmax, const float *scale_codebook,
                       const float *codebook4, float offset, int64_t first,
                       int64_t count, int32_t blocksize, int32_t nested_blocksize,
                       int32_t out_dtype, void *out)
{
    if (count < 0 || first < 0 || blocksize <= 0 || nested_blocksize <= 0)
        return 1;
    if (out_dtype != ORACLE_F32 && out_dtype != ORACLE_F16 && out_dtype != ORACLE_BF16)
        return 1;

    for (int64_t j = 0; j < count; ++j) {
        const int64_t i = first + j;

        /* indexing: outer block, then nested group counted in outer blocks */
        const int64_t b = i / blocksize;
        const int64_t g = b / nested_blocksize;

        /* step 1: scale code -> FP32 (one rounded multiply) */
        const float t = scale_codebook[scale_codes[b]] * nested_absmax[g];
        /* step 2: the nested offset, a separate rounded add */
        const float s = t + offset;

        /* step 3: 4-bit decode, low nibble first */
        const uint8_t byte = packed[i / 2];
        const unsigned nibble = (i % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
        const float v = codebook4[nibble] * s;

        switch (out_dtype) {
        case ORACLE_F32:
            ((float *)out)[j] = v;
            break;
        case ORACLE_F16:
            ((uint16_t *)out)[j] = dq4o_f32_to_f16(v);
            break;
        default:
            ((uint16_t *)out)[j] = dq4o_f32_to_bf16(v);
            break;
        }
    }
    return 0;
}

/* Whole tensor of n elements. */
int dq4o_dequant(const uint8_t *packed, const uint8_t *scale_codes,
                 const float *nested_absmax, const float *scale_codebook,
                 const float *codebook4, float offset, int64_t n,
                 int32_t blocksize, int32_t nested_blocksize, int32_t out_dtype,
                 void *out)
{
    return dq4o_dequant_range(packed, scale_codes, nested_absmax, scale_codebook,
                              codebook4, offset, 0, n, blocksize, nested_blocksize,
                              out_dtype, out);
}

/* Rows [r0, r0 + rows) of an n_rows x n_cols row-major weight. */
int dq4o_dequant_rows(const uint8_t *packed, const uint8_t *scale_codes,
                      const float *nested_absmax, const float *scale_codebook,
                      const float *codebook4, float offset, int64_t n_rows,
                      int64_t n_cols, int64_t r0, int64_t rows, int32_t blocksize,
                      int32_t nested_blocksize, int32_t out_dtype, void *out)
{
    if (n_rows < 0 || n_cols < 0 || r0 < 0 || rows < 0 || r0 + rows > n_rows)
        return 1;
    return dq4o_dequant_range(packed, scale_codes, nested_absmax, scale_codebook,
                              codebook4, offset, r0 * n_cols, rows * n_cols,
                              blocksize, nested_blocksize, out_dtype, out);
}

/*
 * Rows per transient block (llama.cpp PR, review): the transient holds
 * rows_per_block x n_cols elements of elem_bytes each and stays within the
 * budget, with at least one row.
 */
int64_t dq4o_rows_per_block(int64_t n_cols, int64_t elem_bytes, int64_t budget_bytes)
{
    if (n_cols <= 0 || elem_bytes <= 0 || budget_bytes <= 0)
        return 1;
    const int64_t r = budget_bytes / (n_cols * elem_bytes);
    return r < 1 ? 1 : r;
}
