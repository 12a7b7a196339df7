/* IEEE binary32 -> binary16 bit patterns by the host CPU's F16C instruction
 * (vcvtps2ph with the round-to-nearest-even immediate): a reference for the
 * oracle's FP16 conversion that shares nothing with it.  Test infrastructure,
 * built by tests/test_oracle_pins.py with gcc -mf16c. */
#include <immintrin.h>
#include <stddef.h>
#include <stdint.h>

void f16c_convert(const uint32_t *in, uint16_t *out, size_t n)
{
    size_t i = 0;
    for (; i + 8 <= n; i += 8) {
        const __m256 v = _mm256_castsi256_ps(_mm256_loadu_si256((const __m256i *)(in + i)));
        const __m128i h = _mm256_cvtps_ph(v, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
        _mm_storeu_si128((__m128i *)(out + i), h);
    }
    for (; i < n; ++i) {
        const __m128 v = _mm_castsi128_ps(_mm_cvtsi32_si128((int)in[i]));
        const __m128i h = _mm_cvtps_ph(v, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
        out[i] = (uint16_t)_mm_extract_epi16(h, 0);
    }
}
