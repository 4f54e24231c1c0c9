/* Host F16C conversions (x86 vcvtps2ph with immediate 0 = round to nearest
   even, and vcvtph2ps), the instruction the bankML f16 page names for the
   activation rounding (Design notes, "Activation").  Used only to pin the
   oracle's own conversions. */
#include <immintrin.h>
#include <stdint.h>

void f16c_to_f16(const float *x, uint16_t *y, int64_t n)
{
    int64_t i = 0;
    for (; i + 8 <= n; i += 8) {
        __m128i h = _mm256_cvtps_ph(_mm256_loadu_ps(x + i), 0);
        _mm_storeu_si128((__m128i *)(y + i), h);
    }
    for (; i < n; i++) y[i] = _cvtss_sh(x[i], 0);
}

void f16c_widen(const uint16_t *h, float *y, int64_t n)
{
    int64_t i = 0;
    for (; i + 8 <= n; i += 8)
        _mm256_storeu_ps(y + i, _mm256_cvtph_ps(_mm_loadu_si128((const __m128i *)(h + i))));
    for (; i < n; i++) y[i] = _cvtsh_ss(h[i]);
}
