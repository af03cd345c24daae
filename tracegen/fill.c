/* Bulk fill of counter-based synthetic bf16 values (input generation only).
 *
 * Implements exactly the definition in values.py: three SplitMix64 outputs
 * per element, the sum of their twelve 16-bit fields, (S - 393210) / 65536
 * as float32, rounded to bfloat16 nearest-even.  Used to fill large pinned
 * host pools quickly; the NumPy code regenerates any element for checking.
 */
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint16_t value_bits(uint64_t key, uint64_t e) {
  int64_t s = 0;
  for (int i = 0; i < 3; ++i) {
    uint64_t w = mix64(key + (3 * e + (uint64_t)i + 1) * GOLDEN);
    s += (int64_t)(w & 0xFFFF) + (int64_t)((w >> 16) & 0xFFFF) +
         (int64_t)((w >> 32) & 0xFFFF) + (int64_t)((w >> 48) & 0xFFFF);
  }
  float f = (float)(s - 393210) / 65536.0f; /* exact: |s - 393210| < 2^24 */
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* dst[i] = value(key, e0 + i) for i in [0, n). */
void tg_fill(uint16_t* dst, uint64_t key, uint64_t e0, uint64_t n) {
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) dst[i] = value_bits(key, e0 + (uint64_t)i);
}

/* Rows of dim elements: dst[i*dim + d] = value(key, pos[i]*dim + d). */
void tg_fill_rows(uint16_t* dst, uint64_t key, const int64_t* pos, int64_t nrows, int64_t dim) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    uint64_t base = (uint64_t)pos[i] * (uint64_t)dim;
    for (int64_t d = 0; d < dim; ++d) dst[i * dim + d] = value_bits(key, base + (uint64_t)d);
  }
}
