/* Bulk fill of counter-based synthetic bf16 values (input generation only).
 *
 * Implements exactly the definition in values.py: three SplitMix64 outputs
 * per element, the sum of their twelve 16-bit fields, (S - 393210) / 65536
 * as float32, rounded to bfloat16 nearest-even -- or, for FP8 pools, divided
 * by the layer scale (float32) and rounded to an OCP FP8 E4M3 code, nearest
 * with ties to the even code, saturating at 448.  Used to fill large pinned
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

static inline float value_f32(uint64_t key, uint64_t e) {
  int64_t s = 0;
  for (int i = 0; i < 3; ++i) {
    uint64_t w = mix64(key + (3 * e + (uint64_t)i + 1) * GOLDEN);
    s += (int64_t)(w & 0xFFFF) + (int64_t)((w >> 16) & 0xFFFF) +
         (int64_t)((w >> 32) & 0xFFFF) + (int64_t)((w >> 48) & 0xFFFF);
  }
  return (float)(s - 393210) / 65536.0f; /* exact: |s - 393210| < 2^24 */
}

static inline uint16_t value_bits(uint64_t key, uint64_t e) {
  float f = value_f32(key, e);
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* float32 -> OCP FP8 E4M3 code: keep the float32 significand (leading 1
 * included) in quanta of 2^(max(E, -6) - 3), round the dropped bits to
 * nearest-even, saturate at 448 (0x7E). */
static inline uint8_t e4m3_code(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  const uint8_t sign = (uint8_t)((b >> 31) << 7);
  const int e32 = (int)((b >> 23) & 0xFF);
  if (e32 == 0) return sign; /* zero or a float32 subnormal (far below 2^-10) */
  const int64_t sig = (int64_t)((b & 0x7FFFFF) | (1u << 23));
  const int E = e32 - 127;
  const int qexp = (E > -6 ? E : -6) - 3;
  int shift = qexp - (E - 23);
  if (shift > 62) shift = 62;
  int64_t q = sig >> shift;
  const int64_t rem = sig - (q << shift);
  const int64_t half = (int64_t)1 << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  int64_t mag = E >= -6 ? ((int64_t)(E + 7) << 3) + (q - 8) : q;
  if (mag > 0x7E) mag = 0x7E;
  return (uint8_t)(sign | (uint8_t)mag);
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

/* FP8 rows: dst[i*dim + d] = e4m3(value(key, pos[i]*dim + d) / scale). */
void tg_fill_rows_fp8(uint8_t* dst, uint64_t key, const int64_t* pos, int64_t nrows, int64_t dim, float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    uint64_t base = (uint64_t)pos[i] * (uint64_t)dim;
    for (int64_t d = 0; d < dim; ++d) dst[i * dim + d] = e4m3_code(value_f32(key, base + (uint64_t)d) / scale);
  }
}

/* dst[i] = e4m3(value(key, e0 + i) / scale) for i in [0, n). */
void tg_fill_fp8(uint8_t* dst, uint64_t key, uint64_t e0, uint64_t n, float scale) {
  int64_t nn = (int64_t)n;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nn; ++i) dst[i] = e4m3_code(value_f32(key, e0 + (uint64_t)i) / scale);
}
