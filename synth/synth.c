/* Host generator for seeded synthetic inputs (no arithmetic of the decoding
 * method lives here).  Philox4x32-10 (Salmon et al., SC'11) plus the
 * transcendental-free value maps documented in synth/__init__.py; the numpy
 * implementation there is the specification and tests compare the two. */
#include <stdint.h>
#include <stddef.h>

static inline void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

static inline float ih_value(uint64_t i, uint64_t seed, uint32_t stream, uint32_t purpose,
                             float scale) {
  uint32_t c[4] = {(uint32_t)i, (uint32_t)(i >> 32), stream, purpose};
  philox10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  int32_t s = 0;
  for (int j = 0; j < 4; ++j) s += (int32_t)(c[j] & 0xFFFFu) + (int32_t)(c[j] >> 16);
  return (float)(s - 262140) * scale;
}

static inline uint16_t f32_to_bf16(float f) {
  union { float f; uint32_t u; } v; v.f = f;
  uint32_t rnd = ((v.u >> 16) & 1u) + 0x7FFFu;
  return (uint16_t)((v.u + rnd) >> 16);
}

/* kind 0: float32 out; kind 1: bf16 bit patterns (uint16) out. */
void synth_fill_normal(void* out, uint64_t n, uint64_t start, uint64_t seed, uint32_t stream,
                       uint32_t purpose, float scale, int kind) {
  if (kind == 0) {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i)
      o[i] = ih_value(start + (uint64_t)i, seed, stream, purpose, scale);
  } else {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i)
      o[i] = f32_to_bf16(ih_value(start + (uint64_t)i, seed, stream, purpose, scale));
  }
}
