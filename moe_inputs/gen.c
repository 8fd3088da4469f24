/*
 * Seeded synthetic inputs shared by the CPU oracle and the GPU path.
 *
 * This file holds random-number generation only: none of the MoE method's
 * arithmetic (routing, layout, FFN, delivery, combine) lives here.
 *
 * Generator: the i-th value of a stream is the splitmix64 output mix(key + (i+1)*gamma)
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014),
 * which makes it counter-based and trivially parallel.  The stream key is itself a
 * splitmix64 output of (seed, stream id).  Normal deviates use the Box-Muller transform
 * (Box and Muller, 1958) on two 53-bit uniforms in double precision; value 2j uses the
 * cosine branch and value 2j+1 the sine branch of pair j.  Results are scaled by sigma in
 * double, rounded to fp32, and for bf16 outputs rounded once more from fp32 to bf16 with
 * round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GAMMA) ^ (stream * 0xD1B54A32D192ED03ULL));
}

/* uniform in the open interval (0, 1) from the top 53 bits */
static inline double u01(uint64_t r) {
  return ((double)(r >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, int64_t i) {
  int64_t pair = i >> 1;
  uint64_t r1 = mix64(key + (uint64_t)(2 * pair + 1) * GAMMA);
  uint64_t r2 = mix64(key + (uint64_t)(2 * pair + 2) * GAMMA);
  double rad = sqrt(-2.0 * log(u01(r1)));
  double ang = 6.283185307179586476925286766559 * u01(r2);
  return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

static inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t b;
  memcpy(&b, &v, 4);
  uint32_t lsb = (b >> 16) & 1u;
  b += 0x7FFFu + lsb;
  return (uint16_t)(b >> 16);
}

/* out[i] = fp32(mu + sigma * N_i), i in [0, n) */
void gen_normal_f32(uint64_t seed, uint64_t stream, int64_t n, double mu, double sigma, float* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mu + sigma * normal_at(key, i));
}

/* out[i] = bf16_rne(fp32(mu + sigma * N_i)) as raw bits */
void gen_normal_bf16(uint64_t seed, uint64_t stream, int64_t n, double mu, double sigma, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)(mu + sigma * normal_at(key, i)));
}

/* raw 64-bit stream values, for tests of the generator itself */
void gen_raw_u64(uint64_t seed, uint64_t stream, int64_t n, uint64_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = mix64(key + (uint64_t)(i + 1) * GAMMA);
}

/* plain sequential splitmix64 from a given state (the published reference generator), for tests */
void gen_splitmix64_seq(uint64_t state, int64_t n, uint64_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = mix64(state + (uint64_t)(i + 1) * GAMMA);
}
