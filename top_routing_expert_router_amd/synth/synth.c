/*
 * Seeded synthetic inputs, shared by the GPU path's callers and by the tests
 * that feed the CPU oracle.  This file holds no arithmetic of the MoE method:
 * it only turns (seed, element index) into a number.
 *
 * Generator (counter-based, so any slice of a tensor can be produced alone):
 *   - SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014; the 64-bit finaliser constants of Vigna's
 *     public-domain splitmix64): output j of the stream that starts at state s
 *     is mix(s + (j+1)*0x9E3779B97F4A7C15).
 *   - A tensor seed s0 is first whitened into a stream key = output 0 of the
 *     stream at s0; element counters then run on that key.
 *   - Uniform in (0,1]: ((z >> 11) + 1) * 2^-53.
 *   - Normal: Box & Muller (1958).  Pair m uses uniforms 2m and 2m+1:
 *     r = sqrt(-2 ln u1), th = 2 pi u2; element 2m = r cos th, 2m+1 = r sin th.
 *   - Stored value: sigma * n rounded to float32 (round-to-nearest-even),
 *     then, for bf16 tensors, float32 -> bf16 round-to-nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Output j (0-based) of the SplitMix64 stream whose state starts at s. */
uint64_t synth_splitmix64(uint64_t s, uint64_t j) { return sm_mix(s + (j + 1) * SM_GAMMA); }

static inline double sm_uniform(uint64_t key, uint64_t j) {
  return (double)((synth_splitmix64(key, j) >> 11) + 1) * 0x1.0p-53;
}

static inline double sm_normal(uint64_t key, uint64_t i) {
  uint64_t m = i >> 1;
  double u1 = sm_uniform(key, 2 * m);
  double u2 = sm_uniform(key, 2 * m + 1);
  double r = sqrt(-2.0 * log(u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Elements [first, first+count) of the N(0, sigma^2) tensor with seed s0. */
void synth_normal_f64(uint64_t s0, int64_t first, int64_t count, double sigma, double *out) {
  uint64_t key = synth_splitmix64(s0, 0);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = sigma * sm_normal(key, (uint64_t)(first + i));
}

void synth_normal_f32(uint64_t s0, int64_t first, int64_t count, double sigma, float *out) {
  uint64_t key = synth_splitmix64(s0, 0);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)(sigma * sm_normal(key, (uint64_t)(first + i)));
}

void synth_normal_bf16(uint64_t s0, int64_t first, int64_t count, double sigma, uint16_t *out) {
  uint64_t key = synth_splitmix64(s0, 0);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i)
    out[i] = f32_to_bf16_rne((float)(sigma * sm_normal(key, (uint64_t)(first + i))));
}

/* Raw 64-bit draws (for tests that need integers): out[i] = output (first+i) of the keyed stream. */
void synth_u64(uint64_t s0, int64_t first, int64_t count, uint64_t *out) {
  uint64_t key = synth_splitmix64(s0, 0);
  for (int64_t i = 0; i < count; ++i) out[i] = synth_splitmix64(key, (uint64_t)(first + i));
}
