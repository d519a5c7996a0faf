/* Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.
 *
 * This module only draws random numbers and stores them in the input formats (bf16, f32). It holds none of the
 * NVFP4 / LoRA / AQN arithmetic, so neither the oracle nor the HIP library depends on the other through it.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014), with the 64-bit output mixer that S. Vigna's public-domain reference splitmix64.c uses. SplitMix64's
 * state advances by a fixed odd increment, so output i of a stream is a pure function of (seed, i): the streams are
 * counter-based and every element is computed independently (and in parallel) from its index.
 *   output(seed, i) = mix(seed + (i + 1) * 0x9E3779B97F4A7C15)
 * Uniform doubles on [0,1) take the top 53 bits. Normals use the Box-Muller transform (Box & Muller 1958):
 * element 2j and 2j+1 come from uniforms 2j and 2j+1 as r*cos(2 pi u2), r*sin(2 pi u2), r = sqrt(-2 ln(1 - u1)).
 * Conversion to bf16 is double -> f32 (IEEE round-to-nearest-even) -> bf16 (round-to-nearest-even on the upper
 * 16 bits). That fixes the bytes of every input; both sides of every comparison read the same bytes.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static const uint64_t kGamma = 0x9E3779B97F4A7C15ull;

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t sm64_at(uint64_t seed, uint64_t i) { return mix64(seed + (i + 1u) * kGamma); }

static inline double uniform_at(uint64_t seed, uint64_t i) { return (double)(sm64_at(seed, i) >> 11) * 0x1.0p-53; }

/* Standard normal number i of the stream. */
static inline double normal_at(uint64_t seed, uint64_t i) {
  uint64_t pair = i >> 1;
  double u1 = uniform_at(seed, 2 * pair), u2 = uniform_at(seed, 2 * pair + 1);
  double r = sqrt(-2.0 * log(1.0 - u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN stays NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t syn_splitmix64(uint64_t seed, uint64_t i) { return sm64_at(seed, i); }

void syn_uniform_f64(uint64_t seed, int64_t count, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = uniform_at(seed, (uint64_t)i);
}

void syn_normal_f64(uint64_t seed, int64_t count, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = normal_at(seed, (uint64_t)i);
}

void syn_normal_f32(uint64_t seed, double stddev, int64_t count, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)(stddev * normal_at(seed, (uint64_t)i));
}

void syn_normal_bf16(uint64_t seed, double stddev, int64_t count, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = f32_to_bf16_rne((float)(stddev * normal_at(seed, (uint64_t)i)));
}

/* Student-t with nu = 4 degrees of freedom: Z / sqrt(chi2_4 / 4), with Z and the four squared normals of chi2_4
 * taken as normals 5i .. 5i+4 of the stream. If block > 0, every run of `block` consecutive elements is further
 * multiplied by 2^e with e uniform on {emin, ..., 0}, drawn from uniform number (element / block) of exp_seed:
 * this spreads block maxima over many binades of the block-scale format. */
void syn_student_t4_bf16(uint64_t seed, double scale, int64_t count, int64_t block, uint64_t exp_seed, int emin,
                         uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    uint64_t b = 5u * (uint64_t)i;
    double z = normal_at(seed, b);
    double c = 0.0;
    for (int j = 1; j <= 4; ++j) { double v = normal_at(seed, b + (uint64_t)j); c += v * v; }
    double t = z / sqrt(c / 4.0);
    double s = scale;
    if (block > 0) {
      double u = uniform_at(exp_seed, (uint64_t)(i / block));
      int e = emin + (int)floor(u * (double)(1 - emin));
      s = ldexp(scale, e);
    }
    out[i] = f32_to_bf16_rne((float)(s * t));
  }
}

void syn_bernoulli_f32(uint64_t seed, double p, int64_t count, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = uniform_at(seed, (uint64_t)i) < p ? 1.0f : 0.0f;
}
