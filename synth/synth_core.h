/*
 * synth_core.h -- seeded, counter-based synthetic inputs for the optimizer
 * step (gradient replicas and initial master weights).  Holds no arithmetic
 * of the method itself; both the CPU oracle's tests and the device tests draw
 * their inputs from this one definition, so that every element of every
 * stream can be regenerated anywhere from (spec, index) alone.
 *
 * Recipe for element i (a 64-bit global index into the flat vector):
 *   key = mix64(mix64(seed ^ 0x6A09E667F3BCC909) ^ tag),
 *         tag = cfg<<56 | stream<<48 | step<<32 | replica
 *   h   = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)          (mod 2^64)
 *   Z   = sum of the four 16-bit fields of h  - 131070       (Irwin-Hall,
 *         mean 0, standard deviation sqrt((2^32 - 1) / 3) = 37837.227...)
 *   x   = f32(Z) * scale,  scale = f32(sigma / sqrt((2^32 - 1) / 3))
 *   if outlier_threshold > 0 and low 32 bits of mix64(h ^ 0xD1B54A32D192ED03)
 *      < outlier_threshold:  x = x * outlier_mult             (binary32)
 *   x   = x * post_mul                                        (binary32)
 *   stored as binary32, or as bf16 rounded to nearest even.
 * mix64 is the SplitMix64 output function (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014).
 *
 * The including file defines SYNTH_QUAL (the function qualifiers of its
 * language) before including this header.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <math.h>
#include <stdint.h>

typedef struct {
  uint64_t seed;
  uint32_t cfg, stream, step, replica;
  double sigma;
  float outlier_mult;
  uint32_t outlier_threshold; /* floor(rate * 2^32); 0 = no outliers */
  float post_mul;
  uint32_t pad_;
} synth_spec;

/* Per-call constants derived on the host from a spec. */
typedef struct {
  uint64_t key;
  float scale;
  float outlier_mult;
  uint32_t outlier_threshold;
  float post_mul;
} synth_prep;

SYNTH_QUAL uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Host-side preparation of the per-call constants (binary64 sqrt and
 * division, rounded once to binary32). */
SYNTH_QUAL synth_prep synth_make_prep(const synth_spec *s) {
  synth_prep p;
  uint64_t tag = ((uint64_t)s->cfg << 56) | ((uint64_t)(s->stream & 0xFFu) << 48) |
                 ((uint64_t)(s->step & 0xFFFFu) << 32) | (uint64_t)s->replica;
  p.key = synth_mix64(synth_mix64(s->seed ^ 0x6A09E667F3BCC909ull) ^ tag);
  double sd = sqrt(4294967295.0 / 3.0);
  p.scale = (float)(s->sigma / sd);
  p.outlier_mult = s->outlier_mult;
  p.outlier_threshold = s->outlier_threshold;
  p.post_mul = s->post_mul;
  return p;
}

SYNTH_QUAL float synth_value(const synth_prep *p, uint64_t i) {
  uint64_t h = synth_mix64(p->key + (i + 1ull) * 0x9E3779B97F4A7C15ull);
  int32_t z = (int32_t)(h & 0xFFFFu) + (int32_t)((h >> 16) & 0xFFFFu) +
              (int32_t)((h >> 32) & 0xFFFFu) + (int32_t)((h >> 48) & 0xFFFFu) -
              131070;
  float x = (float)z * p->scale;
  if (p->outlier_threshold != 0u) {
    uint64_t h2 = synth_mix64(h ^ 0xD1B54A32D192ED03ull);
    if ((uint32_t)h2 < p->outlier_threshold) x = x * p->outlier_mult;
  }
  return x * p->post_mul;
}

/* bf16 storage of a generated value: round to nearest even on the bits. */
SYNTH_QUAL uint16_t synth_to_bf16(float x) {
  union {
    float f;
    uint32_t u;
  } b;
  b.f = x;
  if ((b.u & 0x7F800000u) == 0x7F800000u && (b.u & 0x007FFFFFu) != 0u)
    return (uint16_t)(((b.u >> 16) & 0x8000u) | 0x7FC0u);
  uint32_t r = b.u + 0x7FFFu + ((b.u >> 16) & 1u);
  return (uint16_t)(r >> 16);
}

#endif
