/* synth_cpu.c -- host implementation of the synthetic input recipe in
 * synth_core.h.  Plain loops; callers split large ranges across threads. */
#define SYNTH_QUAL static inline
#include "synth_core.h"

#include <stddef.h>

static synth_prep prep(const synth_spec *s) { return synth_make_prep(s); }

void synth_fill_f32(const synth_spec *s, uint64_t start, size_t count, float *out) {
  synth_prep p = prep(s);
  for (size_t j = 0; j < count; ++j) out[j] = synth_value(&p, start + j);
}

void synth_fill_bf16(const synth_spec *s, uint64_t start, size_t count,
                     uint16_t *out) {
  synth_prep p = prep(s);
  for (size_t j = 0; j < count; ++j) out[j] = synth_to_bf16(synth_value(&p, start + j));
}

void synth_gather_f32(const synth_spec *s, const uint64_t *idx, size_t count,
                      float *out) {
  synth_prep p = prep(s);
  for (size_t j = 0; j < count; ++j) out[j] = synth_value(&p, idx[j]);
}

void synth_gather_bf16(const synth_spec *s, const uint64_t *idx, size_t count,
                       uint16_t *out) {
  synth_prep p = prep(s);
  for (size_t j = 0; j < count; ++j) out[j] = synth_to_bf16(synth_value(&p, idx[j]));
}
