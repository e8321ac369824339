/* The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: every
 * function of oracle.h on edge inputs (every element count from 0 to 70,
 * values across the binary32 range, infinities, NaN, subnormals, the
 * largest finite value, step indices up to 2^62), each buffer an exact-size
 * heap allocation so that any read or write past it is reported.  Built by
 * the CPU test suite with gcc and the oracle's own floating-point flags. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (uint32_t)(state >> 32);
}
static float edge_value(int i) {
  static const float special[] = {0.0f, -0.0f, 1.0f, -1.0f, 1e-45f, -1e-45f, 1.17549435e-38f,
                                  3.4028235e38f, -3.4028235e38f, INFINITY, -INFINITY, NAN,
                                  4294967296.0f, 5.421011e-20f};
  const int ns = (int)(sizeof special / sizeof special[0]);
  if (i % 5 == 0) return special[(i / 5) % ns];
  uint32_t b = next32();
  float x;
  memcpy(&x, &b, 4);
  return x;
}
static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

int main(void) {
  long cases = 0;
  /* bf16 rounding over many bit patterns */
  for (uint64_t b = 0; b < (1ull << 32); b += 65521) {
    float x;
    uint32_t u = (uint32_t)b;
    memcpy(&x, &u, 4);
    (void)oracle_f32_to_bf16(x);
    ++cases;
  }
  /* scalars, including huge step indices */
  oracle_scalars s;
  const int64_t ts[] = {1, 2, 3, 1000, (int64_t)1 << 40, (int64_t)1 << 62};
  for (int k = 0; k < 6; ++k) cases += oracle_make_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, ts[k], &s) == 0;
  cases += oracle_make_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 0, &s) == -1;
  (void)oracle_pow_u(0.999, -5);
  (void)oracle_inv_scale(8, 65536.0);
  /* norm, reduce, AdamW, the gate and the whole step at every n in 0..70 */
  for (size_t n = 0; n <= 70; ++n) {
    for (int P = 1; P <= 5; P += 2) {
      for (int dtype = 0; dtype < 2; ++dtype) {
        void **reps = xmalloc(sizeof(void *) * (size_t)P);
        for (int k = 0; k < P; ++k) {
          if (dtype == ORACLE_F32) {
            float *r = xmalloc(4 * n);
            for (size_t i = 0; i < n; ++i) r[i] = edge_value((int)(i + 7 * k));
            reps[k] = r;
          } else {
            uint16_t *r = xmalloc(2 * n);
            for (size_t i = 0; i < n; ++i) r[i] = (uint16_t)next32();
            reps[k] = r;
          }
        }
        float *g = xmalloc(4 * n), *master = xmalloc(4 * n), *m = xmalloc(4 * n),
              *v = xmalloc(4 * n);
        uint16_t *param = xmalloc(2 * n);
        for (size_t i = 0; i < n; ++i) {
          master[i] = edge_value((int)i);
          m[i] = 0.0f;
          v[i] = 0.0f;
        }
        oracle_reduce((const void *const *)reps, P, dtype, n, 0.5f, g);
        oracle_acc acc, other;
        oracle_acc_zero(&acc);
        oracle_norm_accumulate(g, n, &acc);
        other = acc;
        oracle_acc_add(&acc, &other);
        (void)oracle_acc_sumsq(&acc);
        float coef;
        for (int check = 0; check < 2; ++check)
          for (int mx = 0; mx < 2; ++mx) (void)oracle_gate(&acc, mx ? 1.0 : 0.0, check, &coef);
        (void)oracle_clip_coef(oracle_acc_sumsq(&acc), 1.0);
        oracle_make_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 3, &s);
        oracle_adamw(n, g, 0.5f, &s, master, m, v, param);
        oracle_adamw(n, g, 1.0f, &s, master, m, v, NULL);
        oracle_acc own;
        for (int check = 0; check < 2; ++check)
          (void)oracle_step((const void *const *)reps, P, dtype, n, 0.5f, 1.0, check, 1e-3, 0.9,
                            0.999, 1e-8, 0.01, 2, &other, 1, g, master, m, v, param, &own);
        for (int k = 0; k < P; ++k) free(reps[k]);
        free(reps);
        free(g);
        free(master);
        free(m);
        free(v);
        free(param);
        ++cases;
      }
    }
  }
  /* fixed point at the extremes of its range */
  oracle_acc big;
  oracle_acc_zero(&big);
  const double S[] = {0.0, 5e-324, 2.9e-39, 1.0, 1.8446744073709552e19, 3.7053464138823652e78};
  for (int r = 0; r < 1000; ++r)
    for (int k = 0; k < 6; ++k) oracle_acc_add_fixed(&big, S[k]);
  (void)oracle_acc_sumsq(&big);
  /* MXFP8: encode every finite bf16 under every scale, pack and decode */
  for (uint32_t x = 0; x < 0x10000; ++x) {
    if ((x & 0x7F80u) == 0x7F80u) continue;
    for (int e = -127; e <= 127; e += 7) (void)oracle_mx_encode((uint16_t)x, e);
  }
  for (int c = 0; c < 256; ++c) {
    double val = oracle_e4m3_value((uint8_t)c);
    if (!isnan(val)) (void)oracle_e4m3_encode(val);
  }
  for (size_t n = 0; n <= 160; n += 16) {
    uint16_t *x = xmalloc(2 * n);
    for (size_t i = 0; i < n; ++i) x[i] = (uint16_t)next32();
    uint8_t *elem = xmalloc(n), *scale = xmalloc(n / 32);
    float *out = xmalloc(4 * n);
    const int rc = oracle_mxfp8_pack(x, n, elem, scale);
    if ((n % 32 == 0) != (rc == 0)) return 1;
    if (rc == 0 && oracle_mxfp8_decode(elem, scale, n, out) != 0) return 1;
    free(x);
    free(elem);
    free(scale);
    free(out);
    ++cases;
  }
  printf("ok: %ld cases\n", cases);
  return 0;
}
