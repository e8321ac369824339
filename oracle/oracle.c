/*
 * oracle.c -- plain scalar CPU reference of one rank's sharded
 * mixed-precision optimizer step.  TEST INFRASTRUCTURE ONLY (see oracle.h):
 * the product library never links it, and it shares no code with the device
 * path.  Written for reading, not for speed: every loop visits elements in
 * index order and every rounding is an explicit IEEE operation.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

static uint32_t f32_bits(float x) {
  uint32_t b;
  memcpy(&b, &x, 4);
  return b;
}
static float bits_f32(uint32_t b) {
  float x;
  memcpy(&x, &b, 4);
  return x;
}

/* ---------------------------------------------------------------- bf16 -- */

float oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* Round to nearest, ties to even, by comparing the exact distances to the two
 * neighbouring bf16 values (all values involved are exact in binary64). */
uint16_t oracle_f32_to_bf16(float x) {
  uint32_t bits = f32_bits(x);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
  uint32_t lo_bits = bits & 0xFFFF0000u;
  if (lo_bits == bits) return (uint16_t)(bits >> 16); /* exact, incl. inf/0 */
  uint16_t lo_mag = (uint16_t)((lo_bits >> 16) & 0x7FFFu);
  double ax = fabs((double)x);
  double lo = fabs((double)bits_f32(lo_bits));
  int ef = (int)((bits >> 23) & 0xFFu);
  /* spacing of bf16 values in this binade (8 significant bits) */
  double ulp = (ef == 0) ? ldexp(1.0, -133) : ldexp(1.0, ef - 127 - 7);
  double hi = lo + ulp; /* may be 2^128, which stands for +inf */
  double dlo = ax - lo, dhi = hi - ax;
  int up;
  if (dlo < dhi)
    up = 0;
  else if (dhi < dlo)
    up = 1;
  else
    up = (lo_mag & 1u) ? 1 : 0; /* tie: keep the even one */
  uint16_t mag = (uint16_t)(lo_mag + (up ? 1 : 0)); /* 0x7F7F+1 = inf */
  return (uint16_t)(sign | mag);
}

void oracle_f32_to_bf16_array(const float *x, size_t n, uint16_t *out) {
  for (size_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------- scalars -- */

/* base^t in binary64: walk the bits of t from the least significant one,
 * multiplying the result by the current power when the bit is set and then
 * squaring the power. */
double oracle_pow_u(double base, int64_t t) {
  double result = 1.0;
  double power = base;
  uint64_t e = (uint64_t)t;
  while (e != 0) {
    if (e & 1u) result = result * power;
    power = power * power;
    e >>= 1;
  }
  return result;
}

int oracle_make_scalars(double lr, double beta1, double beta2, double eps,
                        double wd, int64_t t, oracle_scalars *out) {
  if (t < 1 || out == NULL) return -1;
  out->b1 = (float)beta1;
  out->b2 = (float)beta2;
  out->omb1 = (float)(1.0 - beta1);
  out->omb2 = (float)(1.0 - beta2);
  double bc1 = 1.0 - oracle_pow_u(beta1, t);
  double bc2 = 1.0 - oracle_pow_u(beta2, t);
  out->step_size = (float)(lr / bc1);
  out->sqrt_bc2 = (float)sqrt(bc2);
  double lr_wd = lr * wd;
  out->decay = (float)(1.0 - lr_wd);
  out->eps = (float)eps;
  return 0;
}

float oracle_inv_scale(int P, double loss_scale) {
  double denom = (double)P * loss_scale;
  return (float)(1.0 / denom);
}

/* -------------------------------------------------------------- reduce -- */

static float load_elem(const void *base, int dtype, size_t i) {
  if (dtype == ORACLE_F32) return ((const float *)base)[i];
  return oracle_bf16_to_f32(((const uint16_t *)base)[i]);
}

void oracle_reduce(const void *const *replicas, int P, int dtype, size_t n,
                   float inv_scale, float *g_out) {
  for (size_t i = 0; i < n; ++i) {
    float s = load_elem(replicas[0], dtype, i);
    for (int k = 1; k < P; ++k) s = s + load_elem(replicas[k], dtype, i);
    g_out[i] = s * inv_scale;
  }
}

/* ---------------------------------------------------- exact sum of sq -- */

void oracle_acc_zero(oracle_acc *acc) { memset(acc, 0, sizeof(*acc)); }

#define ACC_WORDS 16 /* 512 bits */

/* X += 2^pos, pos in [0, 512). */
static void big_add_pow2(uint32_t w[ACC_WORDS], int pos) {
  int k = pos / 32;
  uint64_t carry = (uint64_t)1 << (pos % 32);
  while (carry != 0 && k < ACC_WORDS) {
    uint64_t t = (uint64_t)w[k] + carry;
    w[k] = (uint32_t)t;
    carry = t >> 32;
    ++k;
  }
}

void oracle_acc_add(oracle_acc *dst, const oracle_acc *src) {
  uint64_t carry = 0;
  for (int k = 0; k < ACC_WORDS; ++k) {
    uint64_t t = (uint64_t)dst->w[k] + src->w[k] + carry;
    dst->w[k] = (uint32_t)t;
    carry = t >> 32;
  }
  dst->nonfinite += src->nonfinite;
}

void oracle_acc_add_fixed(oracle_acc *acc, double S) {
  if (S == 0.0) return;
  /* S = f * 2^e with f in [0.5, 1); f * 2^53 is an integer below 2^53, so
   * S * 2^128 = mant * 2^(e - 53 + 128).  Add each set bit of mant whose
   * weight is at least 2^0; lower bits are the discarded fraction (floor). */
  int e;
  double f = frexp(S, &e);
  uint64_t mant = (uint64_t)ldexp(f, 53);
  int shift = e - 53 + 128;
  for (int b = 0; b < 53; ++b) {
    if ((mant >> b) & 1u) {
      int pos = b + shift;
      if (pos >= 0) big_add_pow2(acc->w, pos);
    }
  }
}

void oracle_norm_accumulate(const float *g, size_t n, oracle_acc *acc) {
  for (size_t gs = 0; gs < n; gs += 32) {
    double a[4];
    for (int j = 0; j < 4; ++j) {
      double sum = 0.0;
      for (int t = 0; t < 8; ++t) {
        size_t i = gs + (size_t)(8 * j + t);
        double q = 0.0;
        if (i < n) {
          float x = g[i];
          if (isfinite(x)) {
            double xd = (double)x;
            q = xd * xd; /* exact: 24-bit significand squared */
          } else {
            acc->nonfinite += 1;
          }
        }
        sum = sum + q;
      }
      a[j] = sum;
    }
    double S = (a[0] + a[1]) + (a[2] + a[3]);
    oracle_acc_add_fixed(acc, S);
  }
}

static int big_bit(const uint32_t w[ACC_WORDS], int pos) {
  if (pos < 0) return 0;
  return (int)((w[pos / 32] >> (pos % 32)) & 1u);
}

double oracle_acc_sumsq(const oracle_acc *acc) {
  int top = -1;
  for (int pos = 32 * ACC_WORDS - 1; pos >= 0; --pos) {
    if (big_bit(acc->w, pos)) {
      top = pos;
      break;
    }
  }
  if (top < 0) return 0.0;
  /* 53 significant bits from the top, then the rounding bit and the sticky
   * OR of everything below it. */
  uint64_t mant = 0;
  for (int b = 0; b < 53; ++b) mant = (mant << 1) | (uint64_t)big_bit(acc->w, top - b);
  int round_bit = big_bit(acc->w, top - 53);
  int sticky = 0;
  for (int pos = top - 54; pos >= 0; --pos) sticky |= big_bit(acc->w, pos);
  int exp2 = top - 52; /* value = mant * 2^exp2 before rounding */
  if (round_bit && (sticky || (mant & 1u))) {
    mant += 1;
    if (mant == ((uint64_t)1 << 53)) {
      mant >>= 1;
      exp2 += 1;
    }
  }
  return ldexp((double)mant, exp2 - 128);
}

float oracle_clip_coef(double sumsq, double max_norm) {
  if (!(max_norm > 0.0)) return 1.0f;
  double norm = sqrt(sumsq);
  double denom = norm + 1e-6;
  double c = max_norm / denom;
  return (c < 1.0) ? (float)c : 1.0f;
}

int oracle_gate(const oracle_acc *acc, double max_norm, int check_overflow,
                float *coef) {
  *coef = 1.0f;
  if (check_overflow && acc->nonfinite > 0) return 1;
  if (max_norm > 0.0) {
    if (acc->nonfinite > 0)
      *coef = 0.0f;
    else
      *coef = oracle_clip_coef(oracle_acc_sumsq(acc), max_norm);
  }
  return 0;
}

/* --------------------------------------------------------------- AdamW -- */

void oracle_adamw(size_t n, const float *g, float coef, const oracle_scalars *s,
                  float *master, float *m, float *v, uint16_t *param) {
  for (size_t i = 0; i < n; ++i) {
    float gc = g[i] * coef;
    float t1 = s->omb1 * gc;
    float mi = fmaf(s->b1, m[i], t1);
    float t2 = s->omb2 * gc;
    float t3 = t2 * gc;
    float vi = fmaf(s->b2, v[i], t3);
    float root = sqrtf(vi);
    float d = root / s->sqrt_bc2;
    d = d + s->eps;
    float u = mi / d;
    float th = master[i] * s->decay;
    th = fmaf(-s->step_size, u, th);
    master[i] = th;
    m[i] = mi;
    v[i] = vi;
    if (param) param[i] = oracle_f32_to_bf16(th);
  }
}

int oracle_step(const void *const *replicas, int P, int dtype, size_t n,
                float inv_scale, double max_norm, int check_overflow,
                double lr, double beta1, double beta2, double eps, double wd,
                int64_t step, const oracle_acc *extra, int n_extra,
                float *g_tmp, float *master, float *m, float *v,
                uint16_t *param, oracle_acc *acc_out) {
  oracle_acc own, global;
  oracle_acc_zero(&own);
  oracle_reduce(replicas, P, dtype, n, inv_scale, g_tmp);
  oracle_norm_accumulate(g_tmp, n, &own);
  if (acc_out) *acc_out = own;
  global = own;
  for (int k = 0; k < n_extra; ++k) oracle_acc_add(&global, &extra[k]);
  float coef;
  if (oracle_gate(&global, max_norm, check_overflow, &coef)) return 1;
  oracle_scalars s;
  oracle_make_scalars(lr, beta1, beta2, eps, wd, step, &s);
  oracle_adamw(n, g_tmp, coef, &s, master, m, v, param);
  return 0;
}

/* -------------------------------------------------------------- MXFP8 -- */

/* Round a non-negative binary64 to the nearest integer, ties to even. */
static double rne_int(double y) {
  double k = floor(y);
  double frac = y - k; /* exact for the magnitudes used here */
  if (frac > 0.5) return k + 1.0;
  if (frac < 0.5) return k;
  return (fmod(k, 2.0) == 0.0) ? k : k + 1.0;
}

uint8_t oracle_e4m3_encode(double q) {
  uint8_t sign = signbit(q) ? 0x80 : 0x00;
  double a = fabs(q);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E); /* saturate */
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest normal,
     * whose code is also 8 */
    double k = rne_int(ldexp(a, 9));
    return (uint8_t)(sign | (uint8_t)k);
  }
  int e;
  (void)frexp(a, &e);
  int E = e - 1; /* a in [2^E, 2^(E+1)), E in [-6, 8] */
  double k = rne_int(ldexp(a, 3 - E)); /* in [8, 16] */
  if (k == 16.0) {
    k = 8.0;
    E += 1;
  }
  int code = ((E + 7) << 3) | ((int)k - 8);
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

static double bf16_value(uint16_t x) { return (double)oracle_bf16_to_f32(x); }

uint8_t oracle_mx_encode(uint16_t x, int e_s) {
  return oracle_e4m3_encode(ldexp(bf16_value(x), -e_s));
}

void oracle_mx_encode_array(const uint16_t *x, size_t n, int e_s, uint8_t *out) {
  for (size_t i = 0; i < n; ++i) out[i] = oracle_mx_encode(x[i], e_s);
}

int oracle_mxfp8_pack(const uint16_t *x, size_t n, uint8_t *elem,
                      uint8_t *scale) {
  if (n % 32 != 0) return -1;
  for (size_t b = 0; b < n / 32; ++b) {
    const uint16_t *blk = x + 32 * b;
    int special = 0;
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) {
      double val = bf16_value(blk[i]);
      if (!isfinite(val))
        special = 1;
      else if (fabs(val) > amax)
        amax = fabs(val);
    }
    if (special) {
      scale[b] = 0xFF;
      for (int i = 0; i < 32; ++i)
        elem[32 * b + i] = (uint8_t)(((blk[i] & 0x8000u) ? 0x80 : 0x00) | 0x7F);
      continue;
    }
    if (amax == 0.0) {
      scale[b] = 0x00;
      for (int i = 0; i < 32; ++i)
        elem[32 * b + i] = (uint8_t)((blk[i] & 0x8000u) ? 0x80 : 0x00);
      continue;
    }
    int e;
    (void)frexp(amax, &e);
    int E = e - 1;
    int e_s = E - 8;
    if (e_s < -127) e_s = -127;
    if (e_s > 127) e_s = 127;
    scale[b] = (uint8_t)(e_s + 127);
    for (int i = 0; i < 32; ++i) elem[32 * b + i] = oracle_mx_encode(blk[i], e_s);
  }
  return 0;
}

double oracle_e4m3_value(uint8_t code) {
  double sign = (code & 0x80) ? -1.0 : 1.0;
  int ex = (code >> 3) & 0xF;
  int mt = code & 7;
  if (ex == 0xF && mt == 7) return NAN;
  if (ex == 0) return sign * ldexp((double)mt, -9);
  return sign * ldexp(8.0 + mt, ex - 7 - 3);
}

int oracle_mxfp8_decode(const uint8_t *elem, const uint8_t *scale, size_t n,
                        float *out) {
  if (n % 32 != 0) return -1;
  for (size_t i = 0; i < n; ++i) {
    uint8_t code = elem[i];
    uint8_t sb = scale[i / 32];
    double val = oracle_e4m3_value(code);
    if (sb == 0xFF || isnan(val)) {
      out[i] = (code & 0x80) ? -NAN : NAN;
      continue;
    }
    out[i] = (float)ldexp(val, (int)sb - 127);
  }
  return 0;
}
