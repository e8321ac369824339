/*
 * oracle.h -- CPU reference of one rank's sharded mixed-precision optimizer
 * step on a flat parameter vector.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the checker the device path is
 * compared against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product library never links or calls it.
 * It shares no source, header, table or helper with the device library.
 *
 * What it computes (sources):
 *   - Training state: a bf16 parameter, a bf16 gradient, an fp32 master copy
 *     and two fp32 Adam moments per weight, 16 bytes in all
 *     (Zero_From_Scratch, outline item on what is stored per weight; DeepSpeed
 *     documentation review, second paragraph on the master copy and moments).
 *   - Averaging the gradient replicas of the P data-parallel ranks gives the
 *     single-GPU result (Zero_From_Scratch, outline item on data parallel).
 *   - Each rank reduces only its own contiguous shard of the flat vector (the
 *     reduce half of reduce-scatter), and reduce-scatter followed by
 *     all-gather equals all-reduce (Zero_From_Scratch, outline item on the
 *     three collectives and their identity; item on the flat parameter
 *     vector).
 *   - AdamW: Adam moments and bias correction (Kingma & Ba, ICLR 2015) with
 *     decoupled weight decay (Loshchilov & Hutter, ICLR 2019).
 *   - MXFP8 packing: 32-element blocks of E4M3 with one shared E8M0 scale
 *     (OCP Microscaling Formats spec v1.0; Zero_From_Scratch, outline item on
 *     MXFP8 and its stored-state and wire savings).
 *
 * Numeric conventions: IEEE-754 binary32/binary64, round to nearest even,
 * denormals kept, no implicit contraction (built with -ffp-contract=off),
 * fmaf only where written.  Every loop runs in one fixed, documented order.
 */
#ifndef ZERO_ORACLE_H
#define ZERO_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* fp32 -> bf16, round to nearest even; NaN -> quiet NaN 0x7FC0 with the sign
 * kept; values past the largest bf16 round to +-inf like any IEEE format. */
uint16_t oracle_f32_to_bf16(float x);
float oracle_bf16_to_f32(uint16_t h);
void oracle_f32_to_bf16_array(const float *x, size_t n, uint16_t *out);

/* Per-step fp32 scalars of AdamW, each derived in binary64 from the binary64
 * hyperparameters and rounded once to binary32:
 *   b1 = f32(beta1), b2 = f32(beta2), omb1 = f32(1-beta1), omb2 = f32(1-beta2)
 *   beta^t by square-and-multiply over the bits of t, least significant first
 *   bc1 = 1 - beta1^t, bc2 = 1 - beta2^t
 *   step_size = f32(lr/bc1), sqrt_bc2 = f32(sqrt(bc2)),
 *   decay = f32(1 - lr*wd), eps = f32(eps).   t >= 1. */
typedef struct {
  float b1, b2, omb1, omb2, step_size, sqrt_bc2, decay, eps;
} oracle_scalars;
int oracle_make_scalars(double lr, double beta1, double beta2, double eps,
                        double wd, int64_t t, oracle_scalars *out);
double oracle_pow_u(double base, int64_t t);

/* inv_scale = f32(1 / (P * loss_scale)) computed in binary64. */
float oracle_inv_scale(int P, double loss_scale);

/* Shard reduce and average: s = r_0; s = s + r_k for k = 1..P-1 (binary32,
 * rank order), g = s * inv_scale.  replicas[k] points at rank k's copy of
 * the same n elements, dtype ORACLE_F32 or ORACLE_BF16. */
void oracle_reduce(const void *const *replicas, int P, int dtype, size_t n,
                   float inv_scale, float *g_out);

/* Exact global sum of squares.  X is a non-negative integer, the value of
 * the sum is X * 2^-128.  w[] holds X in 32-bit digits, least significant
 * first, always carry-normalised.  512 bits hold the sum of up to 2^32
 * groups, each below 2^(261+128): every finite binary32 gradient counts. */
typedef struct {
  uint32_t w[16];
  uint64_t nonfinite;
} oracle_acc;

void oracle_acc_zero(oracle_acc *acc);
void oracle_acc_add(oracle_acc *dst, const oracle_acc *src);
/* Adds floor(S * 2^128) for one finite, non-negative binary64 S < 2^262. */
void oracle_acc_add_fixed(oracle_acc *acc, double S);
/* The norm contribution of g[0..n): groups of 32 elements aligned to g[0]
 * (a short last group is padded with +0).  In a group, q_i = g_i*g_i in
 * binary64 (exact), a_j = q_{8j} + ... + q_{8j+7} summed left to right,
 * S = (a_0 + a_1) + (a_2 + a_3); non-finite g_i count in `nonfinite` and
 * give q_i = 0; floor(S * 2^128) is added to X exactly (S < 2^261 for
 * finite binary32 inputs, so no group is left out). */
void oracle_norm_accumulate(const float *g, size_t n, oracle_acc *acc);
/* RNE_binary64(X * 2^-128). */
double oracle_acc_sumsq(const oracle_acc *acc);
/* Global-norm clip coefficient of a finite norm: 1.0f if max_norm <= 0;
 * otherwise c = max_norm / (sqrt(sumsq) + 1e-6) in binary64 and
 * coef = c < 1 ? f32(c) : 1.0f. */
float oracle_clip_coef(double sumsq, double max_norm);
/* The step's gate from the global accumulator.  Returns 1 (skip: nothing is
 * written, t is not advanced) when check_overflow is set and nonfinite > 0.
 * Otherwise returns 0 and sets *coef: 1.0f when max_norm <= 0; 0.0f when
 * max_norm > 0 and nonfinite > 0 (a non-finite element makes the global
 * norm infinite, and max_norm / (inf + 1e-6) = 0); else
 * oracle_clip_coef(oracle_acc_sumsq(acc), max_norm). */
int oracle_gate(const oracle_acc *acc, double max_norm, int check_overflow,
                float *coef);

/* Fused AdamW on n elements, in place, per element in binary32:
 *   g' = g * coef
 *   m  = fmaf(b1, m, omb1 * g')
 *   v  = fmaf(b2, v, (omb2 * g') * g')
 *   d  = sqrtf(v) / sqrt_bc2 + eps
 *   u  = m / d
 *   th = th * decay                 (decoupled decay on the old weight)
 *   th = fmaf(-step_size, u, th)
 *   p  = bf16_rne(th)                (param may be NULL)          */
void oracle_adamw(size_t n, const float *g, float coef, const oracle_scalars *s,
                  float *master, float *m, float *v, uint16_t *param);

/* One whole step of one rank: reduce + average of the replicas into g_tmp
 * (caller scratch, n floats), its norm accumulator, plus `n_extra` accs of
 * the other ranks (the all-reduce of the norm state), the gate
 * (oracle_gate: a skip writes nothing and returns 1), then AdamW with
 * t = step and the gate's coefficient.  Returns 0 when applied.
 * acc_out (nullable) receives this rank's own accumulator. */
int oracle_step(const void *const *replicas, int P, int dtype, size_t n,
                float inv_scale, double max_norm, int check_overflow,
                double lr, double beta1, double beta2, double eps, double wd,
                int64_t step, const oracle_acc *extra, int n_extra,
                float *g_tmp, float *master, float *m, float *v,
                uint16_t *param, oracle_acc *acc_out);

/* MXFP8 (E4M3 elements, E8M0 scale, 32-element blocks).
 * oracle_e4m3_encode: q finite; round to nearest even on the E4M3FN grid
 * (bias 7, subnormal step 2^-9), saturating at +-448, sign kept.
 * oracle_mx_encode: the element code of bf16 x under scale exponent e_s,
 * i.e. e4m3_encode(x * 2^-e_s).
 * oracle_mxfp8_pack: n % 32 == 0; per block: any NaN/inf -> scale 0xFF and
 * every element 0x7F|sign; amax == 0 -> scale 0x00 and +-0 elements;
 * otherwise E = floor(log2 amax), e_s = clamp(E - 8, -127, 127), scale byte
 * e_s + 127, elements e4m3_encode(x * 2^-e_s).  Returns 0, or -1 when
 * n % 32 != 0. */
uint8_t oracle_e4m3_encode(double q);
uint8_t oracle_mx_encode(uint16_t x, int e_s);
void oracle_mx_encode_array(const uint16_t *x, size_t n, int e_s, uint8_t *out);
int oracle_mxfp8_pack(const uint16_t *x, size_t n, uint8_t *elem,
                      uint8_t *scale);
double oracle_e4m3_value(uint8_t code);

/* MXFP8 decode: element i of a packed vector is e4m3_value(elem[i]) *
 * 2^(scale[i/32] - 127), rounded once to binary32 (exact except where the
 * product overflows binary32); scale byte 0xFF (NaN) or a NaN code give a
 * NaN with the code's sign.  n % 32 == 0, else -1. */
int oracle_mxfp8_decode(const uint8_t *elem, const uint8_t *scale, size_t n,
                        float *out);

#ifdef __cplusplus
}
#endif
#endif
