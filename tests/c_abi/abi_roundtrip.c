/* abi_roundtrip.c -- a C program that drives libzero_step.so through its C
 * ABI alone (no Python): seeded bf16 gradient replicas and fp32 master
 * weights from the shared input generator, three gated steps on the GPU
 * (accumulator clear, shard reduce with the norm state, AdamW with the bf16
 * param and the fused MXFP8 pack, the skip flag), every output copied back
 * and compared bit for bit with the CPU oracle's step; then the ABI's
 * argument checks.  Test infrastructure: it links the oracle.  Prints one
 * line and exits 0 when everything matches. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"
#include "zero_step.h"

#define SYNTH_QUAL static inline
#include "synth_core.h"

void synth_fill_f32(const synth_spec *s, uint64_t start, size_t count, float *out);
void synth_fill_bf16(const synth_spec *s, uint64_t start, size_t count, uint16_t *out);

#define P 4
#define STEPS 3

static int failures = 0;

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));              \
      exit(2);                                                                \
    }                                                                         \
  } while (0)

#define ZERO_OK_CALL(call)                                                    \
  do {                                                                        \
    int s_ = (call);                                                          \
    if (s_ != ZERO_OK) {                                                      \
      fprintf(stderr, "%s: %s (%d)\n", #call, zero_strerror(s_), s_);         \
      exit(3);                                                                \
    }                                                                         \
  } while (0)

static void expect_status(const char *what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d\n", what, got, zero_strerror(got), want);
    ++failures;
  }
}

static void compare(const char *what, const void *got, const void *want, size_t bytes,
                    size_t elem) {
  if (memcmp(got, want, bytes) != 0) {
    size_t bad = 0, first = (size_t)-1;
    for (size_t i = 0; i < bytes / elem; ++i)
      if (memcmp((const char *)got + i * elem, (const char *)want + i * elem, elem) != 0) {
        if (first == (size_t)-1) first = i;
        ++bad;
      }
    fprintf(stderr, "%s: %zu of %zu elements differ (first at %zu)\n", what, bad,
            bytes / elem, first);
    ++failures;
  }
}

static synth_spec spec(uint32_t stream, uint32_t step, uint32_t replica, double sigma,
                       double outlier_rate) {
  synth_spec s;
  memset(&s, 0, sizeof s);
  s.seed = 11;
  s.cfg = 90;
  s.stream = stream;
  s.step = step;
  s.replica = replica;
  s.sigma = sigma;
  s.outlier_mult = outlier_rate > 0 ? 100.0f : 1.0f;
  s.outlier_threshold = outlier_rate > 0 ? (uint32_t)(outlier_rate * 4294967296.0) : 0u;
  s.post_mul = 1.0f;
  return s;
}

int main(void) {
  const size_t n = 3 * 2048 + 96; /* several tiles and a ragged tail; n % 32 == 0 */
  const double lr = 1e-3, b1 = 0.9, b2 = 0.999, eps = 1e-8, wd = 0.01, max_norm = 1.0;
  if (zero_abi_version() != ZERO_ABI_VERSION) {
    fprintf(stderr, "library ABI %d, header %d\n", zero_abi_version(), ZERO_ABI_VERSION);
    return 4;
  }

  /* host inputs and the oracle's state */
  uint16_t *reps_h[P];
  float *master_h = malloc(n * sizeof(float)), *m_h = calloc(n, sizeof(float)),
        *v_h = calloc(n, sizeof(float)), *g_tmp = malloc(n * sizeof(float));
  uint16_t *param_h = malloc(n * sizeof(uint16_t));
  uint8_t *elem_h = malloc(n), *scale_h = malloc(n / 32);
  for (int k = 0; k < P; ++k) reps_h[k] = malloc(n * sizeof(uint16_t));
  synth_spec ms = spec(0, 0, 0, 0.02, 0.0);
  synth_fill_f32(&ms, 0, n, master_h);
  oracle_f32_to_bf16_array(master_h, n, param_h);

  /* device buffers */
  void *reps_d[P];
  float *master_d, *m_d, *v_d, *g_d;
  uint16_t *param_d;
  uint8_t *elem_d, *scale_d;
  zero_norm_acc *acc_d;
  int32_t *skipped_d;
  for (int k = 0; k < P; ++k) HIP_OK(hipMalloc(&reps_d[k], n * sizeof(uint16_t)));
  HIP_OK(hipMalloc((void **)&master_d, n * sizeof(float)));
  HIP_OK(hipMalloc((void **)&m_d, n * sizeof(float)));
  HIP_OK(hipMalloc((void **)&v_d, n * sizeof(float)));
  HIP_OK(hipMalloc((void **)&g_d, n * sizeof(float)));
  HIP_OK(hipMalloc((void **)&param_d, n * sizeof(uint16_t)));
  HIP_OK(hipMalloc((void **)&elem_d, n));
  HIP_OK(hipMalloc((void **)&scale_d, n / 32));
  HIP_OK(hipMalloc((void **)&acc_d, sizeof(zero_norm_acc)));
  HIP_OK(hipMalloc((void **)&skipped_d, sizeof(int32_t)));
  HIP_OK(hipMemcpy(master_d, master_h, n * sizeof(float), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(param_d, param_h, n * sizeof(uint16_t), hipMemcpyHostToDevice));
  HIP_OK(hipMemset(m_d, 0, n * sizeof(float)));
  HIP_OK(hipMemset(v_d, 0, n * sizeof(float)));

  const float inv = zero_inv_scale(P, 1.0);
  if (inv != oracle_inv_scale(P, 1.0)) {
    fprintf(stderr, "zero_inv_scale differs from the oracle's\n");
    ++failures;
  }
  int64_t applied = 0;
  for (int call = 1; call <= STEPS; ++call) {
    for (int k = 0; k < P; ++k) {
      synth_spec gs = spec(1, (uint32_t)call, (uint32_t)k, 1e-3, 0.01);
      synth_fill_bf16(&gs, 0, n, reps_h[k]);
    }
    if (call == 2) reps_h[P - 1][77] = 0x7F80u; /* +inf: the overflow check skips call 2 */
    for (int k = 0; k < P; ++k)
      HIP_OK(hipMemcpy(reps_d[k], reps_h[k], n * sizeof(uint16_t), hipMemcpyHostToDevice));

    ZERO_OK_CALL(zero_norm_acc_clear(acc_d, 1, NULL));
    ZERO_OK_CALL(zero_shard_reduce((const void *const *)reps_d, P, ZERO_BF16, n, inv, g_d,
                                   acc_d, NULL));
    zero_adamw_args a;
    memset(&a, 0, sizeof a);
    a.n = n;
    a.grad_f32 = g_d;
    a.master = master_d;
    a.m = m_d;
    a.v = v_d;
    a.param_bf16 = param_d;
    a.accs = acc_d;
    a.n_accs = 1;
    a.max_norm = max_norm;
    a.check_overflow = 1;
    a.lr = lr;
    a.beta1 = b1;
    a.beta2 = b2;
    a.eps = eps;
    a.weight_decay = wd;
    a.step = applied + 1;
    a.skipped_out = skipped_d;
    a.mx_elem_out = elem_d;
    a.mx_scale_out = scale_d;
    ZERO_OK_CALL(zero_adamw_step(&a, NULL));
    HIP_OK(hipDeviceSynchronize());

    oracle_acc own;
    const int skipped = oracle_step((const void *const *)reps_h, P, ORACLE_BF16, n, inv,
                                    max_norm, 1, lr, b1, b2, eps, wd, applied + 1, NULL, 0,
                                    g_tmp, master_h, m_h, v_h, param_h, &own);
    int32_t skipped_dev = -1;
    HIP_OK(hipMemcpy(&skipped_dev, skipped_d, sizeof skipped_dev, hipMemcpyDeviceToHost));
    if (skipped_dev != skipped) {
      fprintf(stderr, "call %d: device skip %d, oracle %d\n", call, skipped_dev, skipped);
      ++failures;
    }
    if (skipped != (call == 2)) {
      fprintf(stderr, "call %d: the oracle's skip decision is %d\n", call, skipped);
      ++failures;
    }
    if (!skipped) ++applied;
  }
  oracle_mxfp8_pack(param_h, n, elem_h, scale_h);

  float *buf = malloc(n * sizeof(float));
  uint16_t *buf16 = malloc(n * sizeof(uint16_t));
  uint8_t *buf8 = malloc(n);
  HIP_OK(hipMemcpy(buf, master_d, n * sizeof(float), hipMemcpyDeviceToHost));
  compare("master", buf, master_h, n * sizeof(float), sizeof(float));
  HIP_OK(hipMemcpy(buf, m_d, n * sizeof(float), hipMemcpyDeviceToHost));
  compare("m", buf, m_h, n * sizeof(float), sizeof(float));
  HIP_OK(hipMemcpy(buf, v_d, n * sizeof(float), hipMemcpyDeviceToHost));
  compare("v", buf, v_h, n * sizeof(float), sizeof(float));
  HIP_OK(hipMemcpy(buf, g_d, n * sizeof(float), hipMemcpyDeviceToHost));
  compare("g (last call)", buf, g_tmp, n * sizeof(float), sizeof(float));
  HIP_OK(hipMemcpy(buf16, param_d, n * sizeof(uint16_t), hipMemcpyDeviceToHost));
  compare("param", buf16, param_h, n * sizeof(uint16_t), sizeof(uint16_t));
  HIP_OK(hipMemcpy(buf8, elem_d, n, hipMemcpyDeviceToHost));
  compare("mxfp8 codes", buf8, elem_h, n, 1);
  HIP_OK(hipMemcpy(buf8, scale_d, n / 32, hipMemcpyDeviceToHost));
  compare("mxfp8 scales", buf8, scale_h, n / 32, 1);

  /* the argument checks return their status without launching anything */
  expect_status("P = 0", zero_shard_reduce((const void *const *)reps_d, 0, ZERO_BF16, n, inv,
                                           g_d, acc_d, NULL), ZERO_EINVAL);
  expect_status("no outputs", zero_shard_reduce((const void *const *)reps_d, P, ZERO_BF16, n,
                                                inv, NULL, NULL, NULL), ZERO_EINVAL);
  expect_status("misaligned g", zero_shard_reduce((const void *const *)reps_d, P, ZERO_BF16, n,
                                                  inv, (float *)((char *)g_d + 4), NULL, NULL),
                ZERO_EALIGN);
  expect_status("n beyond the accumulator", zero_grad_norm(g_d, ZERO_F32,
                                                           ((size_t)1 << 37) + 32, 1.0f,
                                                           acc_d, NULL), ZERO_ESIZE);
  expect_status("pack of n % 32 != 0", zero_mxfp8_pack(param_d, 40, elem_d, scale_d, NULL),
                ZERO_ESIZE);
  expect_status("_ws without a workspace",
                zero_shard_reduce_ws((const void *const *)reps_d, P, ZERO_BF16, n, inv, g_d,
                                     acc_d, NULL, 0, NULL), ZERO_EINVAL);
  expect_status("n == 0 is a no-op", zero_shard_reduce((const void *const *)reps_d, P,
                                                       ZERO_BF16, 0, inv, g_d, acc_d, NULL),
                ZERO_OK);

  for (int k = 0; k < P; ++k) {
    HIP_OK(hipFree(reps_d[k]));
    free(reps_h[k]);
  }
  HIP_OK(hipFree(master_d));
  HIP_OK(hipFree(m_d));
  HIP_OK(hipFree(v_d));
  HIP_OK(hipFree(g_d));
  HIP_OK(hipFree(param_d));
  HIP_OK(hipFree(elem_d));
  HIP_OK(hipFree(scale_d));
  HIP_OK(hipFree(acc_d));
  HIP_OK(hipFree(skipped_d));
  free(master_h); free(m_h); free(v_h); free(g_tmp); free(param_h); free(elem_h);
  free(scale_h); free(buf); free(buf16); free(buf8);
  if (failures) {
    fprintf(stderr, "abi_roundtrip: %d failures\n", failures);
    return 1;
  }
  printf("abi_roundtrip ok: %zu elements, P=%d bf16, %d gated calls (one skipped), fused "
         "MXFP8 pack, bitwise equal to the oracle; argument checks as documented\n",
         n, P, STEPS);
  return 0;
}
