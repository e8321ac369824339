// zs_abi.hip -- the extern "C" entry points of libzero_step.so: argument
// checks, the per-step AdamW scalars (binary64, each rounded once to
// binary32), and the launches.  No allocation, no synchronisation, and no
// C++ exception crosses this boundary.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "zero_step.h"
#include "zs_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Elements one accumulator can take: 2^32 norm groups of 32, so that no
// digit, which receives one piece below 2^32 per group, can wrap.
constexpr size_t kMaxNormElems = size_t(1) << 37;

int status_of(hipError_t e) { return e == hipSuccess ? ZERO_OK : ZERO_EHIP; }

int check_replicas(const void* const* replicas, int P, int dtype) {
  if (replicas == nullptr || P < 1 || P > ZERO_MAX_REPLICAS) return ZERO_EINVAL;
  if (dtype != ZERO_F32 && dtype != ZERO_BF16) return ZERO_EINVAL;
  for (int k = 0; k < P; ++k) {
    if (replicas[k] == nullptr) return ZERO_EINVAL;
    if (!aligned16(replicas[k])) return ZERO_EALIGN;
  }
  return ZERO_OK;
}

int check_workspace(const void* workspace, size_t workspace_bytes) {
  if (workspace == nullptr) return ZERO_OK;
  if (!aligned16(workspace)) return ZERO_EALIGN;
  if (workspace_bytes < ZERO_REDUCE_WORKSPACE_BYTES) return ZERO_ESIZE;
  return ZERO_OK;
}

}  // namespace

extern "C" {

int zero_abi_version(void) { return ZERO_ABI_VERSION; }

const char* zero_strerror(int status) {
  switch (status) {
    case ZERO_OK: return "ok";
    case ZERO_EINVAL: return "invalid argument (null pointer, replica count, dtype, step or "
                             "gradient source)";
    case ZERO_EALIGN: return "pointer misaligned (device arrays and accumulators need 16 "
                             "bytes, int32/float outputs 4, the step counter 8)";
    case ZERO_ESIZE: return "size not supported (MXFP8 needs n % 32 == 0; a norm call takes "
                            "n <= 2^37; a reduce workspace needs ZERO_REDUCE_WORKSPACE_BYTES)";
    case ZERO_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

float zero_inv_scale(int P, double loss_scale) {
  const double denom = static_cast<double>(P) * loss_scale;
  return static_cast<float>(1.0 / denom);
}

int zero_norm_acc_clear(zero_norm_acc* accs, int n_accs, void* stream) {
  try {
    if (n_accs < 0) return ZERO_EINVAL;
    if (n_accs == 0) return ZERO_OK;
    if (accs == nullptr) return ZERO_EINVAL;
    if (!aligned16(accs)) return ZERO_EALIGN;
    return status_of(zs::launch_acc_clear(accs, n_accs, as_stream(stream)));
  } catch (...) {
    return ZERO_EHIP;
  }
}

namespace {

// The reduce with an optional workspace (the one-shot form when given).
int reduce_call(const void* const* replicas, int P, int dtype, size_t n, float inv_scale,
                float* g_out, zero_norm_acc* acc, void* workspace, size_t workspace_bytes,
                void* stream) {
  try {
    const int rc = check_replicas(replicas, P, dtype);
    if (rc != ZERO_OK) return rc;
    if (g_out == nullptr && acc == nullptr) return ZERO_EINVAL;
    if ((g_out && !aligned16(g_out)) || (acc && !aligned16(acc))) return ZERO_EALIGN;
    const int wc = check_workspace(workspace, workspace_bytes);
    if (wc != ZERO_OK) return wc;
    if (acc != nullptr && n > kMaxNormElems) return ZERO_ESIZE;
    if (n == 0) return ZERO_OK;
    return status_of(zs::launch_reduce(replicas, P, dtype, n, inv_scale, g_out, acc,
                                       as_stream(stream), nullptr, workspace));
  } catch (...) {
    return ZERO_EHIP;
  }
}

int reduce_mx_call(const uint8_t* const* codes, const uint8_t* const* scales, int P, size_t n,
                   float inv_scale, float* g_out, zero_norm_acc* acc, void* workspace,
                   size_t workspace_bytes, void* stream) {
  try {
    if (codes == nullptr || scales == nullptr || P < 1 || P > ZERO_MAX_REPLICAS)
      return ZERO_EINVAL;
    for (int k = 0; k < P; ++k) {
      if (codes[k] == nullptr || scales[k] == nullptr) return ZERO_EINVAL;
      if (!aligned16(codes[k])) return ZERO_EALIGN;
    }
    if (g_out == nullptr && acc == nullptr) return ZERO_EINVAL;
    if ((g_out && !aligned16(g_out)) || (acc && !aligned16(acc))) return ZERO_EALIGN;
    const int wc = check_workspace(workspace, workspace_bytes);
    if (wc != ZERO_OK) return wc;
    if (n % 32 != 0 || (acc != nullptr && n > kMaxNormElems)) return ZERO_ESIZE;
    if (n == 0) return ZERO_OK;
    const void* c[ZERO_MAX_REPLICAS];
    const void* sc[ZERO_MAX_REPLICAS];
    for (int k = 0; k < P; ++k) {
      c[k] = codes[k];
      sc[k] = scales[k];
    }
    return status_of(zs::launch_reduce(c, P, ZERO_MXFP8, n, inv_scale, g_out, acc,
                                       as_stream(stream), sc, workspace));
  } catch (...) {
    return ZERO_EHIP;
  }
}

}  // namespace

int zero_shard_reduce(const void* const* replicas, int P, int dtype, size_t n, float inv_scale,
                      float* g_out, zero_norm_acc* acc, void* stream) {
  return reduce_call(replicas, P, dtype, n, inv_scale, g_out, acc, nullptr, 0, stream);
}

int zero_shard_reduce_ws(const void* const* replicas, int P, int dtype, size_t n,
                         float inv_scale, float* g_out, zero_norm_acc* acc, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return ZERO_EINVAL;
  return reduce_call(replicas, P, dtype, n, inv_scale, g_out, acc, workspace, workspace_bytes,
                     stream);
}

int zero_shard_reduce_mx(const uint8_t* const* codes, const uint8_t* const* scales, int P,
                         size_t n, float inv_scale, float* g_out, zero_norm_acc* acc,
                         void* stream) {
  return reduce_mx_call(codes, scales, P, n, inv_scale, g_out, acc, nullptr, 0, stream);
}

int zero_shard_reduce_mx_ws(const uint8_t* const* codes, const uint8_t* const* scales, int P,
                            size_t n, float inv_scale, float* g_out, zero_norm_acc* acc,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return ZERO_EINVAL;
  return reduce_mx_call(codes, scales, P, n, inv_scale, g_out, acc, workspace,
                        workspace_bytes, stream);
}

int zero_grad_norm(const void* grad, int dtype, size_t n, float inv_scale, zero_norm_acc* acc,
                   void* stream) {
  try {
    if (grad == nullptr || acc == nullptr) return ZERO_EINVAL;
    const void* reps[1] = {grad};
    const int rc = check_replicas(reps, 1, dtype);
    if (rc != ZERO_OK) return rc;
    if (!aligned16(acc)) return ZERO_EALIGN;
    if (n > kMaxNormElems) return ZERO_ESIZE;
    if (n == 0) return ZERO_OK;
    return status_of(
        zs::launch_reduce(reps, 1, dtype, n, inv_scale, nullptr, acc, as_stream(stream)));
  } catch (...) {
    return ZERO_EHIP;
  }
}

}  // extern "C"

namespace {

// Shared checks of zero_adamw_args; fills the launch description.
int adamw_args_to_launch(const zero_adamw_args* a, zs::AdamLaunch& L) {
  if (a == nullptr) return ZERO_EINVAL;
  if (a->master == nullptr || a->m == nullptr || a->v == nullptr) return ZERO_EINVAL;
  if ((a->grad_f32 == nullptr) == (a->replicas == nullptr)) return ZERO_EINVAL;
  if ((a->step_dev == nullptr && a->step < 1) || a->n_accs < 0 ||
      (a->n_accs > 0 && a->accs == nullptr))
    return ZERO_EINVAL;
  if (a->replicas != nullptr) {
    const int rc = check_replicas(a->replicas, a->P, a->dtype);
    if (rc != ZERO_OK) return rc;
  }
  if (!aligned16(a->master) || !aligned16(a->m) || !aligned16(a->v) ||
      (a->grad_f32 && !aligned16(a->grad_f32)) ||
      (a->param_bf16 && !aligned16(a->param_bf16)) || (a->accs && !aligned16(a->accs)) ||
      (a->skipped_out && !aligned4(a->skipped_out)) ||
      (a->mx_elem_out && !aligned16(a->mx_elem_out)) ||
      (a->mx_scale_out && !aligned16(a->mx_scale_out)) ||
      (a->step_dev && (reinterpret_cast<uintptr_t>(a->step_dev) & 7u) != 0))
    return ZERO_EALIGN;
  if ((a->mx_elem_out == nullptr) != (a->mx_scale_out == nullptr)) return ZERO_EINVAL;
  if (a->mx_elem_out != nullptr && a->n % 32 != 0) return ZERO_ESIZE;
  L.grad = a->grad_f32;
  L.replicas = a->replicas;
  L.P = a->replicas ? a->P : 1;
  L.dtype = a->dtype;
  L.inv_scale = a->inv_scale;
  L.master = a->master;
  L.m = a->m;
  L.v = a->v;
  L.param = a->param_bf16;
  L.mx_elem = a->mx_elem_out;
  L.mx_scale = a->mx_scale_out;
  L.accs = a->n_accs > 0 ? a->accs : nullptr;
  L.n_accs = a->n_accs;
  L.max_norm = a->max_norm;
  L.check_overflow = a->check_overflow;
  L.skipped_out = a->skipped_out;
  L.n = a->n;
  L.h = zs::AdamHyper{a->lr, a->beta1, a->beta2, a->eps, a->weight_decay};
  L.step_dev = a->step_dev;
  L.s = zs::derive_adam_scalars(L.h, a->step_dev ? 1 : a->step);
  return ZERO_OK;
}

}  // namespace

extern "C" {

int zero_adamw_step(const zero_adamw_args* a, void* stream) {
  try {
    zs::AdamLaunch L;
    const int rc = adamw_args_to_launch(a, L);
    if (rc != ZERO_OK) return rc;
    if (a->n == 0 && a->skipped_out == nullptr && a->step_dev == nullptr) return ZERO_OK;
    return status_of(zs::launch_adamw(L, as_stream(stream)));
  } catch (...) {
    return ZERO_EHIP;
  }
}

size_t zero_unfused_workspace_bytes(size_t n, int n_accs) {
  return static_cast<size_t>(zs::unfused_workspace_bytes(n, n_accs < 0 ? 0 : n_accs));
}

int zero_adamw_step_unfused(const zero_adamw_args* a, void* workspace, size_t workspace_bytes,
                            void* stream) {
  try {
    zs::AdamLaunch L;
    const int rc = adamw_args_to_launch(a, L);
    if (rc != ZERO_OK) return rc;
    if (a->mx_elem_out != nullptr && a->param_bf16 == nullptr) return ZERO_EINVAL;
    if (a->step_dev != nullptr) return ZERO_EINVAL;  // the chain takes the host counter
    if (a->n > kMaxNormElems) return ZERO_ESIZE;  // the chain's own norm accumulator
    if (workspace == nullptr) return ZERO_EINVAL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ZERO_EALIGN;
    if (workspace_bytes < zs::unfused_workspace_bytes(a->n, a->n_accs)) return ZERO_ESIZE;
    if (a->n == 0) return ZERO_OK;
    return status_of(
        zs::launch_unfused(L, L.accs, L.n_accs, workspace, as_stream(stream)));
  } catch (...) {
    return ZERO_EHIP;
  }
}

int zero_step_gate(const zero_norm_acc* accs, int n_accs, double max_norm, int check_overflow,
                   float* coef_out, int32_t* skip_out, void* stream) {
  try {
    if (coef_out == nullptr || skip_out == nullptr || n_accs < 0 ||
        (n_accs > 0 && accs == nullptr))
      return ZERO_EINVAL;
    if ((accs && !aligned16(accs)) || !aligned4(coef_out) || !aligned4(skip_out))
      return ZERO_EALIGN;
    return status_of(zs::launch_gate(n_accs > 0 ? accs : nullptr, n_accs, max_norm,
                                     check_overflow, coef_out, skip_out, as_stream(stream)));
  } catch (...) {
    return ZERO_EHIP;
  }
}

int zero_mxfp8_pack(const uint16_t* bf16_in, size_t n, uint8_t* elem_out, uint8_t* scale_out,
                    void* stream) {
  try {
    if (n % 32 != 0) return ZERO_ESIZE;
    if (n == 0) return ZERO_OK;
    if (bf16_in == nullptr || elem_out == nullptr || scale_out == nullptr) return ZERO_EINVAL;
    if (!aligned16(bf16_in) || !aligned16(elem_out) || !aligned16(scale_out))
      return ZERO_EALIGN;
    return status_of(zs::launch_mxfp8(bf16_in, n, elem_out, scale_out, as_stream(stream)));
  } catch (...) {
    return ZERO_EHIP;
  }
}

}  // extern "C"
