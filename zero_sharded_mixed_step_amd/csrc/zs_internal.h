// zs_internal.h -- launchers between the C ABI (zs_abi.hip) and the kernels
// (zs_kernels.hip).  Arguments arrive validated; launchers only pick the
// template instance and the grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_step.h"

namespace zs {

struct AdamScalars {
  float b1, b2, omb1, omb2, step_size, sqrt_bc2, decay, eps;
};

// The AdamW hyperparameters as the caller gives them (binary64).
struct AdamHyper {
  double lr, beta1, beta2, eps, wd;
};

// beta^t by square-and-multiply over the bits of t, least significant bit
// first, in binary64 (the fixed evaluation order of the step's scalars).
__host__ __device__ inline double power_lsb_first(double beta, int64_t t) {
  double acc = 1.0;
  double sq = beta;
  for (uint64_t e = static_cast<uint64_t>(t); e != 0; e >>= 1) {
    if (e & 1u) acc = acc * sq;
    sq = sq * sq;
  }
  return acc;
}

// The per-step binary32 scalars of update t, each computed in binary64 and
// rounded once.  Host and device evaluate the same correctly rounded binary64
// operations (+, -, *, /, sqrt; nothing contracted), so both give the same
// bits: the device derives them itself when the step counter lives in device
// memory.
__host__ __device__ inline AdamScalars derive_adam_scalars(const AdamHyper& h, int64_t t) {
  AdamScalars s;
  s.b1 = static_cast<float>(h.beta1);
  s.b2 = static_cast<float>(h.beta2);
  s.omb1 = static_cast<float>(1.0 - h.beta1);
  s.omb2 = static_cast<float>(1.0 - h.beta2);
  const double bias1 = 1.0 - power_lsb_first(h.beta1, t);
  const double bias2 = 1.0 - power_lsb_first(h.beta2, t);
  s.step_size = static_cast<float>(h.lr / bias1);
  s.sqrt_bc2 = static_cast<float>(__builtin_sqrt(bias2));
  const double lw = h.lr * h.wd;
  s.decay = static_cast<float>(1.0 - lw);
  s.eps = static_cast<float>(h.eps);
  return s;
}

// Workgroups (of 256 threads) per compute unit of the reduce pass's
// persistent grid, from sweeps of 1..10 on MI355X: it needs 4 to keep enough
// loads in flight, except for bucket-sized launches with 4 or 8 replicas,
// whose software-pipelined fast path holds twice the loads per lane and runs
// best at 1.  (Without a workspace the reduce stays persistent: each
// workgroup ends with atomic adds to the one norm accumulator, which a
// one-shot grid would multiply.  AdamW and the pack launch one-shot grids.)
#ifndef ZS_REDUCE_BLOCKS_PER_CU
#define ZS_REDUCE_BLOCKS_PER_CU 4
#endif
#ifndef ZS_REDUCE_PIPE_BLOCKS_PER_CU
#define ZS_REDUCE_PIPE_BLOCKS_PER_CU 1
#endif

int compute_units(int device);

// dtype ZERO_MXFP8: replicas are the code arrays and mx_scales the scales.
hipError_t launch_reduce(const void* const* replicas, int P, int dtype, uint64_t n,
                         float inv_scale, float* g_out, zero_norm_acc* acc,
                         hipStream_t stream, const void* const* mx_scales = nullptr,
                         void* workspace = nullptr);

struct AdamLaunch {
  const float* grad;
  const void* const* replicas;
  int P;
  int dtype;
  float inv_scale;
  float* master;
  float* m;
  float* v;
  uint16_t* param;
  uint8_t* mx_elem;
  uint8_t* mx_scale;
  const zero_norm_acc* accs;
  int n_accs;
  double max_norm;
  int check_overflow;
  int32_t* skipped_out;
  uint64_t n;
  AdamScalars s;         // update `step` (host counter)
  AdamHyper h;
  int64_t* step_dev;     // or: the device counter of applied updates
};

hipError_t launch_adamw(const AdamLaunch& a, hipStream_t stream);

hipError_t launch_gate(const zero_norm_acc* accs, int n_accs, double max_norm,
                       int check_overflow, float* coef_out, int32_t* skip_out,
                       hipStream_t stream);

hipError_t launch_acc_clear(zero_norm_acc* accs, int n_accs, hipStream_t stream);

struct Gate;
hipError_t launch_mxfp8(const uint16_t* in, uint64_t n, uint8_t* elem, uint8_t* scale,
                        hipStream_t stream, const Gate* gate = nullptr);

// The unfused chain (zs_unfused.hip): the step as single-operation passes.
uint64_t unfused_workspace_bytes(uint64_t n, int n_other_accs);
hipError_t launch_unfused(const AdamLaunch& a, const zero_norm_acc* other_accs,
                          int n_other_accs, void* workspace, hipStream_t stream);

}  // namespace zs
