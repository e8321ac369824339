// zs_unfused.hip -- the same optimizer step as a chain of single-operation
// passes, each a kernel of its own that reads its operands from HBM and
// writes its result back: the unfused baseline whose extra trips to memory
// the fused path removes (Zero_From_Scratch, outline item on the unfused
// chain of small operations).  Every pass performs exactly the operation the
// fused kernels perform, in the same order and binary32 rounding, so the
// results are bit for bit those of the fused path; only the traffic differs.
#include "zs_device.h"
#include "zs_internal.h"

namespace zs {

namespace {

enum UnfusedOp { kScale, kClip, kMoment1, kMoment2, kUpdateDir, kWeight, kCast };

struct UnfusedParams {
  const float* a;       // first operand
  const float* b;       // second operand (or nullptr)
  float* out;           // result (may alias a or b: same element only)
  uint16_t* out_bf16;   // kCast result
  const Gate* gate;     // coef / skip of this step (passes after the gate)
  float inv_scale;
  AdamScalars s;
  uint64_t n;
  uint64_t nchunks;
};

template <int OP>
__global__ void __launch_bounds__(kThreads) unfused_kernel(UnfusedParams prm) {
  float coef = 1.0f;
  if constexpr (OP != kScale) {
    const Gate g = *prm.gate;
    if (g.skip) return;
    coef = g.coef;
  }
  const AdamScalars sc = prm.s;
  for (uint64_t c = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; c < prm.nchunks;
       c += static_cast<uint64_t>(gridDim.x) * kThreads) {
    const bool full = c * kVec + kVec <= prm.n;
    float x[kVec], y[kVec], r[kVec];
    load_f32_chunk<false>(prm.a, c, full, prm.n, x);
    if constexpr (OP == kMoment1 || OP == kMoment2 || OP == kUpdateDir || OP == kWeight)
      load_f32_chunk<false>(prm.b, c, full, prm.n, y);
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      if constexpr (OP == kScale) r[j] = x[j] * prm.inv_scale;               // g = s * inv
      if constexpr (OP == kClip) r[j] = x[j] * coef;                         // g' = g * coef
      if constexpr (OP == kMoment1) r[j] = __builtin_fmaf(sc.b1, x[j], sc.omb1 * y[j]);
      if constexpr (OP == kMoment2)
        r[j] = __builtin_fmaf(sc.b2, x[j], (sc.omb2 * y[j]) * y[j]);
      if constexpr (OP == kUpdateDir)                                        // u = m / d
        r[j] = x[j] / (__builtin_sqrtf(y[j]) / sc.sqrt_bc2 + sc.eps);
      if constexpr (OP == kWeight)                                           // new weight
        r[j] = __builtin_fmaf(-sc.step_size, y[j], x[j] * sc.decay);
    }
    if constexpr (OP == kCast) {
      uint16_t* p = prm.out_bf16 + c * kVec;
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        if (!full && c * kVec + j >= prm.n) break;
        const uint32_t b = __float_as_uint(x[j]);
        const uint32_t rounded = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
        p[j] = static_cast<uint16_t>((b & 0x7FFFFFFFu) > 0x7F800000u
                                         ? (((b >> 16) & 0x8000u) | 0x7FC0u) : rounded);
      }
    } else {
      store_f32_chunk<false>(prm.out, c, full, prm.n, r);
    }
  }
}

// One tile per workgroup (a one-shot grid, as the fused passes use), capped
// at the dispatch limit; the kernel's grid-stride loop takes any rest.
template <int OP>
hipError_t run(const UnfusedParams& prm, hipStream_t st) {
  uint64_t blocks = (prm.nchunks + kThreads - 1) / kThreads;
  const uint64_t cap = 0xFFFFFFFFull / kThreads;
  if (blocks > cap) blocks = cap;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(unfused_kernel<OP>, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     st, prm);
  return hipGetLastError();
}

uint64_t round256(uint64_t b) { return (b + 255) / 256 * 256; }

}  // namespace

// Layout: the gate (256 B), 1 + n_other_accs accumulators, the reduce
// workspace (its slots are never touched: the chain's sum pass keeps no norm,
// but the workspace selects the one-shot reduce), then two fp32[n] buffers.
uint64_t unfused_workspace_bytes(uint64_t n, int n_other_accs) {
  return 256 + round256(static_cast<uint64_t>(1 + n_other_accs) * sizeof(zero_norm_acc)) +
         round256(ZERO_REDUCE_WORKSPACE_BYTES) + 2 * round256(n * sizeof(float));
}

hipError_t launch_unfused(const AdamLaunch& a, const zero_norm_acc* other_accs,
                          int n_other_accs, void* workspace, hipStream_t st) {
  char* ws = static_cast<char*>(workspace);
  Gate* gate = reinterpret_cast<Gate*>(ws);
  zero_norm_acc* accs = reinterpret_cast<zero_norm_acc*>(ws + 256);
  char* reduce_ws =
      ws + 256 + round256(static_cast<uint64_t>(1 + n_other_accs) * sizeof(zero_norm_acc));
  float* ws0 = reinterpret_cast<float*>(reduce_ws + round256(ZERO_REDUCE_WORKSPACE_BYTES));
  float* ws1 = ws0 + round256(a.n * sizeof(float)) / sizeof(float);
  hipError_t e;
  UnfusedParams prm{};
  prm.n = a.n;
  prm.nchunks = (a.n + kVec - 1) / kVec;
  prm.s = a.s;
  prm.gate = gate;
  const float* g = a.grad;
  if (a.replicas != nullptr) {
    // pass 1: s = r_0 + ... + r_{P-1};  pass 2: g = s * inv_scale
    if ((e = launch_reduce(a.replicas, a.P, a.dtype, a.n, 1.0f, ws0, nullptr, st, nullptr,
                           reduce_ws)) != hipSuccess)
      return e;
    prm.a = ws0;
    prm.out = ws1;
    prm.inv_scale = a.inv_scale;
    if ((e = run<kScale>(prm, st)) != hipSuccess) return e;
    g = ws1;
  }
  // pass 3: the norm state of g (g * 1.0 is g exactly); then the gate
  if ((e = launch_acc_clear(accs, 1, st)) != hipSuccess) return e;
  const void* gsrc[1] = {g};
  if ((e = launch_reduce(gsrc, 1, ZERO_F32, a.n, 1.0f, nullptr, accs, st)) != hipSuccess) return e;
  if (n_other_accs > 0 &&
      (e = hipMemcpyAsync(accs + 1, other_accs, n_other_accs * sizeof(zero_norm_acc),
                          hipMemcpyDeviceToDevice, st)) != hipSuccess)
    return e;
  if ((e = launch_gate(accs, 1 + n_other_accs, a.max_norm, a.check_overflow, &gate->coef,
                       &gate->skip, st)) != hipSuccess)
    return e;
  if (a.skipped_out != nullptr &&
      (e = hipMemcpyAsync(a.skipped_out, &gate->skip, sizeof(int32_t), hipMemcpyDeviceToDevice,
                          st)) != hipSuccess)
    return e;
  // pass 4: g' = g * coef
  prm.a = g;
  prm.out = ws0;
  if ((e = run<kClip>(prm, st)) != hipSuccess) return e;
  // pass 5: m;  pass 6: v
  prm.a = a.m;
  prm.b = ws0;
  prm.out = a.m;
  if ((e = run<kMoment1>(prm, st)) != hipSuccess) return e;
  prm.a = a.v;
  prm.out = a.v;
  if ((e = run<kMoment2>(prm, st)) != hipSuccess) return e;
  // pass 7: u = m / (sqrt(v) / sqrt_bc2 + eps)
  prm.a = a.m;
  prm.b = a.v;
  prm.out = ws1;
  if ((e = run<kUpdateDir>(prm, st)) != hipSuccess) return e;
  // pass 8: master = fma(-step_size, u, master * decay)
  prm.a = a.master;
  prm.b = ws1;
  prm.out = a.master;
  if ((e = run<kWeight>(prm, st)) != hipSuccess) return e;
  // pass 9: the bf16 param;  pass 10: its MXFP8 pack
  if (a.param != nullptr) {
    prm.a = a.master;
    prm.out_bf16 = a.param;
    if ((e = run<kCast>(prm, st)) != hipSuccess) return e;
    if (a.mx_elem != nullptr) {
      // the pack pass reads the same gate: a skipped step writes nothing
      if ((e = launch_mxfp8(a.param, a.n, a.mx_elem, a.mx_scale, st, gate)) != hipSuccess)
        return e;
    }
  }
  return hipSuccess;
}

}  // namespace zs
