// The C ABI's host-side argument checks under AddressSanitizer and
// UndefinedBehaviorSanitizer (built host-only with zs_abi.hip; no GPU).
// Every launcher is a stub that aborts: each call below must be rejected,
// or be a zero-length no-op, before anything is launched.  Device pointers
// are aligned or misaligned stand-ins that are never dereferenced; host
// arrays (replica pointer lists, the AdamW argument struct) are exact-size
// heap allocations, so a read past them is reported.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "zero_step.h"
#include "zs_internal.h"

namespace zs {
[[noreturn]] static void reached(const char* f) {
  std::fprintf(stderr, "a launch was reached: %s\n", f);
  std::abort();
}
hipError_t launch_reduce(const void* const*, int, int, uint64_t, float, float*, zero_norm_acc*,
                         hipStream_t, const void* const*, void*) { reached("launch_reduce"); }
hipError_t launch_adamw(const AdamLaunch&, hipStream_t) { reached("launch_adamw"); }
hipError_t launch_gate(const zero_norm_acc*, int, double, int, float*, int32_t*, hipStream_t) {
  reached("launch_gate");
}
hipError_t launch_acc_clear(zero_norm_acc*, int, hipStream_t) { reached("launch_acc_clear"); }
hipError_t launch_mxfp8(const uint16_t*, uint64_t, uint8_t*, uint8_t*, hipStream_t, const Gate*) {
  reached("launch_mxfp8");
}
uint64_t unfused_workspace_bytes(uint64_t n, int k) { return 4096 + 8 * n + 128 * k; }
hipError_t launch_unfused(const AdamLaunch&, const zero_norm_acc*, int, void*, hipStream_t) {
  reached("launch_unfused");
}
}  // namespace zs

static int failures = 0, cases = 0;
#define EXPECT(call, want)                                                        \
  do {                                                                            \
    ++cases;                                                                      \
    const int got_ = (call);                                                      \
    if (got_ != (want)) {                                                         \
      std::fprintf(stderr, "line %d: %s = %d, want %d\n", __LINE__, #call, got_, \
                   (want));                                                       \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

template <typename T>
static T* dev(uintptr_t a) { return reinterpret_cast<T*>(a); }

int main() {
  const uintptr_t A = 0x100000;                 // 16-byte aligned stand-in
  float* g = dev<float>(A + 0x1000);
  zero_norm_acc* acc = dev<zero_norm_acc>(A + 0x2000);
  void* ws = dev<void>(A + 0x3000);
  // replica pointer lists on the heap, exactly P entries
  auto reps = [&](int P, uintptr_t misalign) {
    auto* r = new std::vector<const void*>(static_cast<size_t>(P));
    for (int k = 0; k < P; ++k) (*r)[k] = dev<void>(A + 0x10000 * (k + 1) + (k == P - 1 ? misalign : 0));
    return r;
  };
  auto* r2 = reps(2, 0);
  auto* r2m = reps(2, 2);
  auto* r64 = reps(64, 0);
  const void* const* p2 = r2->data();
  EXPECT(zero_shard_reduce(nullptr, 2, ZERO_BF16, 64, 1.f, g, nullptr, nullptr), ZERO_EINVAL);
  EXPECT(zero_shard_reduce(p2, 0, ZERO_BF16, 64, 1.f, g, nullptr, nullptr), ZERO_EINVAL);
  EXPECT(zero_shard_reduce(r64->data(), 65, ZERO_BF16, 64, 1.f, g, nullptr, nullptr), ZERO_EINVAL);
  EXPECT(zero_shard_reduce(p2, 2, 7, 64, 1.f, g, nullptr, nullptr), ZERO_EINVAL);
  EXPECT(zero_shard_reduce(p2, 2, ZERO_MXFP8, 64, 1.f, g, nullptr, nullptr), ZERO_EINVAL);
  EXPECT(zero_shard_reduce(p2, 2, ZERO_BF16, 64, 1.f, nullptr, nullptr, nullptr), ZERO_EINVAL);
  EXPECT(zero_shard_reduce(p2, 2, ZERO_BF16, 64, 1.f, g + 1, nullptr, nullptr), ZERO_EALIGN);
  EXPECT(zero_shard_reduce(p2, 2, ZERO_BF16, 64, 1.f, nullptr, dev<zero_norm_acc>(A + 8), nullptr),
         ZERO_EALIGN);
  EXPECT(zero_shard_reduce(r2m->data(), 2, ZERO_BF16, 64, 1.f, g, nullptr, nullptr), ZERO_EALIGN);
  EXPECT(zero_shard_reduce(r64->data(), 64, ZERO_F32, (size_t(1) << 37) + 1, 1.f, nullptr, acc,
                           nullptr), ZERO_ESIZE);
  EXPECT(zero_shard_reduce(r64->data(), 64, ZERO_F32, 0, 1.f, g, acc, nullptr), ZERO_OK);
  EXPECT(zero_shard_reduce_ws(p2, 2, ZERO_BF16, 64, 1.f, g, acc, nullptr, 1 << 20, nullptr),
         ZERO_EINVAL);
  EXPECT(zero_shard_reduce_ws(p2, 2, ZERO_BF16, 64, 1.f, g, acc, dev<void>(A + 8), 1 << 20, nullptr),
         ZERO_EALIGN);
  EXPECT(zero_shard_reduce_ws(p2, 2, ZERO_BF16, 64, 1.f, g, acc, ws,
                              ZERO_REDUCE_WORKSPACE_BYTES - 1, nullptr), ZERO_ESIZE);
  EXPECT(zero_shard_reduce_ws(p2, 2, ZERO_BF16, 0, 1.f, g, acc, ws, ZERO_REDUCE_WORKSPACE_BYTES,
                              nullptr), ZERO_OK);
  // MXFP8-stored replicas: code and scale pointer lists, exactly P entries
  auto* sc = new std::vector<const uint8_t*>(2);
  (*sc)[0] = dev<uint8_t>(A + 1);
  (*sc)[1] = dev<uint8_t>(A + 3);
  const auto* codes = reinterpret_cast<const uint8_t* const*>(p2);
  EXPECT(zero_shard_reduce_mx(codes, sc->data(), 2, 48, 1.f, g, nullptr, nullptr), ZERO_ESIZE);
  EXPECT(zero_shard_reduce_mx(nullptr, sc->data(), 2, 64, 1.f, g, nullptr, nullptr), ZERO_EINVAL);
  EXPECT(zero_shard_reduce_mx(codes, sc->data(), 2, (size_t(1) << 37) + 32, 1.f, nullptr, acc,
                              nullptr), ZERO_ESIZE);
  EXPECT(zero_shard_reduce_mx(reinterpret_cast<const uint8_t* const*>(r2m->data()), sc->data(), 2,
                              64, 1.f, g, nullptr, nullptr), ZERO_EALIGN);
  EXPECT(zero_shard_reduce_mx(codes, sc->data(), 2, 0, 1.f, g, nullptr, nullptr), ZERO_OK);
  EXPECT(zero_shard_reduce_mx_ws(codes, sc->data(), 2, 64, 1.f, g, nullptr, nullptr, 1 << 20,
                                 nullptr), ZERO_EINVAL);
  EXPECT(zero_shard_reduce_mx_ws(codes, sc->data(), 2, 64, 1.f, g, nullptr, ws, 64, nullptr),
         ZERO_ESIZE);
  EXPECT(zero_grad_norm(nullptr, ZERO_BF16, 64, 1.f, acc, nullptr), ZERO_EINVAL);
  EXPECT(zero_grad_norm(g, ZERO_BF16, 64, 1.f, nullptr, nullptr), ZERO_EINVAL);
  EXPECT(zero_grad_norm(g, 9, 64, 1.f, acc, nullptr), ZERO_EINVAL);
  EXPECT(zero_grad_norm(g, ZERO_F32, 64, 1.f, dev<zero_norm_acc>(A + 4), nullptr), ZERO_EALIGN);
  EXPECT(zero_grad_norm(g, ZERO_F32, (size_t(1) << 37) + 1, 1.f, acc, nullptr), ZERO_ESIZE);
  EXPECT(zero_grad_norm(g, ZERO_F32, 0, 1.f, acc, nullptr), ZERO_OK);
  EXPECT(zero_mxfp8_pack(dev<uint16_t>(A), 33, dev<uint8_t>(A), dev<uint8_t>(A), nullptr),
         ZERO_ESIZE);
  EXPECT(zero_mxfp8_pack(nullptr, 64, dev<uint8_t>(A), dev<uint8_t>(A), nullptr), ZERO_EINVAL);
  EXPECT(zero_mxfp8_pack(dev<uint16_t>(A), 64, dev<uint8_t>(A), dev<uint8_t>(A + 1), nullptr),
         ZERO_EALIGN);
  EXPECT(zero_mxfp8_pack(dev<uint16_t>(A), 0, nullptr, nullptr, nullptr), ZERO_OK);
  EXPECT(zero_norm_acc_clear(nullptr, 1, nullptr), ZERO_EINVAL);
  EXPECT(zero_norm_acc_clear(acc, -1, nullptr), ZERO_EINVAL);
  EXPECT(zero_norm_acc_clear(dev<zero_norm_acc>(A + 8), 1, nullptr), ZERO_EALIGN);
  EXPECT(zero_norm_acc_clear(nullptr, 0, nullptr), ZERO_OK);
  EXPECT(zero_step_gate(acc, 1, 1.0, 1, nullptr, dev<int32_t>(A), nullptr), ZERO_EINVAL);
  EXPECT(zero_step_gate(nullptr, 2, 1.0, 1, g, dev<int32_t>(A), nullptr), ZERO_EINVAL);
  EXPECT(zero_step_gate(acc, 1, 1.0, 1, dev<float>(A + 2), dev<int32_t>(A), nullptr), ZERO_EALIGN);
  EXPECT(zero_step_gate(dev<zero_norm_acc>(A + 8), 1, 1.0, 1, g, dev<int32_t>(A), nullptr),
         ZERO_EALIGN);
  // AdamW arguments: one heap struct per case
  auto adam = [&]() {
    auto* a = new zero_adamw_args{};
    a->n = 64;
    a->grad_f32 = g;
    a->master = dev<float>(A + 0x4000);
    a->m = dev<float>(A + 0x5000);
    a->v = dev<float>(A + 0x6000);
    a->lr = 1e-3; a->beta1 = 0.9; a->beta2 = 0.999; a->eps = 1e-8;
    a->step = 1;
    return a;
  };
  EXPECT(zero_adamw_step(nullptr, nullptr), ZERO_EINVAL);
  { auto* a = adam(); a->master = nullptr; EXPECT(zero_adamw_step(a, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); a->replicas = p2; a->P = 2; a->dtype = ZERO_BF16;   // two sources
    EXPECT(zero_adamw_step(a, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); a->grad_f32 = nullptr; EXPECT(zero_adamw_step(a, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); a->step = 0; EXPECT(zero_adamw_step(a, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); a->n_accs = -1; EXPECT(zero_adamw_step(a, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); a->n_accs = 2; EXPECT(zero_adamw_step(a, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); a->grad_f32 = nullptr; a->replicas = r64->data(); a->P = 65; a->dtype = 1;
    EXPECT(zero_adamw_step(a, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); a->grad_f32 = nullptr; a->replicas = r2m->data(); a->P = 2; a->dtype = 1;
    EXPECT(zero_adamw_step(a, nullptr), ZERO_EALIGN); delete a; }
  { auto* a = adam(); a->m = dev<float>(A + 4); EXPECT(zero_adamw_step(a, nullptr), ZERO_EALIGN); delete a; }
  { auto* a = adam(); a->skipped_out = dev<int32_t>(A + 2); EXPECT(zero_adamw_step(a, nullptr), ZERO_EALIGN); delete a; }
  { auto* a = adam(); a->step_dev = dev<int64_t>(A + 4); EXPECT(zero_adamw_step(a, nullptr), ZERO_EALIGN); delete a; }
  { auto* a = adam(); a->mx_elem_out = dev<uint8_t>(A); EXPECT(zero_adamw_step(a, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); a->n = 33; a->mx_elem_out = dev<uint8_t>(A); a->mx_scale_out = dev<uint8_t>(A);
    EXPECT(zero_adamw_step(a, nullptr), ZERO_ESIZE); delete a; }
  { auto* a = adam(); a->n = 0; EXPECT(zero_adamw_step(a, nullptr), ZERO_OK); delete a; }
  { auto* a = adam(); EXPECT(zero_adamw_step_unfused(a, nullptr, 1 << 20, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); EXPECT(zero_adamw_step_unfused(a, dev<void>(A + 16), 1 << 20, nullptr), ZERO_EALIGN); delete a; }
  { auto* a = adam(); EXPECT(zero_adamw_step_unfused(a, ws, 64, nullptr), ZERO_ESIZE); delete a; }
  { auto* a = adam(); a->step_dev = dev<int64_t>(A); EXPECT(zero_adamw_step_unfused(a, ws, 1 << 20, nullptr), ZERO_EINVAL); delete a; }
  { auto* a = adam(); a->n = (size_t(1) << 37) + 1; EXPECT(zero_adamw_step_unfused(a, ws, ~size_t(0), nullptr), ZERO_ESIZE); delete a; }
  { auto* a = adam(); a->n = 0; EXPECT(zero_adamw_step_unfused(a, ws, 1 << 20, nullptr), ZERO_OK); delete a; }
  for (int s = -6; s <= 2; ++s) cases += zero_strerror(s) != nullptr;
  cases += zero_inv_scale(8, 65536.0) == 1.0f / 524288.0f;
  cases += zero_abi_version() == ZERO_ABI_VERSION;
  delete r2; delete r2m; delete r64; delete sc;
  if (failures) return 1;
  std::printf("ok: %d cases\n", cases);
  return 0;
}
