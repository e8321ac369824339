// synth_dev.hip -- device implementation of the synthetic input recipe in
// synth_core.h, so that multi-gigabyte gradient replicas are generated in
// HBM instead of being copied over PCIe.  Bit-identical to synth_cpu.c.
#include <hip/hip_runtime.h>

#define SYNTH_QUAL static inline __host__ __device__
#include "synth_core.h"

namespace {

template <bool kBf16>
__global__ void __launch_bounds__(256) fill_kernel(synth_prep p, uint64_t start,
                                                   uint64_t count, void* out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count;
       j += stride) {
    float x = synth_value(&p, start + j);
    if (kBf16)
      static_cast<uint16_t*>(out)[j] = synth_to_bf16(x);
    else
      static_cast<float*>(out)[j] = x;
  }
}

int launch(const synth_spec* s, uint64_t start, uint64_t count, void* out,
           hipStream_t stream, bool bf16) {
  if (s == nullptr || (out == nullptr && count != 0)) return -1;
  if (count == 0) return 0;
  synth_prep p = synth_make_prep(s);
  uint64_t blocks = (count + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (bf16)
    hipLaunchKernelGGL(fill_kernel<true>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, p, start, count, out);
  else
    hipLaunchKernelGGL(fill_kernel<false>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, p, start, count, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

extern "C" {

int synth_dev_fill_f32(const synth_spec* s, uint64_t start, uint64_t count,
                       float* out, void* stream) {
  return launch(s, start, count, out, static_cast<hipStream_t>(stream), false);
}

int synth_dev_fill_bf16(const synth_spec* s, uint64_t start, uint64_t count,
                        uint16_t* out, void* stream) {
  return launch(s, start, count, out, static_cast<hipStream_t>(stream), true);
}

}  // extern "C"
