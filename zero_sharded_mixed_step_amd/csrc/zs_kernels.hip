// zs_kernels.hip -- the optimizer step's HIP kernels for CDNA4 (gfx950).
//
// All four are HBM-bandwidth-bound streaming passes (no matrix work, so no
// MFMA): 16-byte vector loads/stores per lane, a persistent grid of a few
// workgroups per compute unit striding over 2048-element tiles, and the norm
// state reduced in registers (quad DPP), lane-private LDS rows and one set
// of integer atomics per workgroup.
#include "zs_device.h"
#include "zs_internal.h"

namespace zs {

// ---------------------------------------------------------------- grid ----

static int g_cu_count[64];

int compute_units(int device) {
  if (device < 0 || device >= 64) return 256;
  int v = __atomic_load_n(&g_cu_count[device], __ATOMIC_RELAXED);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    cus = 256;
  __atomic_store_n(&g_cu_count[device], cus, __ATOMIC_RELAXED);
  return cus;
}

static unsigned grid_for(uint64_t nchunks) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const uint64_t ntiles = (nchunks + kThreads - 1) / kThreads;
  const uint64_t cap = static_cast<uint64_t>(compute_units(dev)) * ZS_BLOCKS_PER_CU;
  const uint64_t g = ntiles < cap ? ntiles : cap;
  return static_cast<unsigned>(g > 0 ? g : 1);
}

static Replicas pack_replicas(const void* const* replicas, int P) {
  Replicas R{};
  for (int k = 0; k < P; ++k) R.p[k] = replicas[k];
  return R;
}

// ------------------------------------------------------ shard reduce -----

struct ReduceParams {
  Replicas R;
  int P;
  float inv_scale;
  uint64_t n;
  uint64_t nchunks;
  float* g_out;
  zero_norm_acc* acc;
};

template <int DT, int PT, bool WRITE, bool NORM>
__global__ void __launch_bounds__(kThreads) shard_reduce_kernel(ReduceParams prm) {
  __shared__ uint64_t s_digit[NORM ? 7 : 1][kThreads];
  __shared__ uint32_t s_count[NORM ? 2 : 1][kThreads];
  const int tid = threadIdx.x;
  const int quad_lane = tid & 3;
  if constexpr (NORM) {
#pragma unroll
    for (int k = 0; k < 7; ++k) s_digit[k][tid] = 0;
  }
  uint32_t nonfinite = 0, overflow = 0;
  const uint64_t ntiles = (prm.nchunks + kThreads - 1) / kThreads;
  for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const uint64_t c = tile * kThreads + tid;
    const bool valid = c < prm.nchunks;
    const bool full = valid && (c * kVec + kVec <= prm.n);
    float g[kVec];
    if (valid) {
      reduce_chunk<DT, PT>(prm.R, prm.P, c, full, prm.n, prm.inv_scale, g);
      if (WRITE) store_f32_chunk(prm.g_out, c, full, prm.n, g);
    } else {
#pragma unroll
      for (int j = 0; j < kVec; ++j) g[j] = 0.0f;
    }
    if constexpr (NORM) {
      const double a = chunk_sumsq(g, nonfinite);
      const double S = quad_group_sum(a);  // all 64 lanes take part
      if (quad_lane == 0 && S >= 18446744073709551616.0) ++overflow;
      int d;
      uint64_t piece;
      fixed_point_piece(S, quad_lane, d, piece);
      if (piece != 0) s_digit[d][tid] += piece;  // lane-private row
    }
  }
  if constexpr (NORM) {
  s_count[0][tid] = nonfinite;
  s_count[1][tid] = overflow;
  __syncthreads();
  for (int stride = kThreads / 2; stride > 0; stride >>= 1) {
    if (tid < stride) {
#pragma unroll
      for (int k = 0; k < 7; ++k) s_digit[k][tid] += s_digit[k][tid + stride];
      s_count[0][tid] += s_count[0][tid + stride];
      s_count[1][tid] += s_count[1][tid + stride];
    }
    __syncthreads();
  }
  if (tid == 0) {
    zero_norm_acc* acc = prm.acc;
#pragma unroll
    for (int k = 0; k < 7; ++k) {
      const uint64_t v = s_digit[k][0];
      if (v != 0) atomicAdd(reinterpret_cast<unsigned long long*>(&acc->digit[k]),
                            static_cast<unsigned long long>(v));
    }
    if (s_count[0][0] != 0) atomicAdd(&acc->nonfinite, s_count[0][0]);
    if (s_count[1][0] != 0) atomicAdd(&acc->overflow, s_count[1][0]);
  }
  }
}

template <int DT, int PT>
static void reduce_dispatch_io(const ReduceParams& prm, bool write, bool norm, unsigned grid,
                               hipStream_t st) {
  if (write && norm)
    hipLaunchKernelGGL((shard_reduce_kernel<DT, PT, true, true>), dim3(grid), dim3(kThreads), 0,
                       st, prm);
  else if (write)
    hipLaunchKernelGGL((shard_reduce_kernel<DT, PT, true, false>), dim3(grid), dim3(kThreads),
                       0, st, prm);
  else
    hipLaunchKernelGGL((shard_reduce_kernel<DT, PT, false, true>), dim3(grid), dim3(kThreads),
                       0, st, prm);
}

template <int DT>
static void reduce_dispatch_p(const ReduceParams& prm, bool write, bool norm, unsigned grid,
                              hipStream_t st) {
  switch (prm.P) {
    case 1: reduce_dispatch_io<DT, 1>(prm, write, norm, grid, st); break;
    case 2: reduce_dispatch_io<DT, 2>(prm, write, norm, grid, st); break;
    case 4: reduce_dispatch_io<DT, 4>(prm, write, norm, grid, st); break;
    case 8: reduce_dispatch_io<DT, 8>(prm, write, norm, grid, st); break;
    default: reduce_dispatch_io<DT, 0>(prm, write, norm, grid, st); break;
  }
}

hipError_t launch_reduce(const void* const* replicas, int P, int dtype, uint64_t n,
                         float inv_scale, float* g_out, zero_norm_acc* acc,
                         hipStream_t stream) {
  ReduceParams prm;
  prm.R = pack_replicas(replicas, P);
  prm.P = P;
  prm.inv_scale = inv_scale;
  prm.n = n;
  prm.nchunks = (n + kVec - 1) / kVec;
  prm.g_out = g_out;
  prm.acc = acc;
  const unsigned grid = grid_for(prm.nchunks);
  if (dtype == ZERO_BF16)
    reduce_dispatch_p<ZERO_BF16>(prm, g_out != nullptr, acc != nullptr, grid, stream);
  else
    reduce_dispatch_p<ZERO_F32>(prm, g_out != nullptr, acc != nullptr, grid, stream);
  return hipGetLastError();
}

// -------------------------------------------------------------- AdamW ----

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return ((b >> 16) & 0x8000u) | 0x7FC0u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

struct AdamParams {
  Replicas R;
  int P;
  float inv_scale;
  const float* grad;
  float* master;
  float* m;
  float* v;
  uint16_t* param;
  const zero_norm_acc* accs;
  int n_accs;
  int check_overflow;
  double max_norm;
  int32_t* skipped_out;
  uint64_t n;
  uint64_t nchunks;
  AdamScalars s;
};

// SRC < 0: gradient from prm.grad (fp32); otherwise the replica dtype.
template <int SRC, int PT, bool PARAM>
__global__ void __launch_bounds__(kThreads) adamw_kernel(AdamParams prm) {
  __shared__ Gate s_gate;
  if (threadIdx.x == 0) {
    const Gate gt = evaluate_gate(prm.accs, prm.n_accs, prm.max_norm, prm.check_overflow);
    s_gate = gt;
    if (blockIdx.x == 0 && prm.skipped_out != nullptr) *prm.skipped_out = gt.skip;
  }
  __syncthreads();
  const Gate gt = s_gate;
  if (gt.skip) return;
  const float coef = gt.coef;
  const AdamScalars sc = prm.s;
  const float neg_step = -sc.step_size;
  const uint64_t ntiles = (prm.nchunks + kThreads - 1) / kThreads;
  for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const uint64_t c = tile * kThreads + threadIdx.x;
    if (c >= prm.nchunks) break;
    const bool full = c * kVec + kVec <= prm.n;
    float g[kVec], th[kVec], mm[kVec], vv[kVec];
    if constexpr (SRC < 0)
      load_f32_chunk(prm.grad, c, full, prm.n, g);
    else
      reduce_chunk<SRC, PT>(prm.R, prm.P, c, full, prm.n, prm.inv_scale, g);
    load_f32_chunk(prm.master, c, full, prm.n, th);
    load_f32_chunk(prm.m, c, full, prm.n, mm);
    load_f32_chunk(prm.v, c, full, prm.n, vv);
    uint32_t pb[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const float gc = g[j] * coef;
      const float mi = __builtin_fmaf(sc.b1, mm[j], sc.omb1 * gc);
      const float vi = __builtin_fmaf(sc.b2, vv[j], (sc.omb2 * gc) * gc);
      const float d = __builtin_sqrtf(vi) / sc.sqrt_bc2 + sc.eps;
      const float u = mi / d;
      const float t = __builtin_fmaf(neg_step, u, th[j] * sc.decay);
      th[j] = t;
      mm[j] = mi;
      vv[j] = vi;
      pb[j] = bf16_rne_bits(t);
    }
    store_f32_chunk(prm.master, c, full, prm.n, th);
    store_f32_chunk(prm.m, c, full, prm.n, mm);
    store_f32_chunk(prm.v, c, full, prm.n, vv);
    if (PARAM) {
      uint16_t* p = prm.param + c * kVec;
      if (full) {
        *reinterpret_cast<uint4*>(p) =
            make_uint4(pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16), pb[4] | (pb[5] << 16),
                       pb[6] | (pb[7] << 16));
      } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j)
          if (c * kVec + j < prm.n) p[j] = static_cast<uint16_t>(pb[j]);
      }
    }
  }
}

template <int SRC, int PT>
static void adamw_dispatch_param(const AdamParams& prm, unsigned grid, hipStream_t st) {
  if (prm.param != nullptr)
    hipLaunchKernelGGL((adamw_kernel<SRC, PT, true>), dim3(grid), dim3(kThreads), 0, st, prm);
  else
    hipLaunchKernelGGL((adamw_kernel<SRC, PT, false>), dim3(grid), dim3(kThreads), 0, st, prm);
}

template <int DT>
static void adamw_dispatch_p(const AdamParams& prm, unsigned grid, hipStream_t st) {
  switch (prm.P) {
    case 1: adamw_dispatch_param<DT, 1>(prm, grid, st); break;
    case 2: adamw_dispatch_param<DT, 2>(prm, grid, st); break;
    case 4: adamw_dispatch_param<DT, 4>(prm, grid, st); break;
    case 8: adamw_dispatch_param<DT, 8>(prm, grid, st); break;
    default: adamw_dispatch_param<DT, 0>(prm, grid, st); break;
  }
}

hipError_t launch_adamw(const AdamLaunch& a, hipStream_t stream) {
  AdamParams prm;
  prm.R = a.replicas ? pack_replicas(a.replicas, a.P) : Replicas{};
  prm.P = a.P;
  prm.inv_scale = a.inv_scale;
  prm.grad = a.grad;
  prm.master = a.master;
  prm.m = a.m;
  prm.v = a.v;
  prm.param = a.param;
  prm.accs = a.accs;
  prm.n_accs = a.n_accs;
  prm.check_overflow = a.check_overflow;
  prm.max_norm = a.max_norm;
  prm.skipped_out = a.skipped_out;
  prm.n = a.n;
  prm.nchunks = (a.n + kVec - 1) / kVec;
  prm.s = a.s;
  const unsigned grid = grid_for(prm.nchunks);
  if (a.grad != nullptr)
    adamw_dispatch_param<-1, 1>(prm, grid, stream);
  else if (a.dtype == ZERO_BF16)
    adamw_dispatch_p<ZERO_BF16>(prm, grid, stream);
  else
    adamw_dispatch_p<ZERO_F32>(prm, grid, stream);
  return hipGetLastError();
}

// ---------------------------------------------------------- small ones ---

__global__ void gate_kernel(const zero_norm_acc* accs, int n_accs, double max_norm,
                            int check_overflow, float* coef_out, int32_t* skip_out) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const Gate g = evaluate_gate(accs, n_accs, max_norm, check_overflow);
    *coef_out = g.coef;
    *skip_out = g.skip;
  }
}

hipError_t launch_gate(const zero_norm_acc* accs, int n_accs, double max_norm,
                       int check_overflow, float* coef_out, int32_t* skip_out,
                       hipStream_t stream) {
  hipLaunchKernelGGL(gate_kernel, dim3(1), dim3(64), 0, stream, accs, n_accs, max_norm,
                     check_overflow, coef_out, skip_out);
  return hipGetLastError();
}

__global__ void acc_clear_kernel(uint64_t* words, int nwords) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nwords) words[i] = 0;
}

hipError_t launch_acc_clear(zero_norm_acc* accs, int n_accs, hipStream_t stream) {
  const int nwords = n_accs * static_cast<int>(sizeof(zero_norm_acc) / 8);
  const int blocks = (nwords + 255) / 256;
  hipLaunchKernelGGL(acc_clear_kernel, dim3(blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint64_t*>(accs), nwords);
  return hipGetLastError();
}

// -------------------------------------------------------------- MXFP8 ----

__device__ __forceinline__ int dpp_quad_int(int x, int which) {
  return which == 1 ? __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false)
                    : __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
}

// E4M3FN code of bf16 x scaled by 2^-e_s: round to nearest even on the E4M3
// grid (bias 7, subnormal step 2^-9), saturating at 448, sign kept.  Pure
// integer arithmetic on the bf16 bits.
__device__ __forceinline__ uint32_t e4m3_code(uint32_t x, int e_s) {
  const uint32_t sign = (x >> 8) & 0x80u;
  const uint32_t mag = x & 0x7FFFu;
  if (mag == 0) return sign;
  const int ex = static_cast<int>(mag >> 7);
  const uint32_t M = ex ? ((mag & 0x7Fu) | 0x80u) : (mag & 0x7Fu);
  const int base = (ex ? ex : 1) - 134 - e_s;  // value = M * 2^base
  const int msb = 31 - __clz(static_cast<int>(M));
  const int Eq = base + msb;                   // floor(log2 |q|)
  const int qe = (Eq > -6 ? Eq : -6) - 3;      // exponent of the E4M3 step
  const int sh = qe - base;                    // >= -3
  uint32_t k;
  if (sh <= 0) {
    k = M << (-sh);
  } else {
    const int s = sh > 31 ? 31 : sh;
    k = M >> s;
    const uint32_t rem = M & ((1u << s) - 1u);
    const uint32_t half = 1u << (s - 1);
    if (rem > half || (rem == half && (k & 1u))) ++k;
  }
  uint32_t code = (static_cast<uint32_t>(qe + 9) << 3) + k;
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

__global__ void __launch_bounds__(kThreads) mxfp8_kernel(const uint16_t* in, uint64_t nchunks,
                                                         uint8_t* elem, uint8_t* scale) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint64_t ntiles = (nchunks + kThreads - 1) / kThreads;
  for (uint64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const uint64_t c = tile * kThreads + tid;
    const bool valid = c < nchunks;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (valid) {
      const uint4 v = *reinterpret_cast<const uint4*>(in + c * kVec);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
    uint32_t xs[kVec];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xs[2 * j] = w[j] & 0xFFFFu;
      xs[2 * j + 1] = w[j] >> 16;
    }
    int special = 0;
    int amax = 0;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int mag = static_cast<int>(xs[j] & 0x7FFFu);
      special |= (mag >= 0x7F80) ? 1 : 0;
      amax = mag > amax ? mag : amax;
    }
    special |= dpp_quad_int(special, 1);
    special |= dpp_quad_int(special, 2);
    {
      const int o1 = dpp_quad_int(amax, 1);
      amax = o1 > amax ? o1 : amax;
      const int o2 = dpp_quad_int(amax, 2);
      amax = o2 > amax ? o2 : amax;
    }
    uint32_t sbyte;
    uint32_t codes[kVec];
    if (special) {
      sbyte = 0xFFu;
#pragma unroll
      for (int j = 0; j < kVec; ++j) codes[j] = ((xs[j] >> 8) & 0x80u) | 0x7Fu;
    } else if (amax == 0) {
      sbyte = 0x00u;
#pragma unroll
      for (int j = 0; j < kVec; ++j) codes[j] = (xs[j] >> 8) & 0x80u;
    } else {
      const int ex = amax >> 7;
      const int E = ex ? ex - 127 : -133 + (31 - __clz(amax & 0x7F));
      int e_s = E - 8;
      e_s = e_s < -127 ? -127 : (e_s > 127 ? 127 : e_s);
      sbyte = static_cast<uint32_t>(e_s + 127);
#pragma unroll
      for (int j = 0; j < kVec; ++j) codes[j] = e4m3_code(xs[j], e_s);
    }
    if (valid) {
      uint2 out;
      out.x = codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
      out.y = codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24);
      *reinterpret_cast<uint2*>(elem + c * kVec) = out;
    }
    // scale bytes: lane 16i gathers the four quads 16i, 16i+4, 16i+8, 16i+12
    const uint32_t s1 = __shfl(sbyte, lane + 4);
    const uint32_t s2 = __shfl(sbyte, lane + 8);
    const uint32_t s3 = __shfl(sbyte, lane + 12);
    if ((lane & 15) == 0 && valid) {
      const uint64_t b = c / 4;  // block index, a multiple of 4
      const uint64_t nblocks = nchunks / 4;
      if (b + 4 <= nblocks) {
        *reinterpret_cast<uint32_t*>(scale + b) = sbyte | (s1 << 8) | (s2 << 16) | (s3 << 24);
      } else {
        const uint32_t sv[4] = {sbyte, s1, s2, s3};
        for (uint64_t k = 0; b + k < nblocks; ++k) scale[b + k] = static_cast<uint8_t>(sv[k]);
      }
    }
  }
}

hipError_t launch_mxfp8(const uint16_t* in, uint64_t n, uint8_t* elem, uint8_t* scale,
                        hipStream_t stream) {
  const uint64_t nchunks = n / kVec;
  const unsigned grid = grid_for(nchunks);
  hipLaunchKernelGGL(mxfp8_kernel, dim3(grid), dim3(kThreads), 0, stream, in, nchunks, elem,
                     scale);
  return hipGetLastError();
}

}  // namespace zs
