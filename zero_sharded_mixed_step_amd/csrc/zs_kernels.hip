// zs_kernels.hip -- the optimizer step's HIP kernels for CDNA4 (gfx950).
//
// The three streaming passes -- the shard reduce, AdamW and the MXFP8 pack --
// are HBM-bandwidth-bound (no matrix work, so no MFMA): 16-byte vector
// loads/stores per lane over 2048-element tiles.  Small one-workgroup
// kernels fold the reduce's slots, evaluate the gate, advance the device
// step counter and clear accumulators.
// AdamW, the pack and (given a workspace) the reduce of 4 or more replicas
// run one-shot grids of a few tiles per workgroup; the reduce's norm state
// (reduced in registers by quad DPP, then in lane-private LDS rows) then
// goes to workspace slots that a one-workgroup kernel folds.  Other reduce
// launches run a persistent grid of a few workgroups per compute unit, each
// ending with one set of integer atomics on the accumulator.
#include "zs_device.h"
#include "zs_internal.h"

namespace zs {

// ---------------------------------------------------------------- grid ----

// Queried per launch (the runtime answers from its own device table), so the
// library keeps no state between calls.
int compute_units(int device) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

static unsigned grid_for(uint64_t nchunks, int blocks_per_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const uint64_t ntiles = (nchunks + kThreads - 1) / kThreads;
  const uint64_t cap = static_cast<uint64_t>(compute_units(dev)) * blocks_per_cu;
  const uint64_t g = ntiles < cap ? ntiles : cap;
  return static_cast<unsigned>(g > 0 ? g : 1);
}

// One-shot grid: every workgroup takes U consecutive tiles and exits, so the
// hardware dispatcher hands out tiles in address order and the stream's
// front stays compact.  Measured on MI355X, write-heavy streams run faster
// this way than on a persistent grid that strides over the array: a plain
// 15 GB write 6.8 vs 5.5-5.8 TB/s, the AdamW pass 2-6 %, the MXFP8 pack
// 15 % and the whole-shard reduce 5 % faster, with bitwise the same results.  Grids beyond the dispatch
// limit (2^32 work-items) are capped; the kernels' grid-stride loops then
// take the rest.
static unsigned grid_oneshot(uint64_t nchunks, int u) {
  const uint64_t ntiles = (nchunks + kThreads - 1) / kThreads;
  const uint64_t cap = 0xFFFFFFFFull / kThreads;
  uint64_t g = (ntiles + u - 1) / u;
  if (g > cap) g = cap;
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
  // One-shot form with a norm: the caller's workspace, kReduceSlots
  // accumulators.
  zero_norm_acc* slots;
};

// Accumulators of the one-shot reduce: workgroup b adds its norm state to
// slot b % kReduceSlots, which spreads the integer atomics over as many
// cache lines; on one line they serialise (about 12 ns each measured on
// MI355X, far slower than the stream).  A one-workgroup kernel launched
// next on the stream folds the slots into the caller's accumulator and
// clears them; the launch boundary orders the two, so neither needs a
// fence (an agent-scope fence per workgroup, which writes back L2, made the
// pass four times slower).
constexpr int kReduceSlots = ZERO_REDUCE_WORKSPACE_BYTES / sizeof(zero_norm_acc);
static_assert(kReduceSlots == 512 && kReduceSlots >= kThreads, "workspace layout");

// Norm totals of a workgroup: the kDigits digits, then the non-finite count.
constexpr int kTot = kDigits + 1;

// Sum over the 64 lanes of a wave (every lane receives it).
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Per-workgroup totals of a norm state (the digits from the lanes' own LDS
// rows, the non-finite count from a register), reduced across the workgroup
// by wave shuffles and one LDS exchange: every lane gets them in tot[].  A
// digit that is zero in every lane of a wave (most of them: a gradient's
// group sums span a few binades) skips its shuffles; the ballot is uniform
// across the wave.  Ends with the workgroup past a barrier.
__device__ __forceinline__ void workgroup_norm_totals(const uint64_t (*s_digit)[kThreads],
                                                      uint64_t count,
                                                      uint64_t (*s_part)[kTot],
                                                      uint64_t tot[kTot]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint64_t v[kTot];
#pragma unroll
  for (int k = 0; k < kDigits; ++k) v[k] = s_digit[k][tid];  // this lane's own row
  v[kDigits] = count;
#pragma unroll
  for (int k = 0; k < kTot; ++k)
    if (__builtin_amdgcn_ballot_w64(v[k] != 0) != 0) v[k] = wave_sum_u64(v[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < kTot; ++k) s_part[wave][k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kTot; ++k) {
    uint64_t t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t += s_part[w][k];
    tot[k] = t;
  }
}

// Adds totals (digits, count) to an accumulator; zero parts are skipped.
__device__ __forceinline__ void acc_add(zero_norm_acc* acc, const uint64_t tot[kTot]) {
#pragma unroll
  for (int k = 0; k < kDigits; ++k)
    if (tot[k] != 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(&acc->digit[k]),
                static_cast<unsigned long long>(tot[k]));
  if (tot[kDigits] != 0)
    atomicAdd(reinterpret_cast<unsigned long long*>(&acc->nonfinite),
              static_cast<unsigned long long>(tot[kDigits]));
}

#ifndef ZS_REDUCE_LOADS
#define ZS_REDUCE_LOADS 24
#endif
#ifndef ZS_REDUCE_PIPE_LOADS
#define ZS_REDUCE_PIPE_LOADS 16
#endif
#ifndef ZS_REDUCE_PIPE_MAX_ELEMS
#define ZS_REDUCE_PIPE_MAX_ELEMS (1ull << 27)
#endif


#ifndef ZS_REDUCE_ONESHOT_LOADS
#define ZS_REDUCE_ONESHOT_LOADS 16
#endif

// Tiles per workgroup iteration of the reduce: about `loads` 16-byte loads
// per lane (P of them per bf16 tile, 2P per fp32 tile; 8 assumed for a
// replica count only known at run time), between 1 and 8.
template <int DT, int PT>
constexpr int reduce_tiles_per_step(int loads) {
  const int raw = PT > 0 ? PT * (DT == ZERO_F32 ? 2 : 1) : 8;
  return loads / raw < 1 ? 1 : (loads / raw > 8 ? 8 : loads / raw);
}

// ONESHOT: a one-shot grid of about ZS_REDUCE_ONESHOT_LOADS 16-byte loads
// per lane per workgroup; with NORM, per-workgroup state goes to prm.slots.
template <int DT, int PT, bool WRITE, bool NORM, bool PIPE, bool ONESHOT>
__global__ void __launch_bounds__(kThreads) shard_reduce_kernel(ReduceParams prm) {
  static_assert(!PIPE || PT >= 4, "the pipelined fast path is built for 4 or 8 replicas");
  static_assert(!(PIPE && ONESHOT), "one loop form per kernel");
  __shared__ uint64_t s_digit[NORM ? kDigits : 1][kThreads];
  __shared__ uint32_t s_count[(NORM && !ONESHOT) ? kThreads : 1];
  const int tid = threadIdx.x;
  const int quad_lane = tid & 3;
  if constexpr (NORM) {
#pragma unroll
    for (int k = 0; k < kDigits; ++k) s_digit[k][tid] = 0;
  }
  uint32_t nonfinite = 0;
  // Averaged-gradient stores of whole tiles.  A lane owns 32 contiguous bytes
  // of g, so two per-lane 16-byte stores would each leave holes across the
  // wave; staging the wave's 2 KB in LDS lets every store instruction write
  // 1 KB contiguous, so the nontemporal write stream carries only full lines
  // (per-lane stores measured 1.20x the algorithmic write bytes, this 1.00x).
  __shared__ f32x4 s_stage[kThreads / 64][128];
  auto store_g_tile = [&](float* g_out, uint64_t c, const float g[kVec]) {
    const int wave = tid >> 6, lane = tid & 63;
    s_stage[wave][2 * lane] = f32x4{g[0], g[1], g[2], g[3]};
    s_stage[wave][2 * lane + 1] = f32x4{g[4], g[5], g[6], g[7]};
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // LDS is in order within a wave
    const f32x4 lo = s_stage[wave][lane];
    const f32x4 hi = s_stage[wave][64 + lane];
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    f32x4* base = reinterpret_cast<f32x4*>(g_out + (c - lane) * kVec);
    store_stream<true>(base + lane, lo);
    store_stream<true>(base + 64 + lane, hi);
  };
  // Norm state of one chunk; reached by all 64 lanes (quad DPP inside).
  auto norm_chunk = [&](const float g[kVec]) {
    const double a = chunk_sumsq(g, nonfinite);
    const double S = quad_group_sum(a);
    int d;
    uint64_t piece;
    fixed_point_piece(S, quad_lane, d, piece);
    if (piece != 0) s_digit[d][tid] += piece;  // lane-private row
  };
  // Norm state of four chunks per lane: every quad lane holds the four
  // group sums, and lane q converts group q whole (three pieces), so the
  // fixed-point work is done once per group instead of once per lane.
  double s4[4];
  auto norm_chunk4 = [&](int u, const float g[kVec]) {
    s4[u & 3] = quad_group_sum(chunk_sumsq(g, nonfinite));
    if ((u & 3) != 3) return;
    const double S = quad_lane == 0 ? s4[0] : (quad_lane == 1 ? s4[1]
                                            : (quad_lane == 2 ? s4[2] : s4[3]));
    int base;
    uint32_t p0, p1, p2;
    fixed_point_split(S, base, p0, p1, p2);
    if (p0 != 0) s_digit[base][tid] += p0;
    if (p1 != 0) s_digit[base + 1][tid] += p1;
    if (p2 != 0) s_digit[base + 2][tid] += p2;
  };
  // Chunks per lane per fast-path iteration.  PIPE (4 or 8 replicas, launches
  // of up to ZS_REDUCE_PIPE_MAX_ELEMS elements) software-pipelines the fast
  // path: the loads of the next U tiles are in flight while the current U
  // tiles are summed, stored and squared, about ZS_REDUCE_PIPE_LOADS 16-byte
  // loads per stage, on one workgroup per compute unit.  Otherwise about
  // ZS_REDUCE_LOADS loads are issued, then consumed.
  constexpr bool kPipe = PIPE;
  constexpr int U = reduce_tiles_per_step<DT, PT>(
      kPipe ? ZS_REDUCE_PIPE_LOADS : (ONESHOT ? ZS_REDUCE_ONESHOT_LOADS : ZS_REDUCE_LOADS));
  const uint64_t ntiles = (prm.nchunks + kThreads - 1) / kThreads;
  const uint64_t full_tiles = prm.n / (static_cast<uint64_t>(kThreads) * kVec);
  const uint64_t step = static_cast<uint64_t>(gridDim.x) * U;
  uint64_t tile = static_cast<uint64_t>(blockIdx.x) * U;
  // Fast path: U whole tiles at a time, no bounds checks.
  if constexpr (kPipe) {
    RawChunk<DT, PT> cur[U];
    if (tile + U <= full_tiles) {
#pragma unroll
      for (int u = 0; u < U; ++u) load_raw<DT, PT>(prm.R, (tile + u) * kThreads + tid, cur[u]);
    }
    for (; tile + U <= full_tiles; tile += step) {
      const uint64_t next = tile + step;
      const bool more = next + U <= full_tiles;  // uniform across the workgroup
      RawChunk<DT, PT> nxt[U];
      if (more) {
#pragma unroll
        for (int u = 0; u < U; ++u) load_raw<DT, PT>(prm.R, (next + u) * kThreads + tid, nxt[u]);
      }
      __builtin_amdgcn_sched_barrier(0);  // the next loads go out before this work
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float g[kVec];
        sum_raw<DT, PT>(cur[u], prm.inv_scale, g);
        if (WRITE) store_g_tile(prm.g_out, (tile + u) * kThreads + tid, g);
        if constexpr (NORM && U % 4 == 0) norm_chunk4(u, g);
        else if constexpr (NORM) norm_chunk(g);
      }
      if (more) {
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
      }
    }
  } else {
    for (; tile + U <= full_tiles; tile += step) {
      if constexpr (PT > 0) {
        RawChunk<DT, PT> raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) load_raw<DT, PT>(prm.R, (tile + u) * kThreads + tid, raw[u]);
        __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the first wait
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float g[kVec];
          sum_raw<DT, PT>(raw[u], prm.inv_scale, g);
          if (WRITE) store_g_tile(prm.g_out, (tile + u) * kThreads + tid, g);
          if constexpr (NORM && U % 4 == 0) norm_chunk4(u, g);
          else if constexpr (NORM) norm_chunk(g);
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float g[kVec];
          reduce_chunk<DT, PT>(prm.R, prm.P, (tile + u) * kThreads + tid, true, prm.n,
                               prm.inv_scale, g);
          if (WRITE)
            store_f32_chunk<true>(prm.g_out, (tile + u) * kThreads + tid, true, prm.n, g);
          if constexpr (NORM) norm_chunk(g);
        }
      }
    }
  }
  // Tail: the remaining tiles of this workgroup one by one, with checks.
  for (; tile < ntiles; tile += step) {
    for (int u = 0; u < U; ++u) {
      if (tile + u >= ntiles) break;  // uniform across the workgroup
      const uint64_t c = (tile + u) * kThreads + tid;
      const bool valid = c < prm.nchunks;
      const bool full = valid && (c * kVec + kVec <= prm.n);
      float g[kVec];
      if (valid) {
        reduce_chunk<DT, PT>(prm.R, prm.P, c, full, prm.n, prm.inv_scale, g);
        if (WRITE) store_f32_chunk<true>(prm.g_out, c, full, prm.n, g);
      } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) g[j] = 0.0f;
      }
      if constexpr (NORM) norm_chunk(g);
    }
  }
  if constexpr (NORM && ONESHOT) {
    // Workgroup totals into slot blockIdx % kReduceSlots.
    __shared__ uint64_t s_part[kThreads / 64][kTot];
    uint64_t tot[kTot];
    workgroup_norm_totals(s_digit, nonfinite, s_part, tot);
    if (tid == 0) acc_add(prm.slots + blockIdx.x % kReduceSlots, tot);
  } else if constexpr (NORM) {
    s_count[tid] = nonfinite;
    __syncthreads();
    for (int stride = kThreads / 2; stride > 0; stride >>= 1) {
      if (tid < stride) {
#pragma unroll
        for (int k = 0; k < kDigits; ++k) s_digit[k][tid] += s_digit[k][tid + stride];
        s_count[tid] += s_count[tid + stride];
      }
      __syncthreads();
    }
    if (tid == 0) {
      uint64_t tot[kTot];
#pragma unroll
      for (int k = 0; k < kDigits; ++k) tot[k] = s_digit[k][0];
      tot[kDigits] = s_count[0];
      acc_add(prm.acc, tot);
    }
  }
}

// Adds the slots of a one-shot reduce to acc and zeroes them (one
// workgroup; each slot field is read and cleared by one atomic exchange).
__global__ void __launch_bounds__(kThreads) slot_fold_kernel(zero_norm_acc* slots,
                                                             zero_norm_acc* acc) {
  __shared__ uint64_t s_rows[kDigits][kThreads];
  __shared__ uint64_t s_part[kThreads / 64][kTot];
  const int tid = threadIdx.x;
  uint64_t mine[kTot];
#pragma unroll
  for (int k = 0; k < kTot; ++k) mine[k] = 0;
  for (int sl = tid; sl < kReduceSlots; sl += kThreads) {
    zero_norm_acc* a = slots + sl;
#pragma unroll
    for (int k = 0; k < kDigits; ++k)
      mine[k] += atomicExch(reinterpret_cast<unsigned long long*>(&a->digit[k]), 0ull);
    mine[kDigits] += atomicExch(reinterpret_cast<unsigned long long*>(&a->nonfinite), 0ull);
  }
#pragma unroll
  for (int k = 0; k < kDigits; ++k) s_rows[k][tid] = mine[k];
  uint64_t tot[kTot];
  workgroup_norm_totals(s_rows, mine[kDigits], s_part, tot);
  if (tid == 0) acc_add(acc, tot);
}

template <int DT, int PT, bool PIPE, bool ONESHOT>
static void reduce_launch(const ReduceParams& prm, bool write, bool norm, unsigned grid,
                          hipStream_t st) {
  if (write && norm)
    hipLaunchKernelGGL((shard_reduce_kernel<DT, PT, true, true, PIPE, ONESHOT>), dim3(grid),
                       dim3(kThreads), 0, st, prm);
  else if (write)
    hipLaunchKernelGGL((shard_reduce_kernel<DT, PT, true, false, PIPE, ONESHOT>), dim3(grid),
                       dim3(kThreads), 0, st, prm);
  else
    hipLaunchKernelGGL((shard_reduce_kernel<DT, PT, false, true, PIPE, ONESHOT>), dim3(grid),
                       dim3(kThreads), 0, st, prm);
}

// Loop forms, all computing the same bits.  With 4 or more replicas and a
// workspace, the one-shot grid: on MI355X the 30B-shard reduce (8 bf16
// replicas, 3.75e9 elements) ran at 5.9 TB/s on it against 5.6 on the
// persistent grid; for 25e6-element buckets, the extra fold launch per
// bucket made it slower than the pipelined form (so callers pass no
// workspace there).  Without a workspace, below ZS_REDUCE_PIPE_MAX_ELEMS
// elements (a bucket) the pipelined form on one workgroup per CU measured
// faster with 4 or 8 replicas; above it the unpipelined form on
// ZS_REDUCE_BLOCKS_PER_CU did.  With one to three replicas the pass is bound
// by the norm's arithmetic, and the persistent grid, which meets the atomics
// once per workgroup, stays.
template <int DT, int PT>
static void reduce_dispatch_io(const ReduceParams& prm, bool write, bool norm,
                               hipStream_t st) {
  if ((PT >= 4 || (PT == 0 && prm.P >= 4)) && prm.slots != nullptr) {
    constexpr int U = reduce_tiles_per_step<DT, PT>(ZS_REDUCE_ONESHOT_LOADS);
    reduce_launch<DT, PT, false, true>(prm, write, norm, grid_oneshot(prm.nchunks, U), st);
    if (norm)
      hipLaunchKernelGGL(slot_fold_kernel, dim3(1), dim3(kThreads), 0, st, prm.slots, prm.acc);
    return;
  }
  if constexpr (PT >= 4) {
    if (prm.n <= static_cast<uint64_t>(ZS_REDUCE_PIPE_MAX_ELEMS)) {
      reduce_launch<DT, PT, true, false>(prm, write, norm,
                                         grid_for(prm.nchunks, ZS_REDUCE_PIPE_BLOCKS_PER_CU),
                                         st);
      return;
    }
  }
  reduce_launch<DT, PT, false, false>(prm, write, norm,
                                      grid_for(prm.nchunks, ZS_REDUCE_BLOCKS_PER_CU), st);
}

template <int DT>
static void reduce_dispatch_p(const ReduceParams& prm, bool write, bool norm, hipStream_t st) {
  switch (prm.P) {
    case 1: reduce_dispatch_io<DT, 1>(prm, write, norm, st); break;
    case 2: reduce_dispatch_io<DT, 2>(prm, write, norm, st); break;
    case 4: reduce_dispatch_io<DT, 4>(prm, write, norm, st); break;
    case 8: reduce_dispatch_io<DT, 8>(prm, write, norm, st); break;
    default: reduce_dispatch_io<DT, 0>(prm, write, norm, st); break;
  }
}

hipError_t launch_reduce(const void* const* replicas, int P, int dtype, uint64_t n,
                         float inv_scale, float* g_out, zero_norm_acc* acc,
                         hipStream_t stream, const void* const* mx_scales, void* workspace) {
  ReduceParams prm;
  prm.slots = static_cast<zero_norm_acc*>(workspace);
  prm.R = pack_replicas(replicas, P);
  if (mx_scales != nullptr)
    for (int k = 0; k < P; ++k) prm.R.s[k] = mx_scales[k];
  prm.P = P;
  prm.inv_scale = inv_scale;
  prm.n = n;
  prm.nchunks = (n + kVec - 1) / kVec;
  prm.g_out = g_out;
  prm.acc = acc;
  const bool write = g_out != nullptr, norm = acc != nullptr;
  if (dtype == ZERO_BF16)
    reduce_dispatch_p<ZERO_BF16>(prm, write, norm, stream);
  else if (dtype == ZERO_MXFP8)
    reduce_dispatch_p<ZERO_MXFP8>(prm, write, norm, stream);
  else
    reduce_dispatch_p<ZERO_F32>(prm, write, norm, stream);
  return hipGetLastError();
}

// -------------------------------------------------------------- AdamW ----

// bf16 of x, round to nearest even; NaN -> quiet NaN with the sign (select,
// no branch).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t rounded = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  const uint32_t qnan = ((b >> 16) & 0x8000u) | 0x7FC0u;
  return (b & 0x7FFFFFFFu) > 0x7F800000u ? qnan : rounded;
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
  uint8_t* mx_elem;
  uint8_t* mx_scale;
  const zero_norm_acc* accs;
  int n_accs;
  int check_overflow;
  double max_norm;
  int32_t* skipped_out;
  uint64_t n;
  uint64_t nchunks;
  AdamScalars s;             // scalars of the host-counted update, or
  AdamHyper h;               // hyperparameters to derive them from
  const int64_t* step_dev;   // the device counter of applied updates
};

#ifndef ZS_ADAMW_UNROLL
#define ZS_ADAMW_UNROLL 2
#endif

// SRC < 0: gradient from prm.grad (fp32); otherwise the replica dtype.
// MX: also pack the new bf16 params to MXFP8 (n % 32 == 0); the loop then
// stays wave-uniform because the block amax is a quad DPP reduction.
// U: tiles per workgroup (one-shot grid).
template <int SRC, int PT, bool PARAM, bool MX, int U, bool EARLY>
__global__ void __launch_bounds__(kThreads) adamw_kernel(AdamParams prm) {
  __shared__ Gate s_gate;
  __shared__ AdamScalars s_sc;
  const uint64_t ntiles = (prm.nchunks + kThreads - 1) / kThreads;
  const uint64_t full_tiles = prm.n / (static_cast<uint64_t>(kThreads) * kVec);
  const uint64_t step = static_cast<uint64_t>(gridDim.x) * U;
  uint64_t tile = static_cast<uint64_t>(blockIdx.x) * U;
  // Loads of U whole tiles (gradient, master, m, v) into registers.
  auto load_tiles = [&](uint64_t t0, float (&g)[U][kVec], float (&th)[U][kVec],
                        float (&mm)[U][kVec], float (&vv)[U][kVec]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t c = (t0 + u) * kThreads + threadIdx.x;
      if constexpr (SRC < 0)
        load_f32_chunk<false>(prm.grad, c, true, prm.n, g[u]);
      else
        reduce_chunk<SRC, PT>(prm.R, prm.P, c, true, prm.n, prm.inv_scale, g[u]);
      load_f32_chunk<false>(prm.master, c, true, prm.n, th[u]);
      load_f32_chunk<false>(prm.m, c, true, prm.n, mm[u]);
      load_f32_chunk<false>(prm.v, c, true, prm.n, vv[u]);
    }
  };
  // EARLY: the workgroup's first U whole tiles are loaded before the gate is
  // evaluated, so the gate's latency overlaps theirs (a skipped step
  // discards them).  It pays on launches of up to about 128 workgroups per
  // compute unit, where every workgroup meets the gate's latency once and
  // little else hides it.
  float g0[U][kVec], th0[U][kVec], mm0[U][kVec], vv0[U][kVec];
  const bool head = EARLY && tile + U <= full_tiles;
  if (head) load_tiles(tile, g0, th0, mm0, vv0);
  if (threadIdx.x == 0) {
    const Gate gt = evaluate_gate(prm.accs, prm.n_accs, prm.max_norm, prm.check_overflow);
    s_gate = gt;
    s_sc = prm.step_dev != nullptr ? derive_adam_scalars(prm.h, *prm.step_dev + 1) : prm.s;
    if (blockIdx.x == 0 && prm.skipped_out != nullptr) *prm.skipped_out = gt.skip;
  }
  __syncthreads();
  // The gate and scalars are the same in every lane: read them into scalar
  // registers (read from LDS they would each hold a VGPR per lane).
  auto uniform = [](float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
  };
  if (__builtin_amdgcn_readfirstlane(s_gate.skip)) return;
  const float coef = uniform(s_gate.coef);
  AdamScalars sc;
  sc.b1 = uniform(s_sc.b1);
  sc.b2 = uniform(s_sc.b2);
  sc.omb1 = uniform(s_sc.omb1);
  sc.omb2 = uniform(s_sc.omb2);
  sc.step_size = uniform(s_sc.step_size);
  sc.sqrt_bc2 = uniform(s_sc.sqrt_bc2);
  sc.decay = uniform(s_sc.decay);
  sc.eps = uniform(s_sc.eps);
  const float neg_step = -sc.step_size;
  // The update of one chunk from its loaded g and state; stores the new
  // state and param and leaves the param bits in pb (for the MXFP8 epilogue).
  auto update_chunk = [&](uint64_t c, bool full, const float g[kVec], float th[kVec],
                          float mm[kVec], float vv[kVec], uint32_t pb[kVec]) {
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
    store_f32_chunk<false>(prm.master, c, full, prm.n, th);
    store_f32_chunk<false>(prm.m, c, full, prm.n, mm);
    store_f32_chunk<false>(prm.v, c, full, prm.n, vv);
    if (PARAM) {
      uint16_t* p = prm.param + c * kVec;
      if (full) {
        store_stream<false>(reinterpret_cast<u32x4*>(p),
                            u32x4{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16),
                                  pb[4] | (pb[5] << 16), pb[6] | (pb[7] << 16)});
      } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j)
          if (c * kVec + j < prm.n) p[j] = static_cast<uint16_t>(pb[j]);
      }
    }
  };
  // Update of U whole tiles from their loaded values.
  auto update_tiles = [&](uint64_t t0, float (&g)[U][kVec], float (&th)[U][kVec],
                          float (&mm)[U][kVec], float (&vv)[U][kVec]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t c = (t0 + u) * kThreads + threadIdx.x;
      uint32_t pb[kVec];
      update_chunk(c, true, g[u], th[u], mm[u], vv[u], pb);
      if constexpr (MX) {
        uint32_t words[2];
        const uint32_t sbyte = mx_quad_encode(pb, words);
        mx_store(prm.mx_elem, prm.mx_scale, c, prm.nchunks, true, words, sbyte);
      }
    }
  };
  if (head) {
    update_tiles(tile, g0, th0, mm0, vv0);
    tile += step;
  }
  // Fast path: U whole tiles, no bounds checks, every load issued first.
  for (; tile + U <= full_tiles; tile += step) {
    float g[U][kVec], th[U][kVec], mm[U][kVec], vv[U][kVec];
    load_tiles(tile, g, th, mm, vv);
    if constexpr (U > 1) __builtin_amdgcn_sched_barrier(0);
    update_tiles(tile, g, th, mm, vv);
  }
  // Tail: remaining tiles one by one with bounds checks (wave-uniform loop,
  // as the MXFP8 epilogue needs all lanes).
  for (; tile < ntiles; tile += step) {
    for (int u = 0; u < U; ++u) {
      if (tile + u >= ntiles) break;
      const uint64_t c = (tile + u) * kThreads + threadIdx.x;
      const bool valid = c < prm.nchunks;
      uint32_t pb[kVec];
      if (valid) {
        const bool full = c * kVec + kVec <= prm.n;
        float g[kVec], th[kVec], mm[kVec], vv[kVec];
        if constexpr (SRC < 0)
          load_f32_chunk<false>(prm.grad, c, full, prm.n, g);
        else
          reduce_chunk<SRC, PT>(prm.R, prm.P, c, full, prm.n, prm.inv_scale, g);
        load_f32_chunk<false>(prm.master, c, full, prm.n, th);
        load_f32_chunk<false>(prm.m, c, full, prm.n, mm);
        load_f32_chunk<false>(prm.v, c, full, prm.n, vv);
        update_chunk(c, full, g, th, mm, vv, pb);
      } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) pb[j] = 0u;
      }
      if constexpr (MX) {
        uint32_t words[2];
        const uint32_t sbyte = mx_quad_encode(pb, words);
        mx_store(prm.mx_elem, prm.mx_scale, c, prm.nchunks, valid, words, sbyte);
      }
    }
  }
}

// ZS_ADAMW_UNROLL tiles per workgroup, except where that grid would leave
// compute units idle (shards below about 2M elements): one tile each, twice
// the workgroups.  Grids of up to kAdamwEarlyPerCU workgroups per compute
// unit (shards up to about 2^27 elements) load their first tiles before the
// gate: measured on MI355X with 8 bf16 replicas and the clip, AdamW took
// 14 % less time at 15.6M elements, 3.6 % at 31M, 2.3 % at 62M and 0.9 % at
// 124M, and 0.6 % more at 249M and 1.5 % more at 875M, where the plain
// order stays.
constexpr unsigned kAdamwEarlyPerCU = 128;

template <int SRC, int PT, bool PARAM, bool MX>
static void adamw_launch(const AdamParams& prm, hipStream_t st) {
  const unsigned g = grid_oneshot(prm.nchunks, ZS_ADAMW_UNROLL);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const unsigned cus = static_cast<unsigned>(compute_units(dev));
  if (g < 2u * cus)
    hipLaunchKernelGGL((adamw_kernel<SRC, PT, PARAM, MX, 1, true>),
                       dim3(grid_oneshot(prm.nchunks, 1)), dim3(kThreads), 0, st, prm);
  else if (g <= kAdamwEarlyPerCU * cus)
    hipLaunchKernelGGL((adamw_kernel<SRC, PT, PARAM, MX, ZS_ADAMW_UNROLL, true>), dim3(g),
                       dim3(kThreads), 0, st, prm);
  else
    hipLaunchKernelGGL((adamw_kernel<SRC, PT, PARAM, MX, ZS_ADAMW_UNROLL, false>), dim3(g),
                       dim3(kThreads), 0, st, prm);
}

template <int SRC, int PT>
static void adamw_dispatch_param(const AdamParams& prm, hipStream_t st) {
  const bool param = prm.param != nullptr, mx = prm.mx_elem != nullptr;
  if (mx && param)
    adamw_launch<SRC, PT, true, true>(prm, st);
  else if (mx)
    adamw_launch<SRC, PT, false, true>(prm, st);
  else if (param)
    adamw_launch<SRC, PT, true, false>(prm, st);
  else
    adamw_launch<SRC, PT, false, false>(prm, st);
}

template <int DT>
static void adamw_dispatch_p(const AdamParams& prm, hipStream_t st) {
  switch (prm.P) {
    case 1: adamw_dispatch_param<DT, 1>(prm, st); break;
    case 2: adamw_dispatch_param<DT, 2>(prm, st); break;
    case 4: adamw_dispatch_param<DT, 4>(prm, st); break;
    case 8: adamw_dispatch_param<DT, 8>(prm, st); break;
    default: adamw_dispatch_param<DT, 0>(prm, st); break;
  }
}

// Device step counter: after the update, count it as applied unless the
// gate (the same evaluation the update made) skipped it.  Runs after every
// workgroup of the update has read the counter (stream order).
__global__ void step_advance_kernel(int64_t* step_dev, const zero_norm_acc* accs, int n_accs,
                                    double max_norm, int check_overflow) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const Gate g = evaluate_gate(accs, n_accs, max_norm, check_overflow);
    if (!g.skip) *step_dev += 1;
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
  prm.mx_elem = a.mx_elem;
  prm.mx_scale = a.mx_scale;
  prm.accs = a.accs;
  prm.n_accs = a.n_accs;
  prm.check_overflow = a.check_overflow;
  prm.max_norm = a.max_norm;
  prm.skipped_out = a.skipped_out;
  prm.n = a.n;
  prm.nchunks = (a.n + kVec - 1) / kVec;
  prm.s = a.s;
  prm.h = a.h;
  prm.step_dev = a.step_dev;
  if (a.grad != nullptr)
    adamw_dispatch_param<-1, 1>(prm, stream);
  else if (a.dtype == ZERO_BF16)
    adamw_dispatch_p<ZERO_BF16>(prm, stream);
  else
    adamw_dispatch_p<ZERO_F32>(prm, stream);
  if (a.step_dev != nullptr)
    hipLaunchKernelGGL(step_advance_kernel, dim3(1), dim3(64), 0, stream, a.step_dev, a.accs,
                       a.n_accs, a.max_norm, a.check_overflow);
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

#ifndef ZS_MX_UNROLL
#define ZS_MX_UNROLL 1
#endif

// ZS_MX_UNROLL tiles per workgroup iteration.  On the one-shot grid one tile
// per workgroup measured fastest on MI355X (30B shard: 1.87 ms against 1.91
// for 2 tiles and 2.00 for 8; on the persistent grid 8 had been best).
__global__ void __launch_bounds__(kThreads) mxfp8_kernel(const uint16_t* in, uint64_t nchunks,
                                                         uint8_t* elem, uint8_t* scale,
                                                         const Gate* gate) {
  if (gate != nullptr && gate->skip) return;  // a skipped step writes nothing
  const uint64_t ntiles = (nchunks + kThreads - 1) / kThreads;
  constexpr int U = ZS_MX_UNROLL;
  for (uint64_t tile = static_cast<uint64_t>(blockIdx.x) * U; tile < ntiles;
       tile += static_cast<uint64_t>(gridDim.x) * U) {
    uint32_t xs[U][kVec];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t c = (tile + u) * kThreads + threadIdx.x;
      valid[u] = (tile + u) < ntiles && c < nchunks;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (valid[u]) w = load_stream<false>(reinterpret_cast<const u32x4*>(in + c * kVec));
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xs[u][2 * j] = ws[j] & 0xFFFFu;
        xs[u][2 * j + 1] = ws[j] >> 16;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t c = (tile + u) * kThreads + threadIdx.x;
      uint32_t words[2];
      const uint32_t sbyte = mx_quad_encode(xs[u], words);
      mx_store(elem, scale, c, nchunks, valid[u], words, sbyte);
    }
  }
}

hipError_t launch_mxfp8(const uint16_t* in, uint64_t n, uint8_t* elem, uint8_t* scale,
                        hipStream_t stream, const Gate* gate) {
  const uint64_t nchunks = n / kVec;
  const unsigned grid = grid_oneshot(nchunks, ZS_MX_UNROLL);
  hipLaunchKernelGGL(mxfp8_kernel, dim3(grid), dim3(kThreads), 0, stream, in, nchunks, elem,
                     scale, gate);
  return hipGetLastError();
}

}  // namespace zs
