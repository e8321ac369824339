// zs_device.h -- device building blocks shared by the step's kernels:
// vector loads of gradient replicas, the fixed-order shard reduce, the exact
// fixed-point sum of squares, and the on-device clip/skip gate.
//
// Data layout: every array is a flat, 16-byte aligned vector.  A lane works
// on a "chunk" of 8 consecutive elements (one 16-byte load of bf16, two of
// fp32).  Four consecutive chunks, held by four consecutive lanes of one
// wavefront, form a 32-element norm group, so the group sum
// (a0 + a1) + (a2 + a3) is two quad-permute DPP steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_step.h"

namespace zs {

constexpr int kThreads = 256;  // four wave64 wavefronts per workgroup
constexpr int kVec = 8;        // elements per chunk
constexpr int kDigits = 13;    // 32-bit digit positions of the norm's fixed point
static_assert(sizeof(zero_norm_acc) == 128 &&
                  sizeof(((zero_norm_acc*)nullptr)->digit) == kDigits * 8,
              "accumulator layout");

struct Replicas {
  const void* p[ZERO_MAX_REPLICAS];  // element data (MXFP8: the E4M3 codes)
  const void* s[ZERO_MAX_REPLICAS];  // MXFP8 only: the scale bytes
};

// Eight MXFP8 elements (codes in lo/hi, block scale byte sb) decoded to
// binary32: v_cvt_pk_f32_fp8 gives the exact E4M3 value, and the product
// with the power of two 2^(sb - 127) is exact too (at least 2^-136, at most
// 448 * 2^127 before rounding of an overflow to inf).  A NaN code (0x7F or
// 0xFF) or the NaN scale byte 0xFF gives the quiet NaN 0x7FC00000 with the
// code's sign, written out explicitly so the bits do not depend on how the
// conversion or the multiply propagates a NaN.  The eight codes are first
// tested four at a time: a byte masked to 0x7F and plus one reaches 0x80
// only when it was a NaN code, with no carry into the next byte; lanes with
// neither a NaN code nor the NaN scale skip the per-element replacement.
__device__ __forceinline__ void decode_mx8(uint32_t lo, uint32_t hi, uint32_t sb,
                                           float x[8]) {
  // (scale byte 0xFF: any finite factor; those results are replaced below)
  const float f = sb == 0u ? __uint_as_float(0x00400000u)
                           : __uint_as_float((sb == 0xFFu ? 0x7Fu : sb) << 23);
  const uint32_t w[2] = {lo, hi};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[h]), false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[h]), true);
    x[4 * h + 0] = a[0] * f;
    x[4 * h + 1] = a[1] * f;
    x[4 * h + 2] = b[0] * f;
    x[4 * h + 3] = b[1] * f;
  }
  const uint32_t nan_bytes = (((lo & 0x7F7F7F7Fu) + 0x01010101u) |
                              ((hi & 0x7F7F7F7Fu) + 0x01010101u)) & 0x80808080u;
  if (sb == 0xFFu || nan_bytes != 0u) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t c = (w[h] >> (8 * q)) & 0xFFu;
        if (sb == 0xFFu || (c & 0x7Fu) == 0x7Fu)
          x[4 * h + q] = __uint_as_float(((c & 0x80u) << 24) | 0x7FC00000u);
      }
    }
  }
}

// ------------------------------------------------------------- loads ------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming-access policy per access: nontemporal (NT) loads/stores tell the
// memory system not to keep the lines, which suits data touched exactly once
// (gradient replicas, the averaged gradient).  The in-place AdamW state is
// read and rewritten through the cache (measured faster on MI355X).
template <bool NT, typename T>
__device__ __forceinline__ T load_stream(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT, typename T>
__device__ __forceinline__ void store_stream(T* p, T v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Eight elements of one replica as fp32 (bf16 widening is exact).  `full`
// is false only for the final, partial chunk: its elements past `n` read as
// +0 and nothing beyond the buffer is touched.
template <int DT, bool NT>
__device__ __forceinline__ void load_chunk(const void* base, uint64_t c, bool full,
                                           uint64_t n, float x[kVec]) {
  const uint64_t e0 = c * kVec;
  if constexpr (DT == ZERO_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + e0;
    if (full) {
      const u32x4 w = load_stream<NT>(reinterpret_cast<const u32x4*>(p));
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(ws[j] << 16);
        x[2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kVec; ++j) x[j] = (e0 + j < n) ? bf16_bits_to_f32(p[j]) : 0.0f;
    }
  } else {
    const float* p = static_cast<const float*>(base) + e0;
    if (full) {
      const f32x4 a = load_stream<NT>(reinterpret_cast<const f32x4*>(p));
      const f32x4 b = load_stream<NT>(reinterpret_cast<const f32x4*>(p + 4));
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < kVec; ++j) x[j] = (e0 + j < n) ? p[j] : 0.0f;
    }
  }
}

template <bool NT>
__device__ __forceinline__ void load_f32_chunk(const float* base, uint64_t c, bool full,
                                               uint64_t n, float x[kVec]) {
  load_chunk<ZERO_F32, NT>(base, c, full, n, x);
}

template <bool NT>
__device__ __forceinline__ void store_f32_chunk(float* base, uint64_t c, bool full,
                                                uint64_t n, const float x[kVec]) {
  float* p = base + c * kVec;
  if (full) {
    store_stream<NT>(reinterpret_cast<f32x4*>(p), f32x4{x[0], x[1], x[2], x[3]});
    store_stream<NT>(reinterpret_cast<f32x4*>(p + 4), f32x4{x[4], x[5], x[6], x[7]});
  } else {
    const uint64_t e0 = c * kVec;
#pragma unroll
    for (int j = 0; j < kVec; ++j)
      if (e0 + j < n) p[j] = x[j];
  }
}

// ------------------------------------------------------------ reduce ------

// g = (r_0 + r_1 + ... + r_{P-1}) * inv_scale in binary32, rank order.
// PT > 0 fixes P at compile time (all P loads issue before the adds);
// PT == 0 reads the runtime count.  Replicas are read once: NT loads.
template <int DT>
__device__ __forceinline__ void load_replica(const Replicas& R, int k, uint64_t c, bool full,
                                             uint64_t n, float x[kVec]) {
  if constexpr (DT == ZERO_MXFP8) {  // n % 32 == 0: chunks are always whole
    const u32x2 w = load_stream<true>(
        reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(R.p[k]) + c * kVec));
    const uint32_t sb = static_cast<const uint8_t*>(R.s[k])[c >> 2];
    decode_mx8(w.x, w.y, sb, x);
  } else {
    load_chunk<DT, true>(R.p[k], c, full, n, x);
  }
}

template <int DT, int PT>
__device__ __forceinline__ void reduce_chunk(const Replicas& R, int P, uint64_t c, bool full,
                                             uint64_t n, float inv_scale, float g[kVec]) {
  if constexpr (PT > 0) {
    float x[PT][kVec];
#pragma unroll
    for (int k = 0; k < PT; ++k) load_replica<DT>(R, k, c, full, n, x[k]);
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      float s = x[0][j];
#pragma unroll
      for (int k = 1; k < PT; ++k) s = s + x[k][j];
      g[j] = s * inv_scale;
    }
  } else {
    float s[kVec];
    load_replica<DT>(R, 0, c, full, n, s);
    for (int k = 1; k < P; ++k) {
      float x[kVec];
      load_replica<DT>(R, k, c, full, n, x);
#pragma unroll
      for (int j = 0; j < kVec; ++j) s[j] = s[j] + x[j];
    }
#pragma unroll
    for (int j = 0; j < kVec; ++j) g[j] = s[j] * inv_scale;
  }
}

// Two-phase form of reduce_chunk for whole chunks (PT > 0): `Raw` holds the
// undecoded 16-byte vectors of all replicas, so a caller can issue the loads
// of several chunks before any of them is summed.
template <int DT, int PT>
struct RawChunk {
  // 16-byte vectors per replica (MXFP8: codes in .x/.y, scale byte in .z)
  static constexpr int kWords = DT == ZERO_F32 ? 2 : 1;
  u32x4 w[PT][kWords];
};

template <int DT, int PT>
__device__ __forceinline__ void load_raw(const Replicas& R, uint64_t c, RawChunk<DT, PT>& r) {
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    if constexpr (DT == ZERO_BF16) {
      r.w[k][0] = load_stream<true>(
          reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(R.p[k]) + c * kVec));
    } else if constexpr (DT == ZERO_MXFP8) {
      const u32x2 w = load_stream<true>(
          reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(R.p[k]) + c * kVec));
      r.w[k][0] = u32x4{w.x, w.y, static_cast<const uint8_t*>(R.s[k])[c >> 2], 0u};
    } else {
      const u32x4* p =
          reinterpret_cast<const u32x4*>(static_cast<const float*>(R.p[k]) + c * kVec);
      r.w[k][0] = load_stream<true>(p);
      r.w[k][1] = load_stream<true>(p + 1);
    }
  }
}

template <int DT, int PT>
__device__ __forceinline__ void sum_raw(const RawChunk<DT, PT>& r, float inv_scale,
                                        float g[kVec]) {
  float x[PT][kVec];
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    if constexpr (DT == ZERO_BF16) {
      const uint32_t ws[4] = {r.w[k][0].x, r.w[k][0].y, r.w[k][0].z, r.w[k][0].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[k][2 * j] = __uint_as_float(ws[j] << 16);
        x[k][2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
      }
    } else if constexpr (DT == ZERO_MXFP8) {
      decode_mx8(r.w[k][0].x, r.w[k][0].y, r.w[k][0].z, x[k]);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        x[k][4 * h + 0] = __uint_as_float(r.w[k][h].x);
        x[k][4 * h + 1] = __uint_as_float(r.w[k][h].y);
        x[k][4 * h + 2] = __uint_as_float(r.w[k][h].z);
        x[k][4 * h + 3] = __uint_as_float(r.w[k][h].w);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    float s = x[0][j];
#pragma unroll
    for (int k = 1; k < PT; ++k) s = s + x[k][j];
    g[j] = s * inv_scale;
  }
}

// -------------------------------------------------- exact sum of squares --

// a = q_0 + q_1 + ... + q_7 left to right in binary64 with q_j = g_j^2
// (exact, so fma(g, g, a) rounds exactly like a + q).  Non-finite values
// add 0 and are counted.
__device__ __forceinline__ double chunk_sumsq(const float g[kVec], uint32_t& nonfinite) {
  double a = 0.0;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const bool fin = __builtin_isfinite(g[j]);
    nonfinite += fin ? 0u : 1u;
    const double xd = fin ? static_cast<double>(g[j]) : 0.0;
    a = __builtin_fma(xd, xd, a);
  }
  return a;
}

__device__ __forceinline__ double dpp_quad_perm(double x, int ctrl_tag) {
  // ctrl_tag 1: lanes (1,0,3,2) of each quad; 2: lanes (2,3,0,1).
  const uint64_t b = __double_as_longlong(x);
  int lo = static_cast<int>(b & 0xFFFFFFFFu);
  int hi = static_cast<int>(b >> 32);
  if (ctrl_tag == 1) {
    lo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false);
    hi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false);
  } else {
    lo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false);
    hi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false);
  }
  return __longlong_as_double((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                              static_cast<uint32_t>(lo));
}

// Group sum S = (a0 + a1) + (a2 + a3) over the quad; every lane of the quad
// ends with the same S (IEEE addition is commutative).  Must be reached by
// all 64 lanes.
__device__ __forceinline__ double quad_group_sum(double a) {
  const double b = a + dpp_quad_perm(a, 1);
  return b + dpp_quad_perm(b, 2);
}

// floor(S * 2^128) split into three 32-bit pieces p0, p1, p2 at digits
// base, base+1, base+2.  0 <= S < 2^262 (a group of finite binary32 values
// gives S < 2^261), so the exponent field is at most 1284, sh below at most
// 337 and base + 2 <= 12 = kDigits - 1.  A zero or subnormal S (below
// 2^-1022, so below one unit) gives three zero pieces; so would anything
// outside that range, which keeps every digit index in bounds.
__device__ __forceinline__ void fixed_point_split(double S, int& base, uint32_t& p0,
                                                  uint32_t& p1, uint32_t& p2) {
  const uint64_t bits = __double_as_longlong(S);
  const int ex = static_cast<int>((bits >> 52) & 0x7FF);
  base = 0;
  p0 = p1 = p2 = 0u;
  if (ex == 0 || ex > 1284) return;
  const uint64_t mant = (bits & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int sh = ex - 947;  // S * 2^128 = mant * 2^sh
  if (sh < 0) {
    const uint64_t v = (sh <= -53) ? 0ull : (mant >> (-sh));
    p0 = static_cast<uint32_t>(v);
    p1 = static_cast<uint32_t>(v >> 32);
  } else {
    const int r = sh & 31;
    base = sh >> 5;
    const uint64_t lo = mant << r;
    const uint64_t hi = r ? (mant >> (64 - r)) : 0ull;
    p0 = static_cast<uint32_t>(lo);
    p1 = static_cast<uint32_t>(lo >> 32);
    p2 = static_cast<uint32_t>(hi);
  }
}

// One piece of floor(S * 2^128) per quad lane: lane q (0..2) returns piece q
// and its digit; lane 3 returns 0.
__device__ __forceinline__ void fixed_point_piece(double S, int quad_lane, int& digit,
                                                  uint64_t& piece) {
  int base;
  uint32_t p0, p1, p2;
  fixed_point_split(S, base, p0, p1, p2);
  piece = quad_lane == 0 ? p0 : (quad_lane == 1 ? p1 : (quad_lane == 2 ? p2 : 0u));
  digit = base + (quad_lane < 3 ? quad_lane : 0);
}

// -------------------------------------------------------------- MXFP8 ----


__device__ __forceinline__ int dpp_quad_int(int x, int which) {
  return which == 1 ? __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false)
                    : __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t dpp_row_shl(uint32_t x, int k) {
  // lane i of each 16-lane row receives lane i + k of the same row
  switch (k) {
    case 4: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x104, 0xF, 0xF, false));
    case 8: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x108, 0xF, 0xF, false));
    default: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x10C, 0xF, 0xF, false));
  }
}

// One 32-element block held by a quad of lanes (8 bf16 per lane): returns
// the block's scale byte (same in all four lanes) and packs this lane's 8
// codes into words[0..1] (code j in byte j).  Must be reached by all 64
// lanes.  NaN and inf have the largest bf16 magnitudes, so the integer
// maximum of the magnitudes also flags a special block.
__device__ __forceinline__ uint32_t mx_quad_encode(const uint32_t xs[kVec], uint32_t words[2]) {
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < kVec; ++j) amax = __builtin_elementwise_max(amax, xs[j] & 0x7FFFu);
  amax = __builtin_elementwise_max(amax, static_cast<uint32_t>(dpp_quad_int(static_cast<int>(amax), 1)));
  amax = __builtin_elementwise_max(amax, static_cast<uint32_t>(dpp_quad_int(static_cast<int>(amax), 2)));
  uint32_t sgn[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    sgn[h] = ((xs[4 * h] >> 8) & 0x80u) | (xs[4 * h + 1] & 0x8000u) |
             ((xs[4 * h + 2] << 8) & 0x800000u) | ((xs[4 * h + 3] << 16) & 0x80000000u);
  if (amax >= 0x7F80u) {  // NaN or inf in the block
    words[0] = sgn[0] | 0x7F7F7F7Fu;
    words[1] = sgn[1] | 0x7F7F7F7Fu;
    return 0xFFu;
  }
  if (amax == 0u) {       // all (signed) zeros
    words[0] = sgn[0];
    words[1] = sgn[1];
    return 0x00u;
  }
  const int ex = static_cast<int>(amax >> 7);
  const int E = ex ? ex - 127 : -133 + (31 - __clz(static_cast<int>(amax & 0x7Fu)));
  const int e_s = E - 8 < -127 ? -127 : E - 8;  // E <= 127, so e_s <= 119
  // Element codes: q = x * 2^-e_s is exact in binary32 whenever it can
  // matter (|q| >= 2^-126; anything smaller encodes to a signed zero either
  // way); the median with +-448 gives the saturation; v_cvt_pk_fp8_f32 then
  // rounds to nearest even onto the E4M3FN grid (subnormal step 2^-9).
  // Checked bit for bit against the CPU oracle for every bf16 value under
  // every scale exponent a block can produce.
  const float scale = __uint_as_float(static_cast<uint32_t>(127 - e_s) << 23);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q[j] = __builtin_amdgcn_fmed3f(__uint_as_float(xs[4 * h + j] << 16) * scale, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
    words[h] = static_cast<uint32_t>(w);
  }
  return static_cast<uint32_t>(e_s + 127);
}

// Stores of one chunk's codes (8 bytes) and, from lane 16i, the scale bytes
// of the four quads 16i, 16i+4, 16i+8, 16i+12 (consecutive blocks).  All 64
// lanes must call it (the scale gather reads other lanes); `valid` masks the
// stores of lanes past the end.  nchunks is a multiple of 4.
__device__ __forceinline__ void mx_store(uint8_t* elem, uint8_t* scale, uint64_t c,
                                         uint64_t nchunks, bool valid,
                                         const uint32_t words[2], uint32_t sbyte) {
  const int lane = static_cast<int>(threadIdx.x & 63);
  if (valid)
    store_stream<false>(reinterpret_cast<u32x2*>(elem + c * kVec), u32x2{words[0], words[1]});
  const uint32_t s1 = dpp_row_shl(sbyte, 4);
  const uint32_t s2 = dpp_row_shl(sbyte, 8);
  const uint32_t s3 = dpp_row_shl(sbyte, 12);
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

// ----------------------------------------------------------- the gate ----

struct Gate {
  float coef;
  int32_t skip;
};

// Words of the accumulators' normalised sum: 13 digits of 32 bits with up
// to 32 pending carry bits each, summed over up to 2^31 accumulators, stay
// below 2^(32*16).
constexpr int kSumWords = 16;

// Sum of the accumulators as a normalised 512-bit integer (16 x 32 bits).
__device__ inline void acc_total(const zero_norm_acc* accs, int n_accs, uint32_t w[kSumWords],
                                 uint64_t& nonfinite) {
#pragma unroll
  for (int k = 0; k < kSumWords; ++k) w[k] = 0u;
  nonfinite = 0;
  for (int a = 0; a < n_accs; ++a) {
    uint32_t t[kDigits + 1];
    uint64_t carry = 0;
#pragma unroll
    for (int k = 0; k < kDigits; ++k) {
      const uint64_t x = accs[a].digit[k];
      const uint64_t s = (x & 0xFFFFFFFFull) + carry;
      t[k] = static_cast<uint32_t>(s);
      carry = (x >> 32) + (s >> 32);
    }
    t[kDigits] = static_cast<uint32_t>(carry);
    uint64_t c2 = 0;
#pragma unroll
    for (int k = 0; k < kSumWords; ++k) {
      const uint64_t s = static_cast<uint64_t>(w[k]) + (k <= kDigits ? t[k] : 0u) + c2;
      w[k] = static_cast<uint32_t>(s);
      c2 = s >> 32;
    }
    nonfinite += accs[a].nonfinite;
  }
}

// RNE_binary64(X * 2^-128) for X held in w[0..kSumWords).
__device__ inline double fixed_to_double(const uint32_t w[kSumWords]) {
  int top_word = -1;
#pragma unroll
  for (int k = kSumWords - 1; k >= 0; --k)
    if (top_word < 0 && w[k] != 0u) top_word = k;
  if (top_word < 0) return 0.0;
  const int top = 32 * top_word + (31 - __clz(static_cast<int>(w[top_word])));
  // bit(pos) of the 512-bit number
  auto bit = [&](int pos) -> uint32_t {
    return pos < 0 ? 0u : ((w[pos >> 5] >> (pos & 31)) & 1u);
  };
  uint64_t mant = 0;
  int exp2;
  if (top <= 52) {
    // exact: X < 2^53
    mant = (static_cast<uint64_t>(w[1]) << 32) | w[0];
    exp2 = 0;
  } else {
    const int s = top - 52;  // lowest kept bit
    // bits [s, s+52] via a funnel over three words
    const int i = s >> 5, off = s & 31;
    const uint64_t lo = (static_cast<uint64_t>(w[i + 1]) << 32) | w[i];
    const uint64_t hi = (i + 2 < kSumWords) ? w[i + 2] : 0u;
    mant = off ? ((lo >> off) | (hi << (64 - off))) : lo;
    mant &= (1ull << 53) - 1ull;
    const uint32_t round_bit = bit(s - 1);
    uint32_t sticky = 0;
    // everything below s-1
    const int below = s - 1;  // number of bits under the rounding bit
    for (int k = 0; k < kSumWords && 32 * k < below; ++k) {
      const int hi_bits = below - 32 * k;  // bits of word k that are below
      const uint32_t mask = hi_bits >= 32 ? 0xFFFFFFFFu : ((1u << hi_bits) - 1u);
      sticky |= (w[k] & mask);
    }
    exp2 = s;
    if (round_bit && (sticky != 0u || (mant & 1ull))) {
      mant += 1;
      if (mant == (1ull << 53)) {
        mant >>= 1;
        exp2 += 1;
      }
    }
  }
  return __builtin_amdgcn_ldexp(static_cast<double>(mant), exp2 - 128);
}

// The step's gate.  Skip when the check is on and any element of the global
// gradient is non-finite.  Otherwise the clip coefficient: 1 without
// clipping; 0 when clipping and a non-finite element makes the global norm
// infinite (max_norm / (inf + 1e-6)); else max_norm / (norm + 1e-6) in
// binary64, clamped to 1 and rounded once to binary32.
__device__ inline Gate evaluate_gate(const zero_norm_acc* accs, int n_accs, double max_norm,
                                     int check_overflow) {
  Gate g{1.0f, 0};
  if (n_accs <= 0 || accs == nullptr) return g;
  uint32_t w[kSumWords];
  uint64_t nonfinite;
  acc_total(accs, n_accs, w, nonfinite);
  if (check_overflow && nonfinite > 0) {
    g.skip = 1;
    return g;
  }
  if (max_norm > 0.0) {
    if (nonfinite > 0) {
      g.coef = 0.0f;
      return g;
    }
    const double sumsq = fixed_to_double(w);
    const double norm = __builtin_sqrt(sumsq);
    const double denom = norm + 1e-6;
    const double c = max_norm / denom;
    g.coef = (c < 1.0) ? static_cast<float>(c) : 1.0f;
  }
  return g;
}

}  // namespace zs
