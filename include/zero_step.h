/*
 * zero_step.h -- C ABI of libzero_step.so: one data-parallel rank's sharded
 * mixed-precision optimizer step on a flat parameter vector, for MI355X
 * (gfx950).
 *
 * The step this library computes, and where its pieces come from:
 *   - The whole model is one flat vector; rank r of P owns the contiguous
 *     shard [r*S, (r+1)*S) (Zero_From_Scratch, outline item on the flat
 *     parameter vector and the three collectives).
 *   - Per weight the training state is a bf16 parameter, a bf16 gradient, an
 *     fp32 master copy and two fp32 Adam moments: 16 bytes (Zero_From_Scratch,
 *     outline item on what is stored per weight; DeepSpeed documentation
 *     review, second paragraph, on the master copy and the two moments).
 *   - The rank sums its shard over the P gradient replicas -- the arithmetic
 *     half of reduce-scatter -- and averages; reduce-scatter followed by
 *     all-gather equals all-reduce, so the shards stepped separately equal
 *     the single-GPU step (Zero_From_Scratch, outline items on data parallel
 *     averaging and on the identity between the three collectives).
 *   - The fused AdamW update (Adam: Kingma & Ba, ICLR 2015, Algorithm 1;
 *     decoupled weight decay: Loshchilov & Hutter, ICLR 2019, Algorithm 2)
 *     runs as one streaming pass, because a chain of separate elementwise
 *     kernels pays a trip to memory per operation (Zero_From_Scratch, outline
 *     item on the unfused chain and its trips to memory).
 *   - The bf16 parameter shard it writes is the all-gather payload; it can be
 *     packed to MXFP8 (E4M3 elements, one E8M0 scale per 32) to halve the
 *     wire bytes (Zero_From_Scratch, outline item on MXFP8; OCP Microscaling
 *     Formats v1.0, sections 5 and 6).
 *   - Gradients are handled in buckets: a reduce call may cover any 32-aligned
 *     sub-range and the norm state of all buckets adds up (Zero_From_Scratch,
 *     outline item on sending gradients bucket by bucket).
 *
 * Conventions for every entry point:
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *     default stream) and is asynchronous: a return of ZERO_OK means the
 *     kernels were launched.  Faults inside them surface at the caller's next
 *     synchronisation.
 *   - Every device pointer is memory of the current HIP device, on which the
 *     kernels are launched (`stream` must belong to it too).
 *   - The caller owns every buffer.  The library allocates nothing, never
 *     synchronises, and lets no C++ exception escape.  It keeps no state
 *     between calls, except zero_shard_reduce_noalloc's static per-device
 *     slots (described there).
 *   - Alignment (ZERO_EALIGN otherwise): every device array and every
 *     zero_norm_acc must be 16-byte aligned; the exceptions are the
 *     per-block scale bytes of MXFP8-stored replicas (any alignment), the
 *     int32/float scalar outputs (4 bytes) and the int64 step counter (8).
 *     Outputs must not overlap inputs, except master/m/v, which are updated
 *     in place.
 *   - Element counts are size_t; n == 0 is a valid no-op returning ZERO_OK.
 *     A call that adds to a norm accumulator takes n <= 2^37 (ZERO_ESIZE
 *     beyond): that is the accumulator's capacity.
 *   - Arithmetic is IEEE binary32/binary64 with round to nearest even and
 *     denormals kept; every sum runs in one fixed order, so results are
 *     bitwise reproducible and independent of grid shape.
 */
#ifndef ZERO_STEP_H
#define ZERO_STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_ABI_VERSION 5
#define ZERO_MAX_REPLICAS 64

/* Element types of gradient replicas.  ZERO_MXFP8 replicas (E4M3 codes plus
 * one E8M0 scale byte per 32 elements) are accepted by zero_shard_reduce_mx
 * and zero_shard_reduce_mx_ws only. */
enum { ZERO_F32 = 0, ZERO_BF16 = 1, ZERO_MXFP8 = 2 };

/* Status codes. */
enum {
  ZERO_OK = 0,
  ZERO_EINVAL = -1, /* null required pointer, P outside [1,64], bad dtype,
                       step < 1, conflicting or missing gradient source */
  ZERO_EALIGN = -2, /* a pointer breaks the alignment rule above */
  ZERO_ESIZE = -3,  /* MXFP8 pack with n % 32 != 0, n > 2^37 in a call
                       that adds to a norm accumulator, or a workspace below
                       ZERO_REDUCE_WORKSPACE_BYTES */
  ZERO_EHIP = -4    /* the HIP runtime reported a launch error */
};

/* Exact, order-independent sum of squares of a gradient, plus its count of
 * non-finite values.  128 bytes in device memory, 16-byte aligned; the
 * caller zeroes it (zero_norm_acc_clear) before the first call that adds to
 * it.
 *
 * The sum is X * 2^-128 with the non-negative integer
 *   X = sum_k digit[k] * 2^(32k)            (k = 0..12; carries pending).
 * Each call splits its range into 32-element groups aligned to the range
 * start (a short last group is padded with +0).  Per group, with g the
 * averaged, unscaled gradient in binary32 and q_i = g_i^2 in binary64
 * (exact), a_j = q_{8j} + ... + q_{8j+7} summed left to right and
 * S = (a_0 + a_1) + (a_2 + a_3); floor(S * 2^128) is added to X exactly.
 * A non-finite g_i counts in `nonfinite` and adds 0.  Every finite group
 * counts: S < 2^261 for finite binary32 values, so floor(S * 2^128) < 2^389
 * fits the 13 digits, each of which receives one piece below 2^32 per
 * group.  Integer addition makes X the same for any grid, bucket split or
 * rank order, and accumulators of different ranks or buckets combine by
 * adding their fields (the norm all-reduce of a multi-GPU run).  Capacity:
 * at most 2^37 elements in total per accumulator (2^32 groups, so no digit
 * wraps).  reserved[] stays zero. */
typedef struct zero_norm_acc {
  uint64_t digit[13];
  uint64_t nonfinite;
  uint64_t reserved[2];
} zero_norm_acc;

/* Workspace of zero_shard_reduce_ws and zero_shard_reduce_mx_ws: 512
 * accumulator slots.  The reduce of 4 or more replicas then runs on a
 * one-shot grid (a few tiles per workgroup, in address order) whose
 * workgroups add their norm state to the slots, and a one-workgroup kernel
 * launched after it adds the slots to `acc` and zeroes them again.  Results
 * are bitwise those of the workspace-free call.  Measured on MI355X it pays
 * for whole multi-GB shards; for bucket-sized calls (25e6 elements) the
 * extra launch made it slower.  Device memory of at least
 * ZERO_REDUCE_WORKSPACE_BYTES, 16-byte aligned, zeroed by the caller before
 * its first use (zero_norm_acc_clear on it as ZERO_REDUCE_WORKSPACE_BYTES /
 * 128 accumulators does that) and left zeroed by every call that returns
 * ZERO_OK; after any other status, zero it again before reusing it.  Calls
 * that share a workspace must not run concurrently (order them on one
 * stream). */
#define ZERO_REDUCE_WORKSPACE_BYTES (128 * 512)

/* Zero n_accs accumulators with a fill kernel (safe inside stream capture). */
int zero_norm_acc_clear(zero_norm_acc *accs, int n_accs, void *stream);

/* f32(1 / (P * loss_scale)), the factor that averages P replicas and removes
 * a static loss scale, computed in binary64 and rounded once.  Host only. */
float zero_inv_scale(int P, double loss_scale);

/* Shard reduce: g[i] = (r_0[i] + r_1[i] + ... + r_{P-1}[i]) * inv_scale,
 * summed in binary32 in rank order 0..P-1 (the reduce half of
 * reduce-scatter, then the data-parallel average), plus the norm state of g.
 *   replicas  HOST array of P device pointers; replicas[k] is rank k's copy
 *             of the same n elements (for a bucket, the same offset into
 *             each replica).  dtype ZERO_F32 or ZERO_BF16.
 *   g_out     device fp32[n], or NULL to skip writing the averaged gradient.
 *   acc       device accumulator to add this range's norm state to, or NULL.
 * At least one of g_out and acc must be given. */
int zero_shard_reduce(const void *const *replicas, int P, int dtype, size_t n,
                      float inv_scale, float *g_out, zero_norm_acc *acc, void *stream);

/* The same reduce with a caller-owned workspace (ZERO_REDUCE_WORKSPACE_BYTES
 * above; workspace_bytes its size, ZERO_ESIZE if too small): the one-shot
 * form for whole shards.  Bitwise the same results. */
int zero_shard_reduce_ws(const void *const *replicas, int P, int dtype, size_t n,
                         float inv_scale, float *g_out, zero_norm_acc *acc,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Shard reduce of MXFP8-stored gradient replicas (the "12 percent off stored
 * state" of Zero_From_Scratch's outline item on MXFP8: bf16 gradients kept
 * as E4M3 codes plus one E8M0 scale per 32 elements, 1.03 instead of 2 bytes
 * per element).  Each element decodes exactly to
 *   x = e4m3_value(code) * 2^(scale - 127)   (binary32, exact; scale byte
 *   0xFF or a NaN code gives the quiet NaN 0x7FC00000 with the code's sign
 *   bit),
 * then g[i] = (x_0[i] + ... + x_{P-1}[i]) * inv_scale exactly as
 * zero_shard_reduce sums, with the same norm state.
 *   codes[k]   HOST array of P device pointers to uint8[n] E4M3 codes
 *              (16-byte aligned)
 *   scales[k]  HOST array of P device pointers to uint8[n/32] scale bytes
 *              (any alignment); for a bucket at element offset `lo` pass
 *              codes + lo and scales + lo/32.
 *   n % 32 == 0 (ZERO_ESIZE otherwise).  g_out / acc as zero_shard_reduce;
 *   the _ws form takes a workspace as zero_shard_reduce_ws. */
int zero_shard_reduce_mx(const uint8_t *const *codes, const uint8_t *const *scales,
                         int P, size_t n, float inv_scale, float *g_out,
                         zero_norm_acc *acc, void *stream);
int zero_shard_reduce_mx_ws(const uint8_t *const *codes, const uint8_t *const *scales,
                            int P, size_t n, float inv_scale, float *g_out,
                            zero_norm_acc *acc, void *workspace, size_t workspace_bytes,
                            void *stream);

/* The same reduce as zero_shard_reduce_ws for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the 512 norm slots live in a static
 * device array of this library (ZERO_REDUCE_WORKSPACE_BYTES = 64 KiB per
 * GPU, held from the first call on that GPU until the process ends) instead
 * of a caller workspace.  Nothing is allocated: the first call on a device,
 * with that device current, looks up that device's address of the array;
 * every call clears the slots with a fill kernel before the reduce and the
 * fold leaves them zero.  The array is not sized by n: n is limited only as
 * for every norm call (n <= 2^37, ZERO_ESIZE beyond).  All calls on one GPU
 * share the array, so calls that overlap on one GPU (concurrent streams,
 * host threads) race and give wrong norms: order them on one stream.
 * Arguments, results and status codes otherwise as zero_shard_reduce; the
 * results are bitwise those of zero_shard_reduce_ws. */
int zero_shard_reduce_noalloc(const void *const *replicas, int P, int dtype, size_t n,
                              float inv_scale, float *g_out, zero_norm_acc *acc,
                              void *stream);

/* Norm state of one buffer: adds the groups of g[i] = grad[i] * inv_scale
 * (grad fp32 or bf16, device) to acc, as zero_shard_reduce with P = 1 and
 * no output.  Used for a single replica (P = 1) or a materialised gradient
 * before a recompute-style update. */
int zero_grad_norm(const void *grad, int dtype, size_t n, float inv_scale,
                   zero_norm_acc *acc, void *stream);

/* Arguments of the fused AdamW step; all device pointers except `replicas`,
 * which is a HOST array of P device pointers. */
typedef struct zero_adamw_args {
  size_t n;                    /* shard elements */
  const float *grad_f32;       /* averaged fp32 gradient, or NULL ...       */
  const void *const *replicas; /* ... the P replicas, reduced in the step   */
  int P;                       /* replica count (fused source only)         */
  int dtype;                   /* replica dtype (fused source only)         */
  float inv_scale;             /* applied to the fused sum (fused only)     */
  float *master;               /* fp32[n], in place                         */
  float *m;                    /* fp32[n], first moment, in place           */
  float *v;                    /* fp32[n], second moment, in place          */
  uint16_t *param_bf16;        /* bf16[n] out (all-gather payload), or NULL */
  const zero_norm_acc *accs;   /* n_accs accumulators whose sum is the      */
  int n_accs;                  /* global norm state (NULL/0: none)          */
  double max_norm;             /* global-norm clip threshold; <= 0: off     */
  int check_overflow;          /* nonzero: skip the step on nonfinite > 0   */
  double lr, beta1, beta2, eps, weight_decay;
  int64_t step;                /* 1-based index of this applied update      */
  int32_t *skipped_out;        /* device int: 1 skipped, 0 applied; or NULL */
  uint8_t *mx_elem_out;        /* uint8[n]: MXFP8 codes of the new params,  */
  uint8_t *mx_scale_out;       /* uint8[n/32]: their scales; both or NULL   */
  int64_t *step_dev;           /* device int64, 8-byte aligned, or NULL:    */
                               /* the count t of updates applied so far.    */
                               /* When set, `step` is ignored, this call    */
                               /* applies update t + 1 with scalars derived */
                               /* on the device, and t advances by one on   */
                               /* the device unless the gate skips.  No     */
                               /* host round trip is left in the step, so a */
                               /* whole step can be captured in a graph.    */
} zero_adamw_args;

/* Fused AdamW step on n elements of fp32 master/m/v.
 * Gate (evaluated on the device from the accumulators, no host sync):
 *   nonfinite summed over accs > 0 and check_overflow -> nothing is written
 *   and *skipped_out = 1 (the caller then keeps `step`); otherwise
 *   coef = 1 if max_norm <= 0;
 *   coef = 0 if max_norm > 0 and nonfinite > 0 (a non-finite element makes
 *   the global norm infinite: max_norm / (inf + 1e-6) = 0);
 *   else sumsq = RNE_binary64(X * 2^-128), c = max_norm / (sqrt(sumsq) +
 *   1e-6) in binary64 and coef = c < 1 ? f32(c) : 1.
 * Scalars (binary64, each rounded once to binary32): b1 = f32(beta1),
 *   b2 = f32(beta2), omb1 = f32(1 - beta1), omb2 = f32(1 - beta2),
 *   beta^t by square-and-multiply over the bits of t from the least
 *   significant, step_size = f32(lr / (1 - beta1^t)),
 *   sqrt_bc2 = f32(sqrt(1 - beta2^t)), decay = f32(1 - lr * wd),
 *   eps = f32(eps).
 * Per element, binary32:
 *   g' = g * coef; m = fma(b1, m, omb1 * g'); v = fma(b2, v, (omb2 * g') * g')
 *   d = sqrt(v) / sqrt_bc2 + eps; u = m / d
 *   master = fma(-step_size, u, master * decay); param = bf16_rne(master)
 * where g comes from grad_f32, or from the replicas exactly as
 * zero_shard_reduce computes it.  NaN params become 0x7FC0 with the sign.
 * With mx_elem_out/mx_scale_out set (n % 32 == 0, else ZERO_ESIZE) the same
 * pass also writes the MXFP8 pack of the new bf16 params, bit for bit what
 * zero_mxfp8_pack would produce from param_bf16, without reading it back.
 * A skipped step writes none of the outputs.
 * With step_dev set, every workgroup derives the scalars above from the
 * counter it reads, in the same binary64 operations, so the bits equal those
 * of the host-counter form; a one-lane kernel queued after the update then
 * re-evaluates the gate and advances the counter if the step applied. */
int zero_adamw_step(const zero_adamw_args *args, void *stream);

/* The gate alone, for inspection: writes *coef_out (device float) and
 * *skip_out (device int32) exactly as zero_adamw_step evaluates them. */
int zero_step_gate(const zero_norm_acc *accs, int n_accs, double max_norm,
                   int check_overflow, float *coef_out, int32_t *skip_out,
                   void *stream);

/* MXFP8 pack of a bf16 vector (n % 32 == 0; ZERO_ESIZE otherwise).  For each
 * block b of 32 elements:
 *   any NaN or inf  -> scale_out[b] = 0xFF, every element 0x7F | sign;
 *   all zero        -> scale_out[b] = 0x00, every element a signed zero;
 *   otherwise E = floor(log2 amax), e_s = clamp(E - 8, -127, 127),
 *   scale_out[b] = e_s + 127 and elem_out[i] = E4M3FN(x_i * 2^-e_s) with
 *   round to nearest even (subnormal step 2^-9) and saturation at +-448.
 * elem_out: uint8[n]; scale_out: uint8[n/32]; both device. */
int zero_mxfp8_pack(const uint16_t *bf16_in, size_t n, uint8_t *elem_out,
                    uint8_t *scale_out, void *stream);

/* The same step as zero_shard_reduce (with its norm state) followed by
 * zero_adamw_step, computed as a chain of single-operation passes, each its
 * own kernel reading its operands from HBM and writing its result back:
 * s = sum of replicas; g = s * inv_scale; norm state of g; gate; g' = g*coef;
 * m; v; u = m / (sqrt(v)/sqrt_bc2 + eps); master; bf16 param; MXFP8 pack.
 * This is the unfused baseline of Zero_From_Scratch's outline item on the
 * trips to memory of an unfused chain: the results are bit for bit those of
 * the fused path, only the HBM traffic and launches differ.
 *   args       as for zero_adamw_step, except that `accs`/`n_accs` hold
 *              only the OTHER ranks' accumulators (this rank's own norm is
 *              computed inside the chain), MXFP8 outputs need param_bf16,
 *              and the step index comes from `step` (step_dev must be NULL).
 *   workspace  device scratch of at least zero_unfused_workspace_bytes(n,
 *              n_accs) bytes, 256-byte aligned; contents are overwritten.
 * ZERO_ESIZE if workspace_bytes is too small. */
size_t zero_unfused_workspace_bytes(size_t n, int n_accs);
int zero_adamw_step_unfused(const zero_adamw_args *args, void *workspace,
                            size_t workspace_bytes, void *stream);

int zero_abi_version(void);
const char *zero_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif
