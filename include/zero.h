/*
 * zero.h -- C ABI of libzero.so: one data-parallel rank's share of a ZeRO
 * (Zero Redundancy Optimizer, arXiv 1910.02054) mixed-precision training step,
 * on one AMD Instinct MI355X (gfx950).
 *
 * The operation, as the pages on ZeRO describe it:
 *   - every rank keeps only its own block of the training state for the long
 *     term (ZeRO mind-map page, paperbridge.wiki, section "shrink the problem:
 *     four GPUs": GPU 1 keeps block A, GPU 2 block B, and so on);
 *   - after backward, gradients are merged across ranks and split again so
 *     that each rank keeps the part it owns (same page, glossary entry
 *     "reduce-scatter", and the section on how a GPU that keeps a quarter of
 *     the state computes); the owner updates that part with mixed-precision
 *     Adam, whose state is 16-bit parameters plus fp32 master weights, first
 *     and second moments (ZeRO concept page, papers.lqhl.me, section "why it
 *     is needed");
 *   - parameters are exchanged so every rank briefly holds them in full
 *     (glossary entry "all-gather"); in Stage 3 this happens per layer, in
 *     forward/backward order, and the copy is freed afterwards (concept page,
 *     "three stages" table);
 *   - collectives run over buckets (concept page, design trade-off 1).
 *
 * On one GPU the N_d ranks are simulated: their gradient contributions are
 * resident buffers, and this library computes the arithmetic of reduce-scatter
 * for the owned partition, the Adam update, and the local layout of
 * all-gather.  No inter-GPU transfer happens here.
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device addresses owned by the caller.  The
 *     library never allocates device memory.
 *   - Host pointer arrays are read before the call returns and not kept.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; no call synchronises.  The caller keeps every buffer
 *     alive until the stream has drained.
 *   - Arguments are checked before anything is launched.  On a failed check
 *     nothing is launched and a negative zero_status is returned; the text of
 *     the last failure on the calling thread is available from
 *     zero_last_error().  The library never aborts, never prints, and lets no
 *     C++ exception cross the ABI.
 *   - Element offsets and counts are int64.  "16-bit" means ZERO_F16 or
 *     ZERO_BF16.  Buffers must be aligned to their element size.  When every
 *     base address is 16-byte aligned, the step and the reduction run the
 *     vector kernel on each piece of the shard whose offsets are multiples
 *     of 4 elements, after at most 3 leading elements; other pieces run an
 *     element kernel with the same arithmetic.
 */
#ifndef ZERO_H_
#define ZERO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ZERO_API __attribute__((visibility("default")))
#else
#define ZERO_API
#endif

/* Largest number of simulated ranks one fused launch reads directly. */
#define ZERO_MAX_RANKS 128

typedef struct zero_plan_s* zero_plan_t;

typedef enum zero_dtype { ZERO_F32 = 0, ZERO_F16 = 1, ZERO_BF16 = 2 } zero_dtype;

typedef enum zero_status {
  ZERO_OK = 0,
  ZERO_EINVAL = -1,          /* bad argument: null, range, alignment, overlap */
  ZERO_EUNSUPPORTED = -2,    /* valid but not supported (dtype pair, N_d) */
  ZERO_ENOMEM = -3,          /* host allocation failed */
  ZERO_EHIP = -4             /* a HIP launch failed; see zero_last_error() */
} zero_status;

/* Adam hyper-parameters, as decimal values.  The step's fp32 constants are
 * computed from them in fp64 and rounded once to fp32: beta1, 1-beta1, beta2,
 * 1-beta2, 1-beta1^t, 1-beta2^t (pow), lr, eps, grad_scale. */
typedef struct zero_adam_hyper {
  double lr;
  double beta1;
  double beta2;
  double eps;
  double grad_scale;   /* multiplies the rank sum; 1/N_d gives the mean */
} zero_adam_hyper;

/* The N_d ranks' gradient contributions for the owner's partition.
 * ptrs[q] is rank q's buffer, either
 *   is_full[q] == 0: a compact shard-local slice of shard_total elements
 *                    (what reduce-scatter hands the owner; Stage 2 and 3), or
 *   is_full[q] == 1: rank q's whole padded flat gradient buffer of psi_pad
 *                    elements, read at the owner's ranges (Stage 1, where
 *                    gradients stay replicated).
 * is_full may be NULL (all compact).  Gradients are read only. */
typedef struct zero_grad_src {
  int32_t dtype;             /* ZERO_F16 or ZERO_BF16 */
  int32_t n;                 /* must equal the plan's n_d */
  const void* const* ptrs;   /* host array of n device pointers */
  const uint8_t* is_full;    /* host array of n flags, or NULL */
} zero_grad_src;

/* Library version: major * 10000 + minor * 100 + patch. */
ZERO_API int32_t zero_version(void);

/* Text of the last non-OK status returned on the calling thread ("" if none). */
ZERO_API const char* zero_last_error(void);

/*
 * zero_plan -- layout of the flat buckets and of every rank's shard.
 * Follows the mind-map page's four-GPU example (rank i owns the i-th
 * contiguous block) and the concept page's buckets.
 *
 *   psi          total parameters; must equal the sum of tensor_numel.
 *   n_d          simulated data-parallel ranks, >= 1.
 *   tensor_numel host array of n_tensors sizes (>= 0), in list order.
 *   bucket_cap   elements per bucket; 0 = one bucket.  Tensors are taken in
 *                list order and never split; a new bucket starts when the next
 *                tensor would push a non-empty bucket past the cap, so a tensor
 *                larger than the cap sits alone.
 *   shard_align  elements, >= 1.  Each bucket is zero-padded at its end to a
 *                multiple of n_d * shard_align, so every rank's slice
 *                S_b = padded_b / n_d is a multiple of shard_align.
 *   out          receives the plan (host memory, immutable, owned by the caller
 *                until zero_plan_destroy).  A plan may be shared by concurrent
 *                calls.
 * The padded layout must satisfy psi_pad * 4 <= INT64_MAX (fp32 buffers stay
 * byte-addressable in int64).
 * Rank r owns [flat_off_b + r*S_b, flat_off_b + (r+1)*S_b) of bucket b; its
 * shard is the concatenation of those ranges over buckets (shard_total
 * elements), bucket b's part starting at shard_off_b.
 * Errors: EINVAL for n_d < 1, shard_align < 1, bucket_cap < 0, n_tensors < 0,
 * negative sizes, sizes not summing to psi, a null pointer, or a padded
 * layout beyond that bound; ENOMEM.
 */
ZERO_API zero_status zero_plan(int64_t psi, int32_t n_d, const int64_t* tensor_numel, int32_t n_tensors,
                      int64_t bucket_cap, int32_t shard_align, zero_plan_t* out);

ZERO_API void zero_plan_destroy(zero_plan_t plan);

/* Plan queries.  Any output pointer may be NULL.  EINVAL on a null plan or an
 * index out of range. */
ZERO_API zero_status zero_plan_info(zero_plan_t plan, int64_t* psi_pad, int64_t* shard_total,
                           int32_t* n_buckets, int32_t* n_d);
ZERO_API zero_status zero_plan_bucket(zero_plan_t plan, int32_t b, int64_t* flat_off, int64_t* numel,
                             int64_t* padded, int64_t* shard_numel, int64_t* shard_off);
ZERO_API zero_status zero_plan_tensor(zero_plan_t plan, int32_t t, int32_t* bucket, int64_t* flat_off);

/*
 * zero_flatten_workspace_bytes -- device workspace zero_flatten needs for this
 * plan.  Always 0: every copy table travels in the kernel arguments (split
 * over several launches when a plan has many tensors), so flatten needs no
 * device memory of its own.  Kept so that callers can size a workspace
 * without knowing that.
 */
ZERO_API size_t zero_flatten_workspace_bytes(zero_plan_t plan);

/*
 * zero_flatten -- pack the ragged tensor list into the padded flat buckets
 * (concept page, design trade-off 1: collectives run over buckets).
 *   tensors    host array of n_tensors device pointers; tensors[t] holds
 *              tensor_numel[t] contiguous elements (may be NULL when that is 0).
 *   dt         element type of tensors and flat (ZERO_F32, ZERO_F16, ZERO_BF16).
 *   flat       device buffer of psi_pad elements.  Tensor t lands at its plan
 *              offset; every padding element is written as zero.
 *   workspace, ws_bytes  device workspace of zero_flatten_workspace_bytes()
 *              bytes; may be NULL and 0 (the size is 0).  Not touched.
 * A bit copy.  Errors: EINVAL for nulls, misaligned pointers, or flat
 * overlapping a tensor.
 */
ZERO_API zero_status zero_flatten(zero_plan_t plan, const void* const* tensors, zero_dtype dt, void* flat,
                                  void* workspace, size_t ws_bytes, void* stream);

/*
 * zero_shard_reduce -- the arithmetic of reduce-scatter for the owner's
 * partition (mind-map page, glossary entry "reduce-scatter").
 *   out[j] = ((g_0[j] + g_1[j]) + ... + g_{n_d-1}[j]) * f32(grad_scale)
 * for every j of the owner's shard (padding included), in fp32, ranks folded
 * in the fixed order 0..n_d-1 whatever `rank` is.
 *   rank   owning rank, 0 <= rank < n_d.
 *   src    the n_d contributions (see zero_grad_src).
 *   out    device fp32 buffer of shard_total elements (shard-local layout).
 * Any n_d is supported (ranks beyond ZERO_MAX_RANKS are folded by further
 * launches that continue from `out`, which keeps the same order).  Stores may
 * be held for a device-wide write window (zero_set_write_window); the result
 * never depends on it.
 * Errors: EINVAL for a bad rank, src->n != n_d, nulls, misalignment, out
 * overlapping a gradient buffer; EUNSUPPORTED for a non-16-bit dtype.
 */
ZERO_API zero_status zero_shard_reduce(zero_plan_t plan, int32_t rank, const zero_grad_src* src,
                                       double grad_scale, float* out, void* stream);

/*
 * zero_adam_step -- the owner's mixed-precision Adam update of its shard
 * (concept page, "why it is needed": fp32 master weights, first and second
 * moments, 16-bit parameters), fused with the reduction above and with the
 * local half of all-gather.  The update rule is the textbook Adam (Kingma &
 * Ba 2015, Algorithm 1), one fp32 operation per line, no FMA:
 *     g  = reduced gradient (as zero_shard_reduce computes it)
 *     m  = b1*m + c1*g            v = b2*v + c2*(g*g)
 *     mh = m / bc1                vh = v / bc2
 *     w  = w - lr * (mh / (sqrt(vh) + eps))
 *     p  = round-to-nearest-even 16-bit value of w
 *   rank        owning rank, 0 <= rank < n_d.
 *   hp          hyper-parameters (host struct).
 *   t           step number, >= 1 (bias corrections use beta^t).
 *   slices      the n_d gradient contributions (fused path, n_d <=
 *               ZERO_MAX_RANKS), or NULL to read `reduced` instead.
 *   reduced     device fp32 buffer of shard_total elements from
 *               zero_shard_reduce (grad_scale is then not applied again);
 *               ignored when slices is non-NULL.
 *   master, m, v  device fp32 buffers of shard_total elements, updated in
 *               place; they must not overlap each other, param_dst or any
 *               gradient buffer.
 *   param_dst   device 16-bit buffer receiving the updated parameters:
 *               dst_is_full != 0: the full flat parameter buffer (psi_pad
 *               elements), written only at the owner's ranges (Stage 1/2);
 *               dst_is_full == 0: the rank's resident parameter shard
 *               (shard_total elements, Stage 3).
 *   param_dt    ZERO_F16 or ZERO_BF16.
 * With slices, the kernel may hold its stores for a device-wide write window
 * (zero_set_write_window); the results never depend on it.
 * Performance: slices written just before the step with ordinary cached
 * stores slow it by 15-17% on MI355X; written with non-temporal stores (as
 * zero_shard_reduce, zero_flatten and zero_gather_pack write their outputs)
 * they cost nothing.  A producer of the slices should store them
 * non-temporally; where it cannot, zero_set_warm_read(1) recovers most of
 * the loss (3.14-3.22 -> 2.79-2.89 ms for 7.5B at N_d = 64).  Where the
 * slices sit matters too: every wave reads the same offset of all n_d slices
 * at once, and slices a power of two apart (say 256 MiB) put those reads on
 * the same HBM channels, which costs the step 4-6%; staggering them by 1-4
 * KiB, or packing them back to back, avoids it.  For about a second after a
 * large release of device memory (about 1 s per 30 GB, e.g. an emptied
 * allocator cache) the step runs 2-5% slower; keep its buffers allocated
 * from step to step.
 * Errors: EINVAL for a bad rank, t < 1, nulls, misalignment, src->n != n_d,
 * overlapping outputs; EUNSUPPORTED for non-16-bit types or for the fused
 * path with n_d > ZERO_MAX_RANKS (use zero_shard_reduce, then reduced).
 */
ZERO_API zero_status zero_adam_step(zero_plan_t plan, int32_t rank, const zero_adam_hyper* hp, int64_t t,
                           const zero_grad_src* slices, const float* reduced, float* master,
                           float* m, float* v, void* param_dst, zero_dtype param_dt,
                           int32_t dst_is_full, void* stream);

/*
 * zero_gather_pack -- the local layout of all-gather: materialise the full
 * flat buffer from all n_d shards (mind-map page, glossary entry
 * "all-gather"; Stage 3 materialises one layer at a time, concept page,
 * "three stages" table).
 *   shards  host array of n_d device pointers, each shard_total elements.
 *   dt      element type (ZERO_F32, ZERO_F16, ZERO_BF16).
 *   full    device buffer of psi_pad elements; rank q's part of bucket b goes
 *           to [flat_off_b + q*S_b, flat_off_b + (q+1)*S_b).
 * A bit copy.  Errors: EINVAL for nulls, misalignment, full overlapping a shard.
 */
ZERO_API zero_status zero_gather_pack(zero_plan_t plan, const void* const* shards, zero_dtype dt, void* full,
                             void* stream);

/*
 * zero_reshard -- re-lay out a sharded per-element state for a different
 * data-parallel degree or bucketing: the shard of rank dst_rank under dst_plan,
 * assembled from all shards under src_plan.  The sharded optimizer state must
 * survive a change of parallel degree -- a rank-local checkpoint restored at
 * another N_d (concept page, design trade-off 4 and the checklist item on
 * restoring rank-local shards after the parallel degree changes).
 *   src_plan, dst_plan  plans over the SAME tensor list (sizes, order); n_d,
 *               bucket_cap and shard_align may differ.
 *   dst_rank    0 <= dst_rank < dst n_d.
 *   src_shards  host array of src n_d device pointers, each src shard_total
 *               elements (shard-local layout).
 *   dt          element type (ZERO_F32 for master/m/v, 16-bit for params).
 *   dst_shard   device buffer of dst shard_total elements: every real element
 *               is copied from the source rank that owns the same tensor
 *               element; padding is written as zero.
 * A bit copy.  Errors: EINVAL for nulls, different tensor lists, a bad rank,
 * misalignment, or dst_shard overlapping a source shard.
 */
ZERO_API zero_status zero_reshard(zero_plan_t src_plan, zero_plan_t dst_plan, int32_t dst_rank,
                                  const void* const* src_shards, zero_dtype dt, void* dst_shard,
                                  void* stream);

/*
 * zero_set_write_window -- scheduling of the stores of zero_shard_reduce and
 * of the fused zero_adam_step (not an operation of the pages: a tuning knob of
 * this library; results are bit-identical whatever it is set to).
 * The fused step reads about ten bytes of gradient for each byte it writes.
 * With a write window, a wave whose results are ready holds its stores until
 * the GPU's constant-rate real-time counter is within the first open_ticks of
 * a period_ticks-long period, and a wave about to issue its first gradient
 * loads waits until that opening has passed, so the device's writes reach HBM
 * in bursts rather than as a thin stream between the reads.  A tick is one count of
 * that counter at the rate the device reports as hipDeviceAttributeWallClockRate
 * (100 MHz on MI355X: 10 ns).
 *   period_ticks  -1: automatic (the default): the library picks the window
 *                 per launch from the rank count, the launch size, the
 *                 kernel's occupancy and the counter's rate, and uses none for
 *                 small launches;
 *                  0: no window, stores issue as soon as results are ready;
 *                 1..100000: this period for every fused or reduce launch.
 *   open_ticks    1..period_ticks when period_ticks > 0; ignored otherwise.
 * Scope: this sets the PROCESS-WIDE DEFAULT, read by launches issued after the
 * call on every stream that has no setting of its own
 * (zero_set_stream_write_window).  The window assumes the step has HBM to
 * itself while it runs; beside other memory-heavy work (a collective or a
 * copy on another stream) it gains little or nothing, and a stream whose step
 * runs so can turn its own window off with
 * zero_set_stream_write_window(stream, 0, 0) rather than change the default
 * for everyone (measured with a concurrent copy: from 1.2% faster to no
 * difference).  Safe to call from any thread.  Adam from a `reduced`
 * buffer, the element-wise (unaligned) kernels and the copy kernels never
 * wait.
 * Errors: EINVAL for values outside these ranges (the setting is unchanged).
 */
ZERO_API zero_status zero_set_write_window(int64_t period_ticks, int64_t open_ticks);

/*
 * zero_set_warm_read -- a read of the step's own buffers just before it
 * (not an operation of the pages: a tuning knob of this library; results are
 * bit-identical whether it is on or off).  With enable = 1, every fused
 * zero_adam_step and every zero_shard_reduce that reads at least 1 GiB of
 * gradients first reads up to 256 MiB of its fp32 state (master, then m, then
 * v) or of its fp32 output with ordinary cached loads, on the same stream,
 * storing nothing.  MI355X's 256 MB memory-side
 * Infinity Cache keeps the last lines written with ordinary stores dirty;
 * when the gradient slices were just written that way (as a collective or a
 * backward kernel may write them), their write-backs otherwise fall among the
 * step's reads and cost it 15-17% (7.5B, N_d = 64).  The warm-up read moves them
 * before the step: measured, the step is then ~11% faster (7.5% for a Stage-3
 * layer, 3% for 13B at N_d = 16), and the reduction ~11%.  When the slices are
 * already clean (written non-temporally, as zero_shard_reduce and the copies
 * write) it costs the step 1-2% and the reduction 2%.  enable = 0 (the
 * default): no warm-up read.  The buffers read must be 16-byte aligned for it
 * to run.  Process-wide; read by calls issued
 * after it, from any thread.  Errors: EINVAL for any other value.
 */
ZERO_API zero_status zero_set_warm_read(int32_t enable);

/*
 * zero_set_stream_write_window -- the same setting for launches on one
 * stream only; it takes precedence over the process-wide default for every
 * zero_shard_reduce and fused zero_adam_step call issued on that stream
 * afterwards, from any thread.
 *   stream        the hipStream_t the calls are issued on (NULL = the default
 *                 stream).
 *   period_ticks  -2: remove the stream's setting (the default applies
 *                 again); -1: automatic; 0: no window; 1..100000: as above.
 *   open_ticks    as above.
 * The library keeps only the stream handle (host memory); remove the setting
 * before destroying the stream if its handle may be reused.  Safe to call
 * from any thread.  Errors: EINVAL for values outside these ranges (the
 * setting is unchanged); ENOMEM.
 */
ZERO_API zero_status zero_set_stream_write_window(void* stream, int64_t period_ticks, int64_t open_ticks);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_H_ */
