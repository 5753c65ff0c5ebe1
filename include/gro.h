/*
 * gro.h -- placement-aware gradient reduction, global L2 norm, clipping and
 * fused AdamW for one MI355X (gfx950).  C ABI.
 *
 * The operation is the per-step gradient-ownership path of data- and
 * tensor-parallel training described in NeMo Automodel issue #3857,
 * "refactor(distributed): establish shared native TP replica ownership":
 *
 *   section "Why this needs separate work" -- a replicated parameter's local
 *     gradient means one of four things: complete (redundant compute; averaged
 *     over the TP ranks), partial (head- or sequence-sharded compute; summed),
 *     a local shard (never synchronised as a replica), or already reduced by
 *     another owner (not reduced again);
 *   section "Preserved prototype and evidence" -- FP32 reduction, BF16
 *     gradients, gradient accumulation including partial windows, clipping,
 *     Adam updates;
 *   section "Proposed scope and acceptance criteria" -- explicit
 *     replica/partial/shard semantics, exactly one reduction owner per
 *     parameter, unsupported compositions rejected, global norms, clipping
 *     on/off, accumulation over 1, >1 and trailing windows.
 *
 * Mixle v0.8.1 "Distributed Transformer Training", section "Backend split":
 * a request that cannot be executed fails before fitting -- here every check
 * happens on the host before any device work, so a failed call has no side
 * effects.  Section "Optimizer and checkpoint semantics": the optimizer
 * addresses parameters by names that stay fixed across wrapping -- here a
 * caller-chosen 64-bit param_id.
 *
 * One GPU holds the R rank contributions of a replicated parameter as R
 * stacked slots in its own HBM; the kernels do that GPU's share of the work.
 *
 * Conventions
 *  - Memory: the caller allocates every device buffer (acc, master, m, v, the
 *    BF16 parameter copy, the per-bucket gradient buffers and the workspace).
 *    The library never allocates or frees device memory and never calls a
 *    collective.  A plan owns only host tables.
 *  - Device pointers must be 16-byte aligned (256-byte for the workspace).
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  All device work is enqueued on it, asynchronously.  Use one
 *    stream per plan at a time.
 *  - Errors: functions return GRO_OK (0) or a negative GRO_E_* code and set
 *    a thread-local message (gro_last_error).  Validation precedes any device
 *    work.  Non-finite data is reported through gro_plan_get_norm's `finite`
 *    flag, not a return code, because device work is asynchronous.
 *  - Only gro_plan_bind, gro_plan_bind_static, gro_init_uniform and
 *    gro_plan_get_norm wait for the device.  The step's calls
 *    (gro_accumulate*, gro_reduce_norm, gro_clip_adamw) only enqueue kernels
 *    -- no allocation, no synchronization, no memory fill -- so a step may be
 *    captured in a HIP graph after binding and replayed; the replay repeats
 *    the captured arguments, the AdamW step count included.
 *  - Not thread-safe per plan; distinct plans may be used from distinct
 *    threads.
 */
#ifndef GRO_H
#define GRO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---- */
#define GRO_OK            0
#define GRO_E_INVALID    (-1)  /* null/misaligned pointer, bad size/shape/step/window, NaN max_norm */
#define GRO_E_PLACEMENT  (-2)  /* unknown placement, shard_index out of range, bad flags */
#define GRO_E_DUPLICATE  (-3)  /* a second owner for one param_id */
#define GRO_E_STATE      (-4)  /* unbound plan, window bookkeeping violated */
#define GRO_E_HIP        (-5)  /* HIP runtime or launch error */

/* ---- placements (what a rank-local gradient means) ---- */
#define GRO_REPLICATE 0  /* complete gradient on every rank: averaged over R */
#define GRO_PARTIAL   1  /* partial contribution per rank: summed over R */
#define GRO_SHARD     2  /* local shard owned by this rank: used as is */
#define GRO_REDUCED   3  /* already reduced by another owner: used as is */

/* ---- per-tensor flags ---- */
#define GRO_NO_DECAY  1u  /* no weight decay for this tensor */
#define GRO_FROZEN    2u  /* no gradient, not in the norm, not updated */
#define GRO_FP32_GRAD 4u  /* gradient contributions arrive in FP32 instead of BF16 */

/* ---- gradient element types (gro_tensor_layout / gro_bucket_info) ---- */
#define GRO_GRAD_BF16 0
#define GRO_GRAD_FP32 1

/* ---- owner classes reported by gro_plan_tensor / gro_plan_bucket ---- */
#define GRO_OWNER_MEAN          0
#define GRO_OWNER_SUM           1
#define GRO_OWNER_LOCAL_SHARD   2
#define GRO_OWNER_LOCAL_REDUCED 3
#define GRO_OWNER_EXCLUDED      4

#define GRO_MAX_NDIM 8

/* One parameter as this GPU sees it.  `shape` (host memory, `ndim`
 * entries, each >= 0; may be NULL when ndim == 0, a scalar) is read only
 * during gro_plan_create.  `shard_index` is this rank's index in [0, R) for
 * GRO_SHARD and must be -1 for the other placements. */
typedef struct gro_tensor_desc {
  int64_t param_id;
  const int64_t* shape;
  int32_t ndim;
  int32_t placement;
  int32_t shard_index;
  uint32_t flags;
} gro_tensor_desc;

typedef struct gro_plan gro_plan;

typedef struct gro_plan_info {
  int32_t R;
  int32_t n_tensors;
  int32_t n_buckets;
  int32_t chunk_elems;      /* elements per chunk (norm partial granularity) */
  int64_t n_chunks;
  int64_t n_flat;           /* elements to allocate for acc, master, m, v, BF16 copy */
  int64_t n_owned;          /* elements inside buckets (reduced, in the norm, updated) */
  int64_t bucket_elems;     /* bucket capacity the plan was created with */
  uint64_t workspace_bytes; /* device workspace gro_plan_bind needs */
} gro_plan_info;

/* The ownership row of one tensor plus where it lives in the flat arrays.
 * A tensor is contiguous in the flat arrays: [flat_offset, flat_offset+numel).
 * It spans buckets first_bucket .. first_bucket+n_buckets-1 (more than one
 * only when it is larger than the bucket capacity). */
typedef struct gro_tensor_layout {
  int64_t param_id;
  int64_t numel;
  int64_t flat_offset;      /* -1 when excluded */
  int32_t owner;            /* GRO_OWNER_* */
  int32_t slots;            /* rank contributions read per microbatch (0 if excluded) */
  int32_t divisor;          /* R for MEAN, 1 for SUM/LOCAL, 0 if excluded */
  int32_t in_norm;
  int32_t updated;
  int32_t decayed;
  int32_t first_bucket;     /* -1 when the tensor has no elements in a bucket */
  int32_t n_buckets;
  int32_t grad_dtype;       /* GRO_GRAD_BF16 or GRO_GRAD_FP32 */
} gro_tensor_layout;

/* A bucket: flat range [flat_base, flat_base+len) of one owner class, one
 * decay setting and one gradient type.  Its gradient buffer is
 * [slots][slot_stride] elements of that type (BF16 or FP32): element
 * flat_base+i of slot r is at index r*slot_stride + i. */
typedef struct gro_bucket_info {
  int64_t flat_base;
  int64_t len;
  int64_t slot_stride;
  int64_t first_chunk;
  int64_t n_chunks;
  int32_t owner;
  int32_t slots;
  int32_t decayed;
  int32_t grad_dtype;       /* GRO_GRAD_BF16 or GRO_GRAD_FP32 */
} gro_bucket_info;

/* AdamW hyper-parameters as the user states them (FP64).  Per-step scalars
 * are derived from them in FP64 and rounded once to FP32. */
typedef struct gro_adamw_hparams {
  double lr;
  double beta1;
  double beta2;
  double eps;
  double weight_decay;
} gro_adamw_hparams;

/* Build a plan.  Passages: NeMo Automodel issue #3857, section "Why this
 * needs separate work" (what a local gradient of a replicated parameter
 * means, per placement) and section "Proposed scope and acceptance criteria"
 * (explicit replica/partial/shard semantics, exactly one reduction owner,
 * unsupported compositions rejected); NeMo AutoModel "Model Parallelizer
 * API", section "Choose the Extension Point" (sharding units may be drawn as
 * groups of one dtype -- here buckets hold one gradient type).
 * First the ownership of every tensor from its placement, one owner per
 * param_id: duplicates -> GRO_E_DUPLICATE; bad placement/shard_index/flags
 * -> GRO_E_PLACEMENT; R < 1, n_tensors < 0, ndim out of [0,8], negative
 * dims, bucket_elems < 64 -> GRO_E_INVALID.  Then the layout: tensors
 * grouped by (owner class, decay, gradient type) in the order MEAN, SUM,
 * LOCAL_SHARD, LOCAL_REDUCED (decayed first, BF16 first), descriptor order
 * within a group, packed into buckets of at most bucket_elems elements; only
 * a tensor larger than the capacity is split.  Host only, deterministic.  On
 * success *out owns the host tables. */
int gro_plan_create(const gro_tensor_desc* tensors, int32_t n_tensors, int32_t R,
                    int64_t bucket_elems, gro_plan** out);

/* Free a plan's host tables (NULL is ignored).  Device memory is the caller's. */
void gro_plan_destroy(gro_plan* plan);

int gro_plan_get_info(const gro_plan* plan, gro_plan_info* info);
int gro_plan_tensor(const gro_plan* plan, int32_t i, gro_tensor_layout* out);
int gro_plan_bucket(const gro_plan* plan, int32_t b, gro_bucket_info* out);

/* Upload the plan's bucket and chunk tables into the caller's device
 * workspace (>= workspace_bytes, 256-byte aligned) on `stream`, and wait for
 * the copy.  Must precede the calls below; may be repeated (rebinding). */
int gro_plan_bind(gro_plan* plan, void* d_workspace, uint64_t bytes, void* stream);

/* Bytes of the library's own device workspace, one per GPU, used by
 * gro_plan_bind_static (enough for about 700,000 chunks, i.e. plans of up to
 * about 2.8e9 elements). */
#define GRO_STATIC_WORKSPACE_BYTES 16777216ull

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): gro_plan_bind on a
 * workspace the library holds itself -- a static device array of
 * GRO_STATIC_WORKSPACE_BYTES per GPU, kept until the process ends -- instead
 * of one the caller allocates.  Every later call of the plan behaves as
 * after gro_plan_bind; the caller still passes the accumulator, the states
 * and the gradient buffers.  Allocates nothing, frees nothing.
 *  - A plan whose workspace_bytes exceeds GRO_STATIC_WORKSPACE_BYTES:
 *    GRO_E_INVALID, nothing done.
 *  - All plans bound this way on one GPU share that GPU's array.  Binding
 *    waits for all work on the current device to finish, then overwrites
 *    the array; from then on a plan bound to it earlier is rejected with
 *    GRO_E_STATE until it is bound again.  Device calls of two plans that
 *    overlap on one GPU would race on the array, which is why only the
 *    last plan bound may use it.
 *  - Binding clears what must start at zero -- the norm's completion
 *    counters (every bind does) -- and the norm scalars; every other byte
 *    of the array is written by a kernel before one reads it.
 *  - Waits for its own upload, like gro_plan_bind.  Not for use inside a
 *    graph capture (it synchronizes); bind first, then capture. */
int gro_plan_bind_static(gro_plan* plan, void* stream);

/* Reduce + cast + accumulate one microbatch for buckets [b0, b1) -- NeMo
 * Automodel issue #3857, section "Why this needs separate work" (Replicate
 * contributions averaged, Partial summed, Shard and already-reduced used as
 * they are) and section "Preserved prototype and evidence" (an FP32
 * reduction hook on BF16 gradients, gradient accumulation).
 * d_grad_buckets: host array of b1-b0 device pointers; entry j is bucket
 * b0+j's BF16 gradient buffer [slots][slot_stride].  d_acc: FP32 [n_flat].
 * Per element: the slots are widened and summed in FP32 in slot order; MEAN
 * divides by R; micro_index 0 starts the window (acc = reduced), later
 * microbatches add (acc += reduced).  micro_index must equal the number of
 * microbatches this bucket has accumulated in the current window (0 restarts).
 * window_size > 0 announces the window length: on its last microbatch the
 * kernel also writes the chunks' norm partials (saving gro_reduce_norm a read
 * of acc); 0 = not known.  Gradient buffers are only read.  All buckets of
 * one window accumulate into one d_acc: starting buckets on another
 * accumulator while other buckets of the window are in progress is
 * GRO_E_STATE (a window ends with gro_clip_adamw or a rebind). */
int gro_accumulate(gro_plan* plan, int32_t b0, int32_t b1, const void* const* d_grad_buckets,
                   float* d_acc, int32_t micro_index, int32_t window_size, void* stream);

/* The whole window of n microbatches for buckets [b0, b1) in one pass
 * (NeMo Automodel issue #3857, section "Proposed scope and acceptance
 * criteria": accumulation windows of one, several and a trailing number of
 * microbatches; the reduction itself as for gro_accumulate):
 * bit for bit what gro_accumulate with micro_index 0..n-1 and window_size n
 * computes (per element: acc = red_0, then acc = acc + red_k in microbatch
 * order; norm partials written at the end), but the accumulator is written
 * once instead of being read and written n times.  For callers that keep
 * every microbatch's gradient buckets resident until the window ends (on a
 * 288 GB MI355X this trades n * sum_b(slots_b * slot_stride_b) BF16
 * elements of memory for (8n - 4) bytes per element less traffic).
 * d_grad_buckets: host array of n*(b1-b0) device pointers, microbatch-major:
 * entry k*(b1-b0) + j is microbatch k's BF16 buffer [slots][slot_stride] of
 * bucket b0+j.  1 <= n <= 64.  Leaves these buckets with a complete window
 * of n (any earlier partial window of theirs is discarded).  The same
 * one-accumulator rule as gro_accumulate applies. */
int gro_accumulate_window(gro_plan* plan, int32_t b0, int32_t b1, const void* const* d_grad_buckets,
                          int32_t n, float* d_acc, void* stream);

/* Microbatches first_micro .. first_micro+n-1 of a window for buckets
 * [b0, b1) in one pass (NeMo Automodel issue #3857, section "Preserved
 * prototype and evidence": accumulation that includes partial windows):
 * bit for bit what gro_accumulate with those micro_index values computes (starting from the accumulator in memory when
 * first_micro > 0), with the accumulator read and written once for the
 * group.  For callers that can keep a few microbatches' gradient buckets
 * resident but not a whole window: n microbatches in g groups move
 * 8 * (n - g) bytes per element less accumulator traffic than one call per
 * microbatch (a window of 8 in groups of 4: 48 bytes per element).
 * d_grad_buckets: host array of n*(b1-b0) device pointers, microbatch-major,
 * as for gro_accumulate_window.  1 <= n <= 64, first_micro >= 0;
 * first_micro > 0 requires every bucket in the range to have accumulated
 * exactly first_micro microbatches of the current window into d_acc (else
 * GRO_E_STATE).  window_size as for gro_accumulate (0 = not known; when
 * first_micro + n == window_size the norm partials are written too;
 * first_micro + n > window_size is GRO_E_INVALID).  gro_accumulate_window is
 * this call with first_micro = 0 and window_size = n.  Calls of both kinds
 * and gro_accumulate may be mixed within a window. */
int gro_accumulate_microbatches(gro_plan* plan, int32_t b0, int32_t b1, const void* const* d_grad_buckets,
                                int32_t first_micro, int32_t n, int32_t window_size, float* d_acc,
                                void* stream);

/* Global L2 norm (NeMo Automodel issue #3857, section "Proposed scope and
 * acceptance criteria": global norms checked against explicit references, no
 * double reduction) of g = acc / window_size over every owned element, in
 * FP64, with no atomics: per-chunk partials summed in a fixed order, so the result
 * does not depend on launch shape and is bit-reproducible.  Every bucket must
 * have accumulated exactly window_size microbatches (else GRO_E_STATE).  The
 * result stays on the device (read it with gro_plan_get_norm). */
int gro_reduce_norm(gro_plan* plan, const float* d_acc, int32_t window_size, void* stream);

/* Wait for the plan's stream and read the last norm.  Any out pointer may be
 * NULL.  finite = 0 when the norm is NaN or infinite.  GRO_E_STATE before
 * the first gro_reduce_norm after binding.
 * Every device call (bind excepted) must run with the device the plan was
 * bound on current, else GRO_E_STATE. */
int gro_plan_get_norm(gro_plan* plan, double* norm, double* norm_sq, int32_t* finite);

/* Clip + fused AdamW on every updated element, after gro_reduce_norm of the
 * same window (NeMo Automodel issue #3857, section "Preserved prototype and
 * evidence": clipping and Adam updates on the owned state; section
 * "Proposed scope and acceptance criteria": clipping on and off; Mixle
 * "Distributed Transformer Training", section "Optimizer and checkpoint
 * semantics": AdamW over parameters addressed by stable names):
 *   g = acc / window_size;  coef = min(1, max_norm / (norm + 1e-6)) in FP64
 *   rounded to FP32 when 0 < max_norm < inf, else 1 (clipping off);
 *   g^ = g*coef; p = p*(1 - lr*wd) (1 when GRO_NO_DECAY); m = b1*m + (1-b1)*g^;
 *   v = b2*v + (1-b2)*g^*g^; p = p - (lr/(1-b1^step)) * m / (sqrt(v)/sqrt(1-b2^step) + eps);
 *   d_param_bf16 (nullable) = p rounded to BF16, nearest-even.
 * A non-finite norm skips the update: master, m, v and the BF16 copy stay
 * bit-unchanged.  step >= 1.  Ends the window. */
int gro_clip_adamw(gro_plan* plan, const float* d_acc, int32_t window_size, double max_norm,
                   const gro_adamw_hparams* hp, int64_t step, float* d_master, float* d_m,
                   float* d_v, uint16_t* d_param_bf16, void* stream);

/* Replica-consistent initialisation of the FP32 master shard (and the
 * optional BF16 copy) of every updated parameter, independent of the rank,
 * of the layout and of when it runs (NeMo Automodel issue #3857, section
 * "Why this needs separate work": parameters can be created after the
 * model is parallelised, and replicas must not rely on each rank's training
 * random stream to start alike -- this draws nothing from any other
 * generator).
 * Element i of parameter p gets offset_p + (2u - 1) * bound_p with u in
 * [0, 1) in steps of 2^-24, from Philox4x64-10 with key (seed, param_id)
 * and counter (g / 4, 0, 0, 0), word g % 4, top 24 bits, where g is the
 * element's index in the unsharded parameter: shard_index * numel + i for a
 * Shard tensor (equal dim-0 shards), i otherwise.  bounds[t] >= 0 and
 * offsets[t] (host, n_tensors entries in descriptor order, FP64 rounded to
 * FP32; NULL offsets = 0) -- e.g. offset 1, bound 0 for a norm weight.
 * Waits for its own upload before returning. */
int gro_init_uniform(gro_plan* plan, uint64_t seed, const double* bounds, const double* offsets,
                     float* d_master, uint16_t* d_param_bf16, void* stream);

/* Thread-local text of the last error ("" if none). */
const char* gro_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GRO_H */
