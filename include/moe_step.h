/*
 * moe_step.h -- C ABI of one training update of a top-k mixture-of-experts
 * feed-forward layer, run as a single persistent HIP program on one MI355X
 * (gfx950).
 *
 * What one update computes (Latch pages, "How a training megakernel works"):
 *   "One training update": a forward pass, the loss, gradients by the chain
 *   rule, then a change of the weights against their gradients;
 *   "From two weights to 200 million": every token goes to k of the E expert
 *   feed-forward blocks chosen by a router; the optimizer is AdamW (moving
 *   averages of the gradient and of its elementwise square);
 *   "What Latch does", steps 1, 3 and 4: the layer is written with the routing
 *   operations token_topk and route_order and the grouped expert product
 *   ragged_mm; clipping by the global gradient norm and AdamW are tensor
 *   expressions of the update; each expert's gradient flows back to the tokens
 *   it received; master weights and both Adam moments stay FP32 while the
 *   matrix products run in BF16;
 *   "What Latch does", step 5: the pages run each update as one persistent
 *   kernel.  Here, too, one update (or one microbatch of it) is one launch of
 *   one persistent kernel; it is an ordinary launch by default (see
 *   moe_step_run) and a cooperative one on request.
 *
 * Layer (readings where the pages are silent are stated in the design notes):
 *   z = x W_r (+ b)                 router logits, fp32
 *   sel_i = k largest z_i, descending, lower expert index first on ties
 *   g_i = softmax over the k selected logits
 *   y_i = sum_j g_ij * gelu_tanh(x_i W1[sel_ij]) W2[sel_ij]
 *   L = sum_i ||y_i - t_i||^2 / (2 * tokens_in_update)
 *   backward through everything except the choice of experts; dx included
 *   c = min(1, clip_norm / (||grad|| + 1e-6)); AdamW with decoupled decay.
 *
 * Conventions for every entry point:
 *   - All tensor pointers in moe_step_io are DEVICE pointers on the handle's
 *     device; the caller owns them and keeps them alive until the stream has
 *     finished the launch.  Row-major, densely packed.
 *   - Nothing throws.  Every function returns a moe_status (0 = success) except
 *     the size queries and moe_step_last_error.
 *   - Argument validation happens on the host before any HIP call.
 */
#ifndef MOE_STEP_H
#define MOE_STEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_STEP_ABI_VERSION 1u

typedef struct moe_step* moe_step_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,    /* NULL or out-of-range argument */
  MOE_ERR_SHAPE = -2,  /* layer shape the kernels do not support */
  MOE_ERR_HIP = -3,    /* a HIP runtime call failed (incl. no device) */
  MOE_ERR_NOMEM = -4,  /* device allocation failed */
  MOE_ERR_DEVICE = -5, /* the kernel reported an error (see last_error) */
  MOE_ERR_STATE = -6   /* handle in a state that forbids the call */
} moe_status;

typedef enum {
  MOE_DTYPE_F32 = 0,  /* x, t, activations and products in fp32 */
  MOE_DTYPE_BF16 = 1  /* x, t, stored activations and GEMM operands in bf16;
                         router, accumulation, grads, master weights fp32 */
} moe_dtype;

/* Layer and optimizer configuration, fixed for the life of a handle.
 * Supported shapes: d_model and d_ff multiples of 8 (>= 8), 1 <= n_experts <= 64,
 * 1 <= top_k <= min(8, n_experts), 1 <= max_tokens <= 2^24. */
typedef struct {
  uint32_t struct_size;   /* sizeof(moe_step_config) */
  uint32_t abi_version;   /* MOE_STEP_ABI_VERSION */
  int32_t d_model;        /* d */
  int32_t d_ff;           /* f, expert hidden width */
  int32_t n_experts;      /* E */
  int32_t top_k;          /* k */
  int32_t max_tokens;     /* largest n_tokens of any run; sizes the arena */
  int32_t dtype;          /* moe_dtype */
  double lr, beta1, beta2, adam_eps, weight_decay;  /* AdamW; the library derives
                             1-beta and the bias corrections in double and
                             rounds them to fp32 once */
  double clip_norm;       /* global-norm clip; <= 0 disables clipping */
  int32_t device;         /* HIP device ordinal */
  int32_t wg_per_cu;      /* persistent workgroups per compute unit: 1, 2, or 0 =
                             automatic (2 for bf16 when max_tokens * top_k >=
                             4096, else 1).  Two per unit runs a kernel built for
                             half the registers and LDS per workgroup; fp32
                             handles always run one.  Results differ between the
                             settings at rounding level only: the split of the
                             router dot products over lanes and the loss's
                             per-workgroup partial sums follow the workgroup
                             count. */
  uint32_t memory_rules;  /* opt-in arena rules (the pages' "Open problems",
                             Generality 2: rules for lifetimes and
                             recomputation); 0 = none.
                             MOE_MEM_RECOMPUTE: of the first expert product only
                             H = x W1 is stored; gelu(H) is recomputed on the
                             operand fragments of the second product and of the
                             dW2 product, gelu'(H) in the dH epilogue.  The arena
                             loses one [tokens * top_k, d_ff] tensor; the update
                             is slower (each H element passes through GELU once
                             per output column tile that reads it).
                             MOE_MEM_GUARDS: a checking layout, not a saving: a
                             zone of max(1 MiB, 128 * max(d_model, d_ff) * 4
                             bytes) follows every sub-buffer of the arena (26
                             of them for bf16, 24 for fp32), zero from create
                             on like the rest of the arena and never written by
                             a correct kernel; moe_step_check_guards reads the
                             zones.  Results are those of the plain layout.
                             Refused by moe_step_run_static. */
  int32_t max_microbatches; /* 0 or 1: every launch adds its expert weight
                             gradients to grads (the default).  M in [2, 16]
                             (bf16 handles, not with MOE_MEM_RECOMPUTE):
                             deferred expert weight gradients.  The pages
                             accumulate one update over several microbatch
                             launches ("How GPUs usually run it"); the expert
                             weights do not change within an update, so here a
                             launch that does not apply the experts keeps the
                             operand rows of its dW1 / dW2 products (about
                             2 * T * k * (d + f) bytes) in one of M arena slots,
                             and the launch that applies them contracts dW1 and
                             dW2 once over the rows of every slot, writing the
                             W1 / W2 part of grads (added to it when the slot-0
                             launch did not zero the gradients).  A launch with
                             MOE_RUN_ZERO_GRAD(_EXPERTS) takes slot 0, each later
                             one the next slot; more than M launches before the
                             experts are applied is MOE_ERR_STATE.  Between those
                             launches the W1 / W2 part of grads is not updated;
                             the router gradient is added every launch as
                             without deferral.  Results equal the default's up to
                             the order of fp32 accumulation. */
} moe_step_config;

#define MOE_MEM_RECOMPUTE 0x1u
#define MOE_MEM_GUARDS 0x2u

/* Buffers of one launch.  Shapes use T = n_tokens, P = moe_step_param_count. */
typedef struct {
  const void* x;            /* [T, d] in dtype (fp32 or bf16)               */
  const void* target;       /* [T, d] in dtype                               */
  const float* router_bias; /* [E] constant logit bias, or NULL for none    */
  float* params;            /* [P] fp32 master weights W_r[d,E] | W1[E,d,f] | W2[E,f,d];
                               updated in place when MOE_RUN_APPLY is set    */
  float* grads;             /* [P] fp32; written (MOE_RUN_ZERO_GRAD) or added to;
                               holds the pre-clip gradient afterwards        */
  float* exp_avg;           /* [P] fp32 first moment, updated on APPLY      */
  float* exp_avg_sq;        /* [P] fp32 second moment, updated on APPLY     */
  float* dx;                /* [T, d] fp32 input gradient, or NULL to skip it */
  float* stats;             /* [4] fp32 or NULL: loss (set with ZERO_GRAD, else
                               added to), grad norm, clip coefficient, unused */
  /* optional debug outputs (NULL = not written): */
  float* router_logits;     /* [T, E] fp32 (bias included)                   */
  int32_t* topk_idx;        /* [T, k] selected experts, largest logit first  */
  float* topk_gate;         /* [T, k] gates                                  */
  int32_t* expert_counts;   /* [E] tokens routed to each expert              */
  int32_t* route_perm;      /* [T*k] flat id i*k+j at each expert-sorted slot */
  uint64_t* trace;          /* [moe_step_trace_words] per-workgroup phase clocks,
                               written only with MOE_RUN_TRACE               */
} moe_step_io;

/* run_flags */
#define MOE_RUN_ZERO_GRAD 0x1u      /* grads := this launch's gradient (else +=) */
#define MOE_RUN_APPLY 0x2u          /* global-norm clip + AdamW after the backward */
#define MOE_RUN_REFRESH_SHADOW 0x4u /* rebuild the bf16 weight copy from params
                                       first (needed after create and whenever the
                                       caller changed params itself) */
#define MOE_RUN_TRACE 0x8u          /* record per-phase clocks into io.trace */
/* Per-group variants (selective updates: the shared router W_r and the experts
 * W1 | W2 keep separate accumulation windows and optimizer steps, the pages'
 * "Other measured compiler work" table: shared weights every microbatch,
 * experts every 16).  MOE_RUN_ZERO_GRAD = both ZERO bits, MOE_RUN_APPLY = both
 * APPLY bits.  The clip norm is taken over the groups applied in the launch. */
#define MOE_RUN_ZERO_GRAD_ROUTER 0x10u   /* router grads := this launch's (else +=)  */
#define MOE_RUN_ZERO_GRAD_EXPERTS 0x20u  /* expert grads := this launch's (else +=)  */
#define MOE_RUN_APPLY_ROUTER 0x40u       /* clip + AdamW on W_r                      */
#define MOE_RUN_APPLY_EXPERTS 0x80u      /* clip + AdamW on W1 | W2                  */
/* Profiling aid: skip phase i (0..7) of the persistent kernel and reuse what the
 * previous launch on this handle left in the arena.  Accepted only when the
 * previous launch ran every phase with the same n_tokens (else MOE_ERR_STATE).
 * Only the timing is meaningful: a skipped phase's output comes from the
 * previous launch, but buffers shared between phases of disjoint lifetimes
 * may by then hold a later phase's data (all values finite).  Phase
 * order: 0 routing, 1 route_order, 2 expert GEMM 1, 3 expert GEMM 2,
 * 4 combine/loss, 5 dH + dW2 + router partials, 6 dW1 + dX + router gradient,
 * 7 dx sum + norm + clip/AdamW. */
#define MOE_RUN_SKIP_PHASE(i) (0x100u << (i))
/* The same for two steps inside phases, so each gets a figure of its own: the
 * dispatch gather (copy of the token rows into expert order, in phase 1) and
 * the k-way sum of the per-slot input gradients (dx, in phase 7). */
#define MOE_RUN_SKIP_GATHER 0x100000u
#define MOE_RUN_SKIP_ROWSUM 0x200000u
#define MOE_RUN_SKIP_MASK (0xff00u | MOE_RUN_SKIP_GATHER | MOE_RUN_SKIP_ROWSUM)
/* Readiness-driven scheduling between expert GEMM 1 and GEMM 2 (the pages'
 * "Open problems", Performance 1: replace whole-grid barriers by finer
 * dependencies).  Without it a grid barrier separates the two products.  With
 * it there is none: every GEMM-1 tile, once its stores are out, releases at
 * agent scope and counts itself done on its 128-row tile, and a GEMM-2 tile
 * waits (bounded) until every GEMM-1 column tile of its rows is counted, then
 * acquires.  Results are identical.  It is slower on MI355X (each release
 * writes the XCD's L2 back to memory, each acquire drops the L2's clean lines),
 * so it is off by default. */
#define MOE_RUN_READY_GEMM12 0x10000u
/* Launch through hipLaunchCooperativeKernel (the runtime guarantees that the
 * whole grid is resident) instead of an ordinary launch. */
#define MOE_RUN_COOPERATIVE 0x20000u
/* Test aid for the failure path (never needed in training): the bounded waits
 * of this launch give up after about 10 us instead of about 2 s, and the last
 * workgroup first waits for a word that nothing ever sets, so it gives up and
 * never arrives at the first grid barrier.  Every other workgroup's wait at that
 * barrier then gives up too; the launch ends with MOE_DEVICE_BARRIER_TIMEOUT,
 * and every workgroup exits normally.  Only the routing phase runs before that
 * barrier: it writes arena buffers, the debug outputs that are given, and (with
 * MOE_RUN_REFRESH_SHADOW) the bf16 weight copy from the unchanged params. */
#define MOE_RUN_TEST_TIMEOUT 0x40000u
/* Grid barriers in which every workgroup writes its XCD's L2 back to memory
 * itself, instead of the last workgroup of each XCD doing it once for all
 * (same results; for comparison). */
#define MOE_RUN_BARRIER_PER_WORKGROUP 0x80000u

/* Status-word bits reported by moe_step_status as MOE_ERR_DEVICE. */
#define MOE_DEVICE_BARRIER_TIMEOUT 0x1u
#define MOE_DEVICE_NONFINITE_LOGIT 0x2u
#define MOE_DEVICE_BAD_ROUTE 0x4u        /* internal consistency check of the routing */

/* Number of fp32 parameters P = d*E + 2*E*d*f (0 if cfg is NULL). Host only. */
size_t moe_step_param_count(const moe_step_config* cfg);

/* Host-only check of a configuration: MOE_OK, MOE_ERR_ARG or MOE_ERR_SHAPE.
 * Makes no HIP call. */
int moe_step_check_config(const moe_step_config* cfg);

/* Creates a handle on cfg->device: validates cfg, allocates the device arena
 * (the planned GPU-memory arena that holds every value passed between phases,
 * Latch "How a training megakernel works", "What Latch does", step 4: routing
 * structures, stored activations, bf16 weight copy, barrier words) and
 * checks that the persistent grid fits co-resident.  Synchronous.
 * On failure *out is set to NULL and the reason is available from
 * moe_step_last_error(NULL). */
int moe_step_create(const moe_step_config* cfg, moe_step_t* out);

/* Enqueues one update on hip_stream (a hipStream_t; NULL = default stream):
 * one launch of the persistent kernel that runs the forward pass, loss,
 * backward pass and weight update of the layer (Latch "How a training
 * megakernel works", "What Latch does": one resident program per update, one
 * launch per microbatch at the published batch in "How GPUs usually run it").
 * Asynchronous.
 * The kernel needs all of its workgroups resident at once (grid barriers).  Its
 * grid is sized at create to exactly what the device holds (occupancy x CUs),
 * and by default it goes out as an ordinary launch: a cooperative launch costs
 * about 19 us more per update on MI355X.  Launches of two handles on different
 * streams of one device must then not overlap (order them with events); with
 * MOE_RUN_COOPERATIVE the runtime guarantees co-residency instead.  If the
 * grid cannot become resident (another kernel holds compute units for longer
 * than the barrier's bound of about 2 s), the launch ends with
 * MOE_DEVICE_BARRIER_TIMEOUT from moe_step_status; it never hangs.
 * n_tokens in [0, max_tokens]; tokens_in_update >= max(1, n_tokens) is the loss
 * denominator (the tokens of all microbatches of one update); step >= 1 is the
 * 1-based AdamW step, used only with MOE_RUN_APPLY.
 * Gradient accumulation over microbatches: ZERO_GRAD on the first, neither flag
 * on the middle ones, APPLY on the last. */
int moe_step_run(moe_step_t h, const moe_step_io* io, int32_t n_tokens, int64_t tokens_in_update,
                 int64_t step, uint32_t run_flags, void* hip_stream);

/* moe_step_run with a separate 1-based AdamW step per parameter group, for
 * selective updates: step_router is used when W_r is applied, step_experts
 * when W1 | W2 are (each >= 1 when its group is applied).  With both groups
 * applied, the global-norm clip covers all parameters as in moe_step_run;
 * with one, only that group's gradients enter the norm.  The loss in
 * io.stats restarts whenever a ZERO bit is set.  moe_step_run(.., step, ..) is
 * moe_step_run_groups(.., step, step, ..).  Same errors as moe_step_run. */
int moe_step_run_groups(moe_step_t h, const moe_step_io* io, int32_t n_tokens, int64_t tokens_in_update,
                        int64_t step_router, int64_t step_experts, uint32_t run_flags, void* hip_stream);

/* Bytes of the static device array behind moe_step_run_static (per GPU). */
#define MOE_STEP_STATIC_SCRATCH_BYTES (32u << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  One update
 * like moe_step_run, with no handle and no allocation of any kind.
 *   - The arena lives in a static device array of MOE_STEP_STATIC_SCRATCH_BYTES
 *     (32 MiB) that every GPU the library runs on holds from the library's load
 *     until the process ends.  cfg is validated as by moe_step_create and its
 *     max_tokens sizes the arena; a configuration whose arena (about
 *     moe_step_arena_bytes of a handle with the same cfg, plus 128 KiB of
 *     barrier words) does not fit is refused with MOE_ERR_SHAPE.
 *   - Enqueues three launches on hip_stream: a fill kernel that clears the
 *     barrier words, the update (the same kernel and grid as a handle with the
 *     same cfg, so the results are bit-identical to moe_step_run), and a
 *     one-thread kernel that writes the device status bits of the update into
 *     io->stats[3] (0 = no error, else the MOE_DEVICE_* bits as a float).  The
 *     three are ordered on the stream only, so the call can be captured.
 *   - io->stats is required.  The bf16 weight copy is rebuilt from params on
 *     every call (MOE_RUN_REFRESH_SHADOW is implied), because the array keeps
 *     whatever the last call on that GPU left in it.  MOE_RUN_SKIP_PHASE is
 *     refused (there is no previous launch of this caller to reuse).
 *   - Every call on a GPU shares that GPU's array: calls that overlap on one
 *     GPU (different streams without an order between them) race and give
 *     wrong results.
 *   - Host errors return as from moe_step_run, with the text in
 *     moe_step_last_error(NULL). */
int moe_step_run_static(const moe_step_config* cfg, const moe_step_io* io, int32_t n_tokens,
                        int64_t tokens_in_update, int64_t step, uint32_t run_flags, void* hip_stream);

/* Waits for the handle's last stream and reads the device status word: the
 * numerical check of the launch (non-finite router logits) and the bounded
 * waits of its grid barriers (Latch "How a training megakernel works", "What
 * Latch does", step 4: a phase waits at a grid-wide barrier; step 5: run the
 * program's numerical checks).  Returns MOE_ERR_DEVICE (with the bits in
 * last_error) if a kernel reported an error, after resetting the device-side
 * barrier state and the abort word.  A launch enqueued after one that failed
 * and before this call makes no writes (every workgroup finds the abort word
 * set on entry and returns). */
int moe_step_status(moe_step_t h);

/* Checks the guard zones of a handle created with MOE_MEM_GUARDS in
 * memory_rules: each sub-buffer of the planned arena (Latch "How a training
 * megakernel works", "What Latch does", step 4) is followed by a zone that
 * must still hold the zeros that create wrote.  Waits for the handle's last
 * stream, then copies every zone to the host.  Returns MOE_OK if all are
 * intact; MOE_ERR_STATE if a zone holds a nonzero byte (last_error names the
 * buffer before the first such zone and the offset past its end) or if the
 * handle has no zones; MOE_ERR_HIP or MOE_ERR_NOMEM if a copy or a host
 * buffer fails.  *damaged (optional) receives the number of written zones
 * (0 on every other outcome).  A write of zeros past a buffer's end is not
 * seen. */
int moe_step_check_guards(moe_step_t h, int32_t* damaged);

/* Words of io.trace needed for MOE_RUN_TRACE: workgroups * phases * 3. */
size_t moe_step_trace_words(moe_step_t h);

/* Persistent workgroups of the handle's launches. */
int moe_step_grid_size(moe_step_t h);

/* Bytes of device memory the handle holds (its arena; 0 for NULL).  Stored
 * activations whose lifetimes do not overlap share memory (the expert outputs
 * O with dH, the activations A with the per-slot input gradients), the
 * memory rule of the pages' "Open problems", Generality 2. */
size_t moe_step_arena_bytes(moe_step_t h);

/* Text of the last error on h (or, if h is NULL, of the last failed create or
 * moe_step_run_static call on this thread).
 * Valid until the next call on the same handle. Never NULL. */
const char* moe_step_last_error(moe_step_t h);

/* Waits for the last stream, frees the arena (the planned GPU-memory arena of
 * Latch "How a training megakernel works", "What Latch does", step 4) and the
 * handle.  NULL-safe. */
void moe_step_destroy(moe_step_t h);

#ifdef __cplusplus
}
#endif

#endif /* MOE_STEP_H */
