/*
 * lr.h -- C ABI of the MI355X (gfx950) FP32 row-reduction library, liblr.so.
 *
 * Row operations over a row-major rows x cols FP32 tensor (row stride = cols
 * elements).  Each is a composition of max/min/add folds over the column
 * axis, as defined on the page "TIRx Metal reduction lowering"
 * (LuisaCompute), section 1 (softmax and cross-entropy sources), section 5.1
 * (LayerNorm statistics and the fused residual LayerNorm), section 5.2
 * (guarded label gather), section 8 (row sums, row minimum and maximum).  The
 * reduction-order contract (unordered tree versus ordered fold) is the
 * ReductionPolicy of section 1.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   All tensor pointers are DEVICE pointers owned by the caller.  The
 *           library allocates no device memory and never reads or writes
 *           outside the ranges described per call (the SPLIT family's
 *           partials go to a workspace the caller passes to lr_run_f32, or
 *           to the one device array per GPU that lr_run_f32_noalloc owns,
 *           the library's only device state).
 *           FP32 pointers must be 4-byte aligned and the int64 label pointer
 *           8-byte aligned (else LR_ERR_MISALIGNED); 16-byte alignment is not
 *           required (misaligned rows take a guarded path).
 * Aliasing. Inputs and outputs must not overlap, except that an operation's
 *           output may be exactly its input tensor (y == x: in place).  Any
 *           other overlap returns LR_ERR_ALIASING (the pages' kernel ABI is
 *           noalias, section 3).
 * Shapes.   0 <= rows <= INT32_MAX, cols >= 1, rows*cols*4 must fit in
 *           int64, cols < 2^24 (so that cols is exact in FP32); else
 *           LR_ERR_INVALID_SHAPE.  rows == 0 returns LR_OK and launches
 *           nothing.  A call whose grid would pass one dispatch's reach runs
 *           as several dispatches in order on `stream` (lr_dispatch_rows).
 * Streams.  Work is enqueued on `stream` (NULL = the default stream) and the
 *           call returns without synchronising.  A launch failure reported
 *           by the HIP runtime returns LR_ERR_HIP.
 * Errors.   Every argument is validated before any HIP call; nothing falls
 *           back to the CPU.  An explicit plan that cannot be realised
 *           returns LR_ERR_UNREALIZABLE_PLAN; it is never clamped.
 * Values.   Inputs are finite, with one exception: softmax and cross-entropy
 *           rows may hold -infinity (masked positions) as long as every
 *           row keeps at least one finite element; a masked element's
 *           softmax output is +0 and it adds nothing to the sum.  A row of
 *           nothing but -infinity, NaN, +infinity, or a non-finite value
 *           in any other operation is outside the contract: no error is
 *           reported and the result is unspecified (it may differ between
 *           policies and plans).  For lr_row_minmax_f32 in particular, a
 *           NaN element may be skipped or returned depending on the
 *           policy.  RMSNorm and LayerNorm square the elements in FP32:
 *           with eps = 0 (or eps far below the row's mean square or
 *           variance), a row whose magnitude is below about 1e-20 loses
 *           accuracy to the subnormal range, and one whose squares all
 *           round to zero (below about 1e-23) gives +-infinity or NaN, as
 *           the FP32 formula does.  Rows down to about 1e-19 (squares and
 *           mean square subnormal) keep the stated accuracy.
 * Threads.  All entry points are thread-safe.
 * Policy.   See lr_reduction_policy below: LR_UNORDERED_TREE lets every
 *           add fold be reassociated; the three ordered policies fix the
 *           order of every add fold, round every operation on its own and
 *           give results that do not depend on the plan.
 */
#ifndef LR_H
#define LR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;

/* ReductionPolicy ("TIRx Metal reduction lowering", section 1): the order in
 * which each add fold may be evaluated.  Max and min folds are exact in any
 * order under every policy.
 *   LR_UNORDERED_TREE  any order (lane stripes, wave trees); hardware
 *                      exp/log/rcp/rsqrt; repeatable for a fixed plan.
 *   LR_ORDERED_FOLD    fold_left: one FP32 chain j = 0 .. cols-1 from +0.0f.
 *   LR_ORDERED_TREE    the pairwise tree in index order over the row's
 *                      contributions padded with -0.0f (the exact add
 *                      identity) to the next power of two (adjacent pairs
 *                      added level by level).
 *   LR_FOLD_RIGHT      one FP32 chain j = cols-1 .. 0 from +0.0f
 *                      (acc = c_j + acc).
 * Under the three ordered policies every operation is rounded on its own (no
 * fused multiply-add), division and square root are IEEE, exp and log are
 * the precise library functions, and the result does not depend on the
 * plan. */
typedef enum lr_reduction_policy {
    LR_UNORDERED_TREE = 0,
    LR_ORDERED_FOLD = 1,
    LR_ORDERED_TREE = 2,
    LR_FOLD_RIGHT = 3,
    LR_FOLD_LEFT = LR_ORDERED_FOLD
} lr_reduction_policy;

typedef enum lr_status {
    LR_OK = 0,
    LR_ERR_NULL_POINTER = 1,
    LR_ERR_INVALID_SHAPE = 2,
    LR_ERR_INVALID_EPS = 3,
    LR_ERR_INVALID_POLICY = 4,
    LR_ERR_MISALIGNED = 5,
    LR_ERR_ALIASING = 6,
    LR_ERR_UNREALIZABLE_PLAN = 7,
    LR_ERR_HIP = 8,
    LR_ERR_INVALID_ARGUMENT = 9,
    LR_ERR_WORKSPACE = 10
} lr_status;

typedef enum lr_op {
    LR_OP_SOFTMAX = 0,
    LR_OP_RMSNORM = 1,
    LR_OP_LAYERNORM = 2,
    LR_OP_CROSS_ENTROPY = 3,
    LR_OP_ADD_LAYERNORM = 4,
    LR_OP_ROW_SUM = 5,
    LR_OP_ROW_MINMAX = 6
} lr_op;

/* Kernel families.
 * CACHE:   each lane keeps its stripe of the row in registers (VGPRs), so
 *          the row is read from memory once and every later pass reads
 *          registers (the pages' worker-private stripe, section 5).  Narrow
 *          rows may take sub-wave teams: lanes_per_row = 4, 8, 16 or 32
 *          lanes serve one row, so one wavefront holds 64 / lanes_per_row
 *          rows and its cross-lane reductions stop at the team's width.
 * STREAM:  no register copy; passes that need the row again reload it
 *          (softmax and cross-entropy fold max and sum-of-exp in one
 *          online pass).  Any row length.
 * ORDERED: the ordered policies for any row: one wavefront per row, the row
 *          staged through LDS in 256-element slabs, folded in order
 *          (LR_ORDERED_FOLD, LR_FOLD_RIGHT) or summed as the pairwise tree
 *          (LR_ORDERED_TREE).  Rows of at most 64 floats may instead take
 *          one lane per row (lanes_per_row = 1): 64 rows per wavefront,
 *          staged through an LDS tile, each lane's order its own chain.
 * TREE:    LR_ORDERED_TREE on the CACHE layout, for rows whose start is
 *          16-byte aligned and cols <= 32768: each wave's 256-element slab
 *          is one wave tree, and the slab sums one more.  Narrow aligned
 *          rows may take sub-wave teams (lanes_per_row = 4 .. 32, one
 *          chunk per lane).
 * SPLIT:   LR_UNORDERED_TREE for rows too few to fill the device: each row
 *          is cut into `splits` segments of whole 16-byte chunks, one
 *          workgroup per segment.  A first kernel writes every segment's
 *          partial statistics (max and sum of exp, sum of squares, mean and
 *          sum of squared deviations, sum, minimum and maximum) to a
 *          workspace, and a second merges a row's partials and writes its
 *          outputs, re-reading the segment from L2.  Needs a caller workspace
 *          (lr_run_f32); the automatic plan of the other entry points never
 *          splits rows. */
typedef enum lr_family {
    LR_FAMILY_CACHE = 0,
    LR_FAMILY_STREAM = 1,
    LR_FAMILY_ORDERED = 2,
    LR_FAMILY_TREE = 3,
    LR_FAMILY_SPLIT = 4
} lr_family;

/* A launch plan (the pages' GroupPlan decision record, section 2, mapped to
 * wave64: workers per row W = lanes_per_row = 64 * waves_per_row, or a
 * sub-wave team of a CACHE plan, section 4). */
typedef struct lr_plan {
    int32_t family;            /* lr_family */
    int32_t waves_per_row;     /* S: wavefronts cooperating on one row, 1..16
                                  (1 for a sub-wave team) */
    int32_t rows_per_block;    /* Q: rows packed into one workgroup, S*Q <= 16;
                                  sub-wave teams: a multiple of
                                  64 / lanes_per_row, lanes_per_row * Q <= 1024 */
    int32_t vec;               /* V: consecutive FP32 a lane owns per chunk (4 = 128-bit) */
    int32_t chunks_per_lane;   /* CACHE: 128-bit chunks held per lane (a compiled
                                  instance: 1,2,3,4,6,8,12,16,24 or 32);
                                  SPLIT: chunks per lane of one segment
                                  (1,2,3,4,6 or 8);
                                  STREAM: chunks loaded per lane per loop trip;
                                  ORDERED: 0, or with one lane per row the
                                  instance width N4 (1,2,4,8 or 16; the row
                                  fits 4 * N4 floats) */
    int32_t threads_per_block; /* 64 * S * Q, or lanes_per_row * Q */
    int64_t blocks;            /* ceil(rows / Q); SPLIT: rows * splits */
    int32_t lds_bytes;         /* static LDS the kernel uses */
    int32_t reductions;        /* |R|: cross-lane reductions per row */
    int32_t row_aligned;       /* 1: planned for 16-byte aligned rows */
    int32_t splits;            /* SPLIT: segments per row, 2..64 (Q = 1);
                                  0 for every other family */
    int32_t lanes_per_row;     /* lanes serving one row: 64 * S (0 reads as
                                  64 * S, so a plan filled in field by field
                                  without it keeps whole waves); 4, 8, 16
                                  or 32 for sub-wave teams (S = 1; CACHE
                                  with chunks_per_lane 1 or 2, TREE with 1);
                                  1 for ORDERED with one lane per row (S = 1,
                                  Q = 64); the planner always fills it in */
} lr_plan;

/* What the planner needs to know about a device. */
typedef struct lr_device_facts {
    int32_t compute_units;          /* 256 on MI355X */
    int32_t max_threads_per_block;  /* 1024 */
    int32_t simds_per_cu;           /* 4 */
    int32_t wave_size;              /* 64 */
} lr_device_facts;

/* ---------------------------------------------------------------------------
 * Operations
 * ------------------------------------------------------------------------- */

/* Row softmax ("TIRx Metal reduction lowering", section 1, softmax source):
 *   y[r][j] = exp(x[r][j] - m_r) / sum_k exp(x[r][k] - m_r),  m_r = max_k x[r][k].
 * x: rows*cols FP32 in; y: rows*cols FP32 out (y == x allowed). */
lr_status lr_softmax_f32(const float* x, float* y, int64_t rows, int64_t cols,
                         lr_reduction_policy policy, hipStream_t stream);

/* RMSNorm (timed on the page "Whole-launch reduction cost policy", held-out
 * table; no formula on the pages -- eps inside the root as LayerNorm does in
 * section 5.1):
 *   y[r][j] = gamma[j] * x[r][j] / sqrt(mean_k x[r][k]^2 + eps).
 * gamma: cols FP32, or NULL for 1.  eps: finite, >= 0 (else LR_ERR_INVALID_EPS).
 * Under LR_ORDERED_FOLD the FP32 sequence is ss = fold(x*x), ms = ss/cols,
 * r = 1/sqrt(ms + eps), y = (x*r)*gamma. */
lr_status lr_rmsnorm_f32(const float* x, const float* gamma, float* y,
                         int64_t rows, int64_t cols, float eps,
                         lr_reduction_policy policy, hipStream_t stream);

/* LayerNorm ("TIRx Metal reduction lowering", section 5.1 statistics, section
 * 8 affine):  mu = sum_k x/cols;  var = sum_k (x - mu)^2 / cols (biased,
 * centred two-pass);  y = (x - mu) / sqrt(var + eps) * gamma + beta.
 * gamma, beta: cols FP32 each, or NULL for 1 / 0.  eps: finite, >= 0.
 * Under LR_ORDERED_FOLD: mu = fold(x)/cols, var = fold((x-mu)*(x-mu))/cols,
 * r = 1/sqrt(var + eps), y = ((x-mu)*r)*gamma + beta (absent terms skipped). */
lr_status lr_layernorm_f32(const float* x, const float* gamma, const float* beta,
                           float* y, int64_t rows, int64_t cols, float eps,
                           lr_reduction_policy policy, hipStream_t stream);

/* Per-row cross-entropy ("TIRx Metal reduction lowering", section 1
 * cross-entropy source; section 5.2 guarded gather):
 *   m = max_k x[r][k];  s = sum_k exp(x[r][k] - m);
 *   sel = (0 <= labels[r] < cols) ? x[r][labels[r]] : 0   (int64 compare);
 *   losses[r] = log(s) + (m - sel), the difference first (exact in FP32
 *   whenever sel >= m / 2, so a small loss next to large logits keeps its
 *   accuracy).
 * logits: rows*cols FP32; labels: rows int64 (any value: out-of-range labels
 * are not an error, they select 0); losses: rows FP32 out. */
lr_status lr_cross_entropy_f32(const float* logits, const int64_t* labels,
                               float* losses, int64_t rows, int64_t cols,
                               lr_reduction_policy policy, hipStream_t stream);

/* Fused residual LayerNorm ("TIRx Metal reduction lowering", section 5.1:
 * combined = X + residual, then the two-pass LayerNorm of combined; each
 * input element is read from memory once):
 *   c[r][j] = x[r][j] + residual[r][j]      (one FP32 addition)
 *   mu = sum_k c/cols;  var = sum_k (c - mu)^2 / cols;
 *   y = (c - mu) / sqrt(var + eps) * gamma + beta.
 * x, residual: rows*cols FP32 in.  gamma, beta: cols FP32 each, or NULL for
 * 1 / 0 (NULL, NULL is the pages' program).  y: rows*cols FP32 out.
 * sum_out: rows*cols FP32 out receiving c, or NULL (not written).
 * Aliasing: y may be exactly x or exactly residual, and so may sum_out; y and
 * sum_out must not overlap each other or gamma/beta (else LR_ERR_ALIASING).
 * Under LR_ORDERED_FOLD the statistics are the left folds of LayerNorm taken
 * over c.  Errors as for lr_layernorm_f32; residual is required. */
lr_status lr_add_layernorm_f32(const float* x, const float* residual, const float* gamma,
                               const float* beta, float* y, float* sum_out, int64_t rows,
                               int64_t cols, float eps, lr_reduction_policy policy,
                               hipStream_t stream);

/* Row sum: the plain add fold over the column axis ("TIRx Metal reduction
 * lowering", section 8 checks row sums at widths 127, 257, 1024, 4096):
 *   sums[r] = sum_j x[r][j]   (FP32 accumulation).
 * x: rows*cols FP32 in; sums: rows FP32 out.  Under LR_ORDERED_FOLD the sum
 * is one FP32 chain j = 0 .. cols-1 from +0.0f; under LR_UNORDERED_TREE any
 * order (lane stripes, then trees).  sums must not overlap x. */
lr_status lr_row_sum_f32(const float* x, float* sums, int64_t rows, int64_t cols,
                         lr_reduction_policy policy, hipStream_t stream);

/* Row minimum and maximum together, in one pass over the row (section 8:
 * minimum and maximum at 7 x 1024):
 *   mins[r] = min_j x[r][j],  maxs[r] = max_j x[r][j].
 * mins, maxs: rows FP32 out each; either may be NULL, not both
 * (LR_ERR_NULL_POINTER).  Exact (both are input values), so every policy
 * gives the same result.  Outputs must not overlap x or each other. */
lr_status lr_row_minmax_f32(const float* x, float* mins, float* maxs, int64_t rows,
                            int64_t cols, lr_reduction_policy policy, hipStream_t stream);

/* The same operations under an explicit plan (the pages' exact
 * thread/packing constraints, section 6: honoured exactly or rejected).
 * `plan->family` must match the policy: CACHE or STREAM (or SPLIT, which
 * needs lr_run_f32's workspace: LR_ERR_WORKSPACE here) for
 * LR_UNORDERED_TREE, ORDERED for LR_ORDERED_FOLD and LR_FOLD_RIGHT, TREE or
 * ORDERED for LR_ORDERED_TREE.  A plan that does not cover the row, exceeds a device
 * limit or names a chunk count with no compiled instance returns
 * LR_ERR_UNREALIZABLE_PLAN before any launch. */
lr_status lr_softmax_f32_with_plan(const float* x, float* y, int64_t rows, int64_t cols,
                                   lr_reduction_policy policy, const lr_plan* plan,
                                   hipStream_t stream);
lr_status lr_rmsnorm_f32_with_plan(const float* x, const float* gamma, float* y,
                                   int64_t rows, int64_t cols, float eps,
                                   lr_reduction_policy policy, const lr_plan* plan,
                                   hipStream_t stream);
lr_status lr_layernorm_f32_with_plan(const float* x, const float* gamma, const float* beta,
                                     float* y, int64_t rows, int64_t cols, float eps,
                                     lr_reduction_policy policy, const lr_plan* plan,
                                     hipStream_t stream);
lr_status lr_cross_entropy_f32_with_plan(const float* logits, const int64_t* labels,
                                         float* losses, int64_t rows, int64_t cols,
                                         lr_reduction_policy policy, const lr_plan* plan,
                                         hipStream_t stream);
lr_status lr_add_layernorm_f32_with_plan(const float* x, const float* residual,
                                         const float* gamma, const float* beta, float* y,
                                         float* sum_out, int64_t rows, int64_t cols, float eps,
                                         lr_reduction_policy policy, const lr_plan* plan,
                                         hipStream_t stream);
lr_status lr_row_sum_f32_with_plan(const float* x, float* sums, int64_t rows, int64_t cols,
                                   lr_reduction_policy policy, const lr_plan* plan,
                                   hipStream_t stream);
lr_status lr_row_minmax_f32_with_plan(const float* x, float* mins, float* maxs, int64_t rows,
                                      int64_t cols, lr_reduction_policy policy,
                                      const lr_plan* plan, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Every operation through one call, with an optional workspace
 * ------------------------------------------------------------------------- */

/* The tensors of an operation; members an operation does not use must be
 * NULL.  Meanings, shapes and aliasing rules are those of the typed entry
 * points above (x is the logits for LR_OP_CROSS_ENTROPY). */
typedef struct lr_tensors {
    const float* x;
    const float* residual;   /* LR_OP_ADD_LAYERNORM */
    const float* gamma;      /* norms, or NULL */
    const float* beta;       /* LayerNorms, or NULL */
    const int64_t* labels;   /* LR_OP_CROSS_ENTROPY */
    float* y;                /* softmax and norms */
    float* sum_out;          /* LR_OP_ADD_LAYERNORM, or NULL */
    float* losses;           /* LR_OP_CROSS_ENTROPY */
    float* sums;             /* LR_OP_ROW_SUM */
    float* mins;             /* LR_OP_ROW_MINMAX, or NULL */
    float* maxs;             /* LR_OP_ROW_MINMAX, or NULL */
} lr_tensors;

/* Runs `op` exactly as its typed entry point does, and may also use the
 * SPLIT family, whose partial statistics live in `workspace`.
 *   workspace:  device memory owned by the caller, 16-byte aligned
 *               (LR_ERR_MISALIGNED), overlapping no tensor of the call
 *               (LR_ERR_ALIASING); NULL when workspace_bytes is 0.  Its
 *               contents on entry do not matter; the call overwrites the
 *               first lr_plan_workspace_bytes(plan, rows) bytes (stream
 *               order: the call's kernels finish with it before later
 *               work on `stream`).  Calls that may run concurrently need
 *               workspaces of their own.
 *   plan NULL:  the automatic plan; it splits rows only when that is
 *               faster and workspace_bytes >= lr_workspace_query's figure,
 *               and otherwise equals the typed entry point's plan.
 *   plan given: honoured exactly or rejected, as for the _with_plan calls;
 *               a SPLIT plan with a smaller workspace returns LR_ERR_WORKSPACE.
 * Unused members of `tensors` must be NULL (else LR_ERR_INVALID_ARGUMENT). */
lr_status lr_run_f32(lr_op op, const lr_tensors* tensors, int64_t rows, int64_t cols, float eps,
                     lr_reduction_policy policy, const lr_plan* plan, void* workspace,
                     uint64_t workspace_bytes, hipStream_t stream);

/* A measurement, not an operation of the pages: copies each row through the
 * CACHE family's data path under `plan`,
 *   y[r][j] = x[r][j],
 * with the same workgroup per row, the same 16-byte buffer reads of the
 * row's chunks (lane w of the team reads chunks w, w + W, ..., W = 64 x
 * waves_per_row) and the same streamed stores as the reductions, with no
 * arithmetic and no parameter read between them.  sync = 1: every wave
 * waits for its reads and the workgroup meets at one barrier before the
 * first store, as the reductions' cross-wave exchange makes them do; sync =
 * 0: each wave stores as soon as its own reads land; any other value is
 * LR_ERR_INVALID_ARGUMENT.  Its time under an operation's plan is the floor
 * under that operation's launch-to-launch time ("Whole-launch reduction
 * cost policy" measures whole launches).
 * Aligned rows only: cols % 4 == 0 and x, y 16-byte aligned, else
 * LR_ERR_MISALIGNED.  plan: a CACHE plan with rows_per_block 1, lanes_per_row
 * 64 x waves_per_row, chunks_per_lane 1, 2, 3, 4, 6 or 8, whose lanes cover
 * the row (64 x waves_per_row x chunks_per_lane x 4 >= cols), else
 * LR_ERR_UNREALIZABLE_PLAN before any launch.  y may equal x; a partial
 * overlap is LR_ERR_ALIASING.  rows == 0 returns LR_OK without a launch. */
lr_status lr_copy_rows_f32(const float* x, float* y, int64_t rows, int64_t cols,
                           const lr_plan* plan, int32_t sync, hipStream_t stream);

/* Bytes of the device array lr_run_f32_noalloc uses in place of a workspace
 * (one copy per GPU, held until the process ends): room for 131072 split-row
 * partials, e.g. 2048 rows cut into 64 segments. */
#define LR_NOALLOC_SCRATCH_BYTES (1u << 20)

/* lr_run_f32 for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as lr_run_f32 with a workspace of
 * LR_NOALLOC_SCRATCH_BYTES bytes, except that the workspace is a device array
 * the library owns, one per GPU (its address on the current device is looked
 * up on the first call there).  The call allocates and frees nothing.
 *   - An explicit SPLIT plan whose partials (lr_plan_workspace_bytes) exceed
 *     LR_NOALLOC_SCRATCH_BYTES returns LR_ERR_WORKSPACE before any launch;
 *     the automatic plan splits rows only when its partials fit.
 *   - Every call on one GPU shares that GPU's array.  Each call writes every
 *     partial it reads, so nothing carries over, but calls whose work
 *     overlaps in time on one GPU (different streams or host threads) race
 *     on the array: order them on one stream.
 *   - `stream` must belong to the current device.  LR_ERR_HIP if the array's
 *     address cannot be looked up. */
lr_status lr_run_f32_noalloc(lr_op op, const lr_tensors* tensors, int64_t rows, int64_t cols, float eps,
                             lr_reduction_policy policy, const lr_plan* plan, hipStream_t stream);

/* Workspace bytes lr_run_f32's automatic plan uses for this problem on the
 * current device with a workspace available (0 when it does not split):
 * the larger of the figures for 16-byte aligned and for misaligned rows. */
lr_status lr_workspace_query(lr_op op, int64_t rows, int64_t cols, lr_reduction_policy policy,
                             uint64_t* bytes);

/* Workspace bytes `plan` needs for `rows` rows: rows * splits * 8 for a SPLIT
 * plan, 0 for any other (and for a NULL plan). */
uint64_t lr_plan_workspace_bytes(const lr_plan* plan, int64_t rows);

/* Rows one kernel dispatch of `plan` covers in a call over `rows` rows.  A
 * dispatch carries at most 2^31 work-items (the dispatch packet's grid size
 * is 32 bits), so a call whose grid would be larger -- only possible with
 * about 2^21 rows or more -- runs as consecutive dispatches of this many rows
 * on its stream, the last one holding the rest; results are those of one
 * dispatch.  Returns 0 for a NULL plan or rows < 1. */
int64_t lr_dispatch_rows(const lr_plan* plan, int64_t rows);

/* ---------------------------------------------------------------------------
 * Planner (host only; no device memory touched)
 * ------------------------------------------------------------------------- */

/* Facts of the current HIP device (hipGetDeviceProperties).  LR_ERR_HIP when
 * no device is usable. */
lr_status lr_device_facts_query(lr_device_facts* out);

/* Facts of an MI355X, for planning without a device. */
void lr_device_facts_mi355x(lr_device_facts* out);

/* The current HIP device's memory clock (kHz) and memory bus width (bits),
 * as the runtime reports them, so that a measurement can state the device it
 * ran on beside the peak bandwidth it divides by.  NULL outputs:
 * LR_ERR_NULL_POINTER; no usable device: LR_ERR_HIP. */
lr_status lr_device_memory_query(int32_t* clock_khz, int32_t* bus_width_bits);

/* The plan an operation launches with on the current device, assuming
 * 16-byte aligned tensor bases and, for RMSNorm and LayerNorm, gamma or beta
 * given (a norm called without both may take a plan measured for that case). */
lr_status lr_plan_query(lr_op op, int64_t rows, int64_t cols,
                        lr_reduction_policy policy, lr_plan* out);

/* Pure planner: the automatic plan for `facts`.  row_aligned = 1 when every
 * row starts 16-byte aligned (cols % 4 == 0 and aligned bases).  Never a
 * SPLIT plan (the typed entry points have no workspace).  For RMSNorm and
 * LayerNorm, the plan of a call that gives gamma or beta. */
lr_status lr_plan_for_device(const lr_device_facts* facts, lr_op op, int64_t rows,
                             int64_t cols, lr_reduction_policy policy,
                             int32_t row_aligned, lr_plan* out);

/* The automatic plan when a workspace is available: lr_plan_for_device's
 * plan, or a SPLIT plan for rows too few to fill the device. */
lr_status lr_plan_for_device_ws(const lr_device_facts* facts, lr_op op, int64_t rows,
                                int64_t cols, lr_reduction_policy policy,
                                int32_t row_aligned, lr_plan* out);

/* Every legal plan, in enumeration order (family, S, Q; SPLIT plans last,
 * for splits = 2, 4, .., 64 up to the row's chunk count).  Writes at most
 * `capacity` plans to `out` (out may be NULL when capacity is 0) and the
 * total number of legal plans to *count. */
lr_status lr_plan_enumerate(const lr_device_facts* facts, lr_op op, int64_t rows,
                            int64_t cols, lr_reduction_policy policy,
                            int32_t row_aligned, lr_plan* out, int32_t capacity,
                            int32_t* count);

/* LR_OK when `plan` is realisable for this problem on `facts`, else the
 * reason (LR_ERR_UNREALIZABLE_PLAN or an argument error). */
lr_status lr_plan_validate(const lr_device_facts* facts, lr_op op, int64_t rows,
                           int64_t cols, lr_reduction_policy policy,
                           int32_t row_aligned, const lr_plan* plan);

/* Host replay of a plan's thread -> element mapping (the same index functions
 * the kernels are compiled from): adds 1 to counts[r*cols + e] for every
 * (row r, element e) some thread of the launch owns, for rows whose first
 * element sits `phase` floats past a 16-byte boundary when r == 0 (each later
 * row shifted by cols).  counts: rows*cols uint32 host array.  Used to prove
 * that each element is covered exactly once (section 4.4 of the pages). */
lr_status lr_coverage_check(const lr_plan* plan, int64_t rows, int64_t cols,
                            int32_t phase, uint32_t* counts);

/* Human-readable name of a status code (static storage). */
const char* lr_status_string(lr_status status);

/* Library version string, e.g. "lr 0.1.0 gfx950". */
const char* lr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LR_H */
