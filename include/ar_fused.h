/*
 * ar_fused.h -- C ABI of the MI355X (gfx950) fused all-reduce-sum (+ residual + RMSNorm) core.
 *
 * The library computes one GPU's share of a one-shot all-reduce: the element-wise sum of W
 * per-rank partial tensors [M, H] that are all readable from this GPU, optionally followed by a
 * residual add and RMSNorm, in one kernel launch.  The two operations are the fusion patterns
 * "kAllReduce" and "kARResidualRMSNorm" named in the tokenspeed pull request "perf(comm): route
 * generic MNNVL AR patterns to upstream flashinfer" (Summary, Routing).
 *
 * Arithmetic (the same for every launch shape):
 *   a            = x_0 + x_1 + ... + x_{W-1}        binary32, in rank order 0..W-1, one
 *                                                   round-to-nearest-even per add, seeded with
 *                                                   x_0 (a sum of -0 stays -0)
 *   ar_sum:        out = RN_T(a)
 *   ar_residual_rmsnorm:
 *                  a            = a + residual      (the residual is the last term)
 *                  residual_out = RN_T(a)
 *                  v            = residual_out, widened exactly to binary32
 *                  norm_out     = RN_T( v * rsqrt(mean_i(v_i^2) + eps) * gamma )
 * out and residual_out are bit-identical to that definition; norm_out is computed in binary32
 * (sum of squares reduced in a fixed tree order) and is within one unit in the last place of T
 * of the same expression evaluated exactly.  RMSNorm is the textbook form (mean over the whole
 * row, eps inside the square root, gamma after normalising, no bias); the pages name the
 * pattern but give no formula.  Subnormals are kept (no flush to zero); T overflow gives inf.
 *
 * Layout: every [M, H] tensor is row-major and contiguous (row stride H elements), one
 * allocation per partial.  gamma is binary32 [H] for every element type.
 *
 * Ownership: the caller owns every buffer.  `inputs` is a HOST array of W DEVICE pointers; it is
 * read during the call and not retained.  The library allocates no device memory and retains
 * no pointer (the one scratch buffer, the split form's workspace below, is the caller's, except
 * for ar_residual_rmsnorm_noalloc, whose slots are a fixed device array of the library), so
 * calls are safe to capture in a hipGraph and replay.  The only other state is a per-device
 * cache of the compute-unit count.
 *
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue one kernel (two
 * for ar_residual_rmsnorm_unfused) and return without synchronising; the return code reports
 * argument validation and the launch only.
 * Device faults surface on the stream as usual.
 *
 * Errors: every entry point returns an ar_status_t.  On any non-zero status nothing was launched
 * and no output byte was written.  Rejections follow the pages' runtime rejection of unsupported
 * world sizes with a caller-side fallback (vLLM pull request "[Perf] Tune FlashInfer all-reduce
 * selection on SM103", Scope and Tests: world size 12 is rejected, {2, 4, 8, 16, 32, 64} are
 * supported); W = 1 is accepted as well.
 */
#ifndef AR_FUSED_H
#define AR_FUSED_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type T of the partials, residual and outputs. */
typedef enum {
  AR_DTYPE_FP32 = 0, /* binary32 */
  AR_DTYPE_FP16 = 1, /* binary16 */
  AR_DTYPE_BF16 = 2  /* bfloat16 */
} ar_dtype_t;

/* Fusion pattern (for ar_supports / ar_launch_config). */
typedef enum {
  AR_PATTERN_ALLREDUCE = 0,             /* kAllReduce: out = sum */
  AR_PATTERN_AR_RESIDUAL_RMSNORM = 1    /* kARResidualRMSNorm */
} ar_pattern_t;

typedef enum {
  AR_OK = 0,
  AR_ERR_INVALID_ARG = 1, /* null pointer, W < 1, M < 0, H < 1, bad dtype/pattern, bad eps,
                             malformed launch config */
  AR_ERR_UNSUPPORTED = 2, /* W not in {1,2,4,8,16,32,64}; H not a multiple of 16/sizeof(T)
                             (norm pattern) or H above AR_MAX_H_16BIT / AR_MAX_H_FP32 */
  AR_ERR_MISALIGNED = 3,  /* a tensor pointer is not 16-byte aligned (gamma: 16 bytes too) */
  AR_ERR_ALIAS = 4,       /* outputs overlap each other, gamma, or partially overlap an input */
  AR_ERR_LAUNCH = 5,      /* the HIP launch itself failed */
  AR_ERR_DEVICE = 6       /* no usable HIP device (device query failed) */
} ar_status_t;

/* Largest hidden size accepted by the residual+RMSNorm pattern (a row is held in registers
 * by at most 1024 threads x 8 vectors of 16 bytes). */
#define AR_MAX_H_16BIT 65536
#define AR_MAX_H_FP32 32768
/* Largest number of partials. */
#define AR_MAX_W 64

/* Launch shape.  Produced by ar_launch_config; accepted by the *_with_config entry points for
 * tuning (the kernel and its arithmetic are the same for every valid shape).
 *   threads_per_block : multiple of 64, 64..1024
 *   vecs_per_thread   : 16-byte vectors each thread handles per row (norm: 1, 2, 4 or 8) or
 *                       per grid-stride iteration (sum: 1, 2 or 4)
 *   lanes_per_row     : norm pattern only: threads that share one row; a power of two <= 64
 *                       or a multiple of 64; threads_per_block % lanes_per_row == 0 and
 *                       lanes_per_row * vecs_per_thread >= H / (16 / sizeof(T))
 *   rows_per_block    : norm pattern only: threads_per_block / lanes_per_row
 *   grid              : number of blocks (>= 1); blocks loop over the work with a grid stride
 *   flat              : 1 for the sum pattern (flat vector decomposition), 0 for the norm
 *   nt_store          : 1 = outputs are written with non-temporal stores, 0 = ordinary stores
 *                       (inputs are always read with non-temporal loads)
 *   ranks_per_batch   : norm pattern only: 0 = each thread issues up to 16 loads across ranks
 *                       per batch; 1, 2 or 4 = it loads that many ranks' vectors per batch
 *                       (same results).  Allowed with nt_store = 1 for: 1 with 2 vectors per
 *                       thread at 4 <= W <= 16 or 4 vectors at W = 2 and 4; 2 with 2 vectors
 *                       at W >= 4 or 1 vector at W >= 32; 4 with 2 vectors at W = 8.  0 for the
 *                       sum pattern */
typedef struct {
  int32_t threads_per_block;
  int32_t vecs_per_thread;
  int32_t lanes_per_row;
  int32_t rows_per_block;
  int32_t grid;
  int32_t flat;
  int32_t nt_store;
  int32_t ranks_per_batch;
} ar_launch_cfg_t;

/* kAllReduce.  out[m, i] = RN_T(x_0[m, i] + ... + x_{W-1}[m, i]).
 *   inputs : host array of W device pointers to [M, H] tensors of type `dtype`
 *   out    : device [M, H]; may be exactly one of the inputs (in place), must not partially
 *            overlap any input
 * M = 0 returns AR_OK without launching.  Any M * H is accepted (a tail shorter than one
 * 16-byte vector is handled element-wise). */
int ar_sum(const void* const* inputs, int W, int64_t M, int64_t H, int dtype, void* out,
           void* stream);

/* kARResidualRMSNorm.
 *   inputs       : host array of W device pointers to [M, H] tensors of type `dtype`
 *   residual     : device [M, H] of type `dtype`
 *   gamma        : device [H] binary32
 *   eps          : finite, >= 0
 *   residual_out : device [M, H]; may be exactly `residual` or an input (in place)
 *   norm_out     : device [M, H]; may be exactly `residual` or an input; must not overlap
 *                  residual_out or gamma
 * H must be a multiple of 16 / sizeof(T) (8 for 16-bit types, 4 for binary32).
 * M = 0 returns AR_OK without launching. */
int ar_residual_rmsnorm(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                        const void* residual, const float* gamma, float eps, void* residual_out,
                        void* norm_out, void* stream);

/* Shape-level support check, no device access: AR_OK if the pattern accepts (W, M, H, dtype),
 * else the status the entry point would return.  Lets a caller pick its fallback first.  This is
 * the supports() of the tokenspeed pull request (Summary, Memory), which also bounds a call by
 * the buffer bytes it actually needs: ar_sum and ar_residual_rmsnorm need no workspace, so the
 * shape is the whole check here (the split form's bound is ar_split_workspace_bytes, the
 * no-alloc form's AR_NOALLOC_MAX_ROWS). */
int ar_supports(int pattern, int W, int64_t M, int64_t H, int dtype);

/* Launch-shape heuristic: maps (pattern, W, M, H, dtype) and the compute-unit count to a launch
 * shape -- the MI355X counterpart of the thread-block / cluster sizing against the SM count in
 * the flashinfer pull request "update allreduce to match trtllm" (Description, Summary).
 *   cu_count : compute units to plan for; <= 0 queries the current HIP device (cached).
 * Pure host arithmetic when cu_count > 0.  Returns AR_OK and fills *cfg, or an error status. */
int ar_launch_config(int pattern, int W, int64_t M, int64_t H, int dtype, int cu_count,
                     ar_launch_cfg_t* cfg);

/* Same as ar_sum / ar_residual_rmsnorm with an explicit launch shape (tuning and tests).
 * A shape that is malformed or does not cover the row returns AR_ERR_INVALID_ARG. */
int ar_sum_with_config(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                       void* out, void* stream, const ar_launch_cfg_t* cfg);
int ar_residual_rmsnorm_with_config(const void* const* inputs, int W, int64_t M, int64_t H,
                                    int dtype, const void* residual, const float* gamma,
                                    float eps, void* residual_out, void* norm_out, void* stream,
                                    const ar_launch_cfg_t* cfg);

/* ---- few rows: one row split over several blocks ---------------------------------------------------
 *
 * At decode sizes (few rows) the launch shape, not the arithmetic, sets the time (the flashinfer
 * pull request "update allreduce to match trtllm", Description: the thread-block / cluster
 * retuning for a concurrency-128 decode step).  One block per row then leaves most CUs idle and
 * one CU streams the row's W + 1 inputs.  ar_residual_rmsnorm_ws lets S blocks share a row
 * (the CDNA4 stand-in for a thread-block cluster): each sums its segment, writes residual_out,
 * publishes its segment's sum of squares in a caller workspace, reads the others' and finishes
 * the norm.  Results as ar_residual_rmsnorm (residual_out bit-identical; norm_out within one ulp
 * of T of the exact expression, deterministic for a given launch shape).
 *
 * Workspace: device memory of ar_split_workspace_bytes(M) bytes (AR_SPLIT_SLOTS 8-byte slots
 * per row), 16-byte aligned, owned by the caller, zero-filled once before its first use (e.g. by
 * ar_workspace_clear) and then left to the library: every call leaves it valid for the next,
 * for any shape up to the rows it was sized for.  Calls that share a workspace must not run
 * concurrently (issue them on one stream).  A workspace that was not zero-filled can make
 * norm_out wrong.  The workspace must not overlap any tensor argument.
 *
 * Waits are bounded: a block that has polled max_polls times without seeing every segment's sum
 * computes them all itself (same arithmetic, same result, slower), so the kernel always ends. */
#define AR_SPLIT_SLOTS 64

/* Split launch shape.
 *   threads_per_block : L, multiple of 64, 64..1024
 *   vecs_per_thread   : 1 or 2
 *   segments          : S = ceil((H / (16 / sizeof(T))) / (L * vecs_per_thread)), 1..64
 *                       (checked).  Split launches take up to 65535 rows (AR_ERR_UNSUPPORTED
 *                       beyond; the planner splits only far fewer rows): a grid of 8 x S blocks
 *                       below 8 rows, S x M from 8
 *   max_polls         : polls of the exchange before a block computes the row alone (0: never
 *                       wait; every block then reads the whole row) */
typedef struct {
  int32_t threads_per_block;
  int32_t vecs_per_thread;
  int32_t segments;
  uint32_t max_polls;
} ar_split_cfg_t;

/* Workspace bytes for calls of up to M rows: M * AR_SPLIT_SLOTS * 8; -1 for M < 0 or
 * M > 2^40. */
int64_t ar_split_workspace_bytes(int64_t M);

/* Zero-fills `workspace_bytes` (a multiple of 8) bytes at `workspace` (16-byte aligned) with a
 * kernel on `stream` (no memset node, so it may be captured in a hipGraph). */
int ar_workspace_clear(void* workspace, int64_t workspace_bytes, void* stream);

/* The split the heuristic picks for (W, M, H, dtype) on cu_count CUs (<= 0: the current device):
 * AR_OK with *cfg filled, or all fields 0 when it keeps one block per row for this shape; the
 * shape's status otherwise.  Pure host arithmetic when cu_count > 0. */
int ar_split_config(int W, int64_t M, int64_t H, int dtype, int cu_count, ar_split_cfg_t* cfg);

/* kARResidualRMSNorm with a workspace.  Arguments as ar_residual_rmsnorm plus
 *   workspace, workspace_bytes : as described above (bytes >= ar_split_workspace_bytes(M))
 * Runs the split kernel when ar_split_config splits the shape and neither output overlaps the
 * residual or an input; otherwise exactly ar_residual_rmsnorm (in-place calls included).
 * AR_ERR_INVALID_ARG for a null or too small workspace, AR_ERR_MISALIGNED, AR_ERR_ALIAS if it
 * overlaps a tensor. */
int ar_residual_rmsnorm_ws(const void* const* inputs, int W, int64_t M, int64_t H, int dtype,
                           const void* residual, const float* gamma, float eps,
                           void* residual_out, void* norm_out, void* workspace,
                           int64_t workspace_bytes, void* stream);

/* kARResidualRMSNorm for callers that cannot allocate: code under hipGraph capture, tight
 * serving loops, harnesses that forbid allocation.  Arguments, results and rejections as
 * ar_residual_rmsnorm; the launch as ar_residual_rmsnorm_ws, with the split kernel's exchange
 * slots in a device array inside the library instead of a caller workspace: AR_NOALLOC_MAX_ROWS
 * rows of AR_SPLIT_SLOTS 8-byte slots (256 KiB), one copy per GPU, held until the process ends.
 * Nothing is allocated: the first call on a device looks up that array's address and clears it
 * with a kernel on `stream` (no memset node); make that first call outside graph capture (a
 * warm-up call, as before any capture).
 *   M > AR_NOALLOC_MAX_ROWS : AR_ERR_UNSUPPORTED (ar_residual_rmsnorm needs no scratch at all)
 * Every call on one GPU shares that GPU's array and leaves it valid for the next call; calls
 * that overlap in time on one GPU (other streams, other threads) race on it and may produce
 * wrong norm_out: issue them on one stream. */
#define AR_NOALLOC_MAX_ROWS 512
int ar_residual_rmsnorm_noalloc(const void* const* inputs, int W, int64_t M, int64_t H,
                                int dtype, const void* residual, const float* gamma, float eps,
                                void* residual_out, void* norm_out, void* stream);

/* The split kernel with an explicit shape (tuning and tests).  AR_ERR_INVALID_ARG for a
 * malformed shape, AR_ERR_ALIAS if an output overlaps the residual or an input. */
int ar_residual_rmsnorm_split_with_config(const void* const* inputs, int W, int64_t M, int64_t H,
                                          int dtype, const void* residual, const float* gamma,
                                          float eps, void* residual_out, void* norm_out,
                                          void* workspace, int64_t workspace_bytes, void* stream,
                                          const ar_split_cfg_t* cfg);

/* ---- two-shot share -----------------------------------------------------------------------
 *
 * The two-shot form of the all-reduce (named beside the one-shot form in the vLLM pull request
 * "[Perf] Tune FlashInfer all-reduce selection on SM103", Tests, and the tokenspeed pull
 * request, Summary) splits the rows among the W ranks: rank k reduces only its row slice
 * (reduce-scatter), then every rank gathers the W reduced slices (all-gather).  Rows are
 * independent, so rank k's reduce-scatter share is ar_sum / ar_residual_rmsnorm called on the
 * row slice (pointers advanced by row_begin * H elements, M = row_count); ar_all_gather is the
 * gather share.  Both use the partition below. */

/* Row slice of `rank` (0 <= rank < W) in the W-way partition of M rows:
 * row_begin = floor(rank * M / W), row_count = floor((rank + 1) * M / W) - row_begin.
 * Pure host arithmetic.  AR_OK, or AR_ERR_INVALID_ARG for bad arguments or null outputs. */
int ar_row_partition(int W, int64_t M, int rank, int64_t* row_begin, int64_t* row_count);

/* All-gather share: out[row_begin(j) + i, :] = slices[j][i, :] for every rank j and every row i
 * of its slice (the partition above), one launch for all W slices.
 *   slices : host array of W device pointers; slices[j] is [row_count(j), H] of type `dtype`
 *            (row-major, contiguous, 16-byte aligned).  A slice that already sits at its place
 *            in `out` (slices[j] == out + row_begin(j) * H) is skipped.
 *   out    : device [M, H]; must not partially overlap any slice
 * W must be in the supported set; H must be a multiple of 16 / sizeof(T).  A byte copy (non-
 * temporal loads and stores): the result is bit-identical to the slices. */
int ar_all_gather(const void* const* slices, int W, int64_t M, int64_t H, int dtype, void* out,
                  void* stream);

/* ---- Lamport-style one-shot exchange ------------------------------------------------------------
 *
 * The one-shot exchange of the MNNVL all-reduce (flashinfer pull request "Optimizations for
 * TRTLLM MNNVL Allreduce", Description and Summary: Lamport polling with vectorized loads,
 * buffer state kept in the data) carries no separate flag.  A receive buffer `rbuf` holds
 * AR_LAMPORT_BUFFERS (3) buffers of W slots of [M, H] elements of type `dtype`: slot r of buffer b
 * sits at byte offset (b * W + r) * M * H * sizeof(T).  An empty element holds the all-ones bit
 * pattern (a NaN in every type).  Rounds are numbered 0, 1, 2, ... by the caller; round k uses
 * buffer k mod 3.  The producer of rank r in round k writes its partial into slot r of buffer
 * k mod 3 and empties slot r of buffer (k + 1) mod 3 (the one round k - 2 used); consumers poll
 * each element of buffer k mod 3 until it is not all ones and reduce exactly as ar_sum /
 * ar_residual_rmsnorm, reading only.  A partial element that is itself all ones is delivered
 * with its lowest bit cleared (a NaN either way).
 *
 * Ordering contract: every rank calls, per round, push then a consumer, on one stream (or with
 * the consumer of round k - 1 complete before the push of round k).  Then the push of round k
 * empties a slot no consumer still reads: its rank finished consuming round k - 1, which needed
 * every rank's push of round k - 1, made after that rank consumed round k - 2.  Producers and
 * consumers of one round may run concurrently on other streams of the same GPU: slots move as
 * 16-byte device-coherent accesses (agent scope; each aligned dword single-copy atomic; elements
 * are tested one by one), and each producer thread empties its vector of the next buffer, and
 * waits for that store to complete, before it stores its vector of the current one.  (Producers
 * on other GPUs writing through peer mappings would need system-scope accesses; this library
 * runs the exchange on one GPU.)  A captured graph replays the same round numbers: capture 3 consecutive rounds (or a
 * multiple of 3) so that replays keep the rotation.
 *
 * Every wait is bounded: after `spin_limit` polls of one 16-byte vector (0 = 65536) the consumer
 * gives up on it, sets bit 0 of *status (a device int the caller clears) and carries on; the
 * outputs are then meaningless and the exchange must be re-armed.  H must be a multiple of
 * 16 / sizeof(T); the fused consumer takes rows of at most 8192 16-byte vectors for W <= 4
 * and 4096 for W >= 8 (H <= 65536 / 32768 at 16 bits).  round < 0 is AR_ERR_INVALID_ARG. */

#define AR_LAMPORT_BUFFERS 3

/* Empties every slot of the 3 buffers (every element all ones).  Call once before round 0, and
 * again after a consumer reported a time-out. */
int ar_lamport_arm(void* rbuf, int W, int64_t M, int64_t H, int dtype, void* stream);

/* Producer of rank `rank` in round `round`: copies `partial` ([M, H], must not overlap rbuf)
 * into slot `rank` of buffer round mod 3 and empties slot `rank` of buffer (round + 1) mod 3. */
int ar_lamport_push(const void* partial, int rank, void* rbuf, int W, int64_t M, int64_t H,
                    int dtype, int64_t round, void* stream);

/* Consumer of round `round`, kAllReduce: out = sum of the W slots of buffer round mod 3 (as
 * ar_sum).  out must not overlap rbuf or *status. */
int ar_lamport_sum(void* rbuf, int W, int64_t M, int64_t H, int dtype, int64_t round, void* out,
                   int* status, uint32_t spin_limit, void* stream);

/* Consumer of round `round`, kARResidualRMSNorm (as ar_residual_rmsnorm) over buffer round mod 3.
 * residual, gamma and both outputs must not overlap rbuf; outputs must not overlap *status. */
int ar_lamport_residual_rmsnorm(void* rbuf, int W, int64_t M, int64_t H, int dtype, int64_t round,
                                const void* residual, const float* gamma, float eps,
                                void* residual_out, void* norm_out, int* status,
                                uint32_t spin_limit, void* stream);

/* ---- two-kernel (unfused) path and the stand-alone RMSNorm -------------------------------------------
 *
 * The pages' policy layer sends calls the fused kernel cannot take to an unfused fallback (the
 * tokenspeed pull request, Body and Routing, uses each path as the other's shape fallback; the
 * vLLM pull request, Scope, routes unsupported cases to the fallback).  This library's own
 * fallback for kARResidualRMSNorm is two kernels on the stream: the flat sum kernel with the
 * residual as the last addend (residual_out), then RMSNorm of residual_out (norm_out).  It takes
 * rows of any width H >= 1 (the fused kernel needs whole 16-byte vectors per row and at most
 * AR_MAX_H_16BIT / AR_MAX_H_FP32 elements), with the same results: residual_out bit-identical,
 * norm_out within one unit in the last place of T of the exact expression. */

/* RMSNorm of a stored tensor, the normalisation step of kARResidualRMSNorm alone:
 *   y[m, i] = RN_T( x[m, i] * rsqrt(mean_i(x[m, i]^2) + eps) * gamma[i] )
 *   x     : device [M, H] of type `dtype`, 16-byte aligned; any H >= 1
 *   gamma : device [H] binary32, 16-byte aligned
 *   eps   : finite, >= 0
 *   y     : device [M, H]; may be exactly x (in place); must not partially overlap x or overlap
 *           gamma
 * Rows of whole 16-byte vectors up to AR_MAX_H_16BIT / AR_MAX_H_FP32 elements run the fused
 * kernel's row machinery (one read, values kept in registers); other rows run a two-pass kernel
 * (the second pass re-reads the row, normally from cache).  M = 0 returns AR_OK. */
int ar_rmsnorm(const void* x, int64_t M, int64_t H, int dtype, const float* gamma, float eps,
               void* y, void* stream);

/* kARResidualRMSNorm as two kernels, for any H >= 1.  Arguments, aliasing rules and results as
 * ar_residual_rmsnorm; W in the same supported set.  Enqueues two kernels on `stream`.  The one
 * exception to "nothing launched on error": if the second launch fails, AR_ERR_LAUNCH is
 * returned after the first (residual_out) was enqueued; norm_out is then not written. */
int ar_residual_rmsnorm_unfused(const void* const* inputs, int W, int64_t M, int64_t H,
                                int dtype, const void* residual, const float* gamma, float eps,
                                void* residual_out, void* norm_out, void* stream);

/* ---- routing policy ------------------------------------------------------------------------------
 *
 * The policy layer that picks a path per call, after the pages: the tokenspeed pull request
 * (Body, Routing) splits by token count (32 by default: decode sizes stay on the latency path)
 * and treats an unsupported shape as a reason to take the other path; the vLLM pull request
 * (Scope, Performance) keys strict per-rank payload cutoffs by topology and sends world size 12
 * to the fallback.  ar_route is pure host arithmetic. */
typedef enum {
  AR_ROUTE_ONE_SHOT = 0,  /* ar_sum / ar_residual_rmsnorm over all W peers' buffers */
  AR_ROUTE_TWO_SHOT = 1,  /* reduce-scatter share on the rank's rows, then ar_all_gather */
  AR_ROUTE_FALLBACK = 2,  /* not this library: the caller's collective (e.g. RCCL) */
  AR_ROUTE_UNFUSED = 3    /* kARResidualRMSNorm rows the fused kernel does not take:
                             ar_residual_rmsnorm_unfused */
} ar_route_t;

typedef struct {
  int64_t min_tokens;          /* M below this always takes one-shot (latency-bound sizes) */
  int64_t two_shot_min_bytes;  /* from this per-rank payload (M * H * sizeof(T)) on, and with
                                  M >= min_tokens, two-shot */
  int64_t max_payload_bytes;   /* per-rank payload above this goes to the fallback (the
                                  workspace capacity); 0 = no limit */
} ar_policy_t;

/* Default policy for W ranks of one MI355X node (all-to-all xGMI: one ~153 GB/s link per peer
 * pair).  min_tokens = 32 (the tokenspeed default).  two_shot_min_bytes comes from a link model:
 * one-shot moves the whole payload S over each peer link, two-shot 2 S / W but pays a second
 * exchange (~5 us); two-shot wins once S (1 - 2 / W) / 153 GB/s exceeds 5 us, i.e. from
 * 5 us * 153 GB/s / (1 - 2 / W) (W = 8: 1.02 MB); for W <= 2 two-shot never wins (INT64_MAX).
 * max_payload_bytes = 0: no path here needs a payload-sized workspace.  A model, not a
 * measurement: the crossover needs two GPUs to measure. */
int ar_policy_default(int W, ar_policy_t* policy);

/* Route for one call: AR_ROUTE_FALLBACK if neither the fused kernel nor the two-kernel path
 * takes the shape (e.g. W = 12) or the payload exceeds max_payload_bytes; AR_ROUTE_UNFUSED for a
 * norm row only the two-kernel path takes (H not a multiple of 16 / sizeof(T), or above the
 * fused limit); otherwise AR_ROUTE_ONE_SHOT below min_tokens or below two_shot_min_bytes, else
 * AR_ROUTE_TWO_SHOT.  Returns AR_OK and sets *route, or
 * AR_ERR_INVALID_ARG for a null pointer, a negative threshold or a bad pattern. */
int ar_route(int pattern, int W, int64_t M, int64_t H, int dtype, const ar_policy_t* policy,
             int* route);

/* One call on the path ar_route picks, on this GPU: the tokenspeed pull request (Summary and
 * Routing) has a dispatch check the shape (supports()) and a token threshold before choosing a
 * path, each path serving as the other's shape fallback, and an unsupported call leaves the
 * library.  `pattern` is AR_PATTERN_ALLREDUCE (`out` receives the sum; residual, gamma, eps and
 * norm_out are ignored and may be null) or AR_PATTERN_AR_RESIDUAL_RMSNORM (`out` is
 * residual_out).  Arguments, layouts and aliasing rules are those of the entry point the route
 * runs; `policy` is as for ar_route; 0 <= rank < W is the calling rank.
 *   AR_ROUTE_ONE_SHOT : ar_sum / ar_residual_rmsnorm over all M rows
 *   AR_ROUTE_UNFUSED  : ar_residual_rmsnorm_unfused over all M rows
 *   AR_ROUTE_TWO_SHOT : this rank's reduce-scatter share only: the same reduction over the rows
 *                       [row_begin, row_begin + row_count) of ar_row_partition(W, M, rank),
 *                       written to those rows of the outputs; the caller completes the call with
 *                       ar_all_gather once every rank's share is done
 *   AR_ROUTE_FALLBACK : nothing is launched; returns AR_ERR_UNSUPPORTED (the caller's own
 *                       collective takes the call)
 * *route is set to the route taken whenever ar_route succeeds and rank is valid; the status is
 * that of the entry point run, or ar_route's error, or AR_ERR_INVALID_ARG for a null `route` or a
 * bad rank. */
int ar_allreduce_routed(int pattern, const void* const* inputs, int W, int64_t M, int64_t H,
                        int dtype, const void* residual, const float* gamma, float eps, void* out,
                        void* norm_out, int rank, const ar_policy_t* policy, int* route,
                        void* stream);

/* Static, human-readable name of a status code ("unknown status" for anything else). */
const char* ar_status_string(int status);

/* Compute units of the current HIP device (cached per device).  AR_OK or AR_ERR_DEVICE. */
int ar_device_cu_count(int* cu_count);

#ifdef __cplusplus
}
#endif

#endif /* AR_FUSED_H */
