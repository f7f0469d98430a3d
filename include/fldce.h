/*
 * fldce.h - fused linear diffusion cross-entropy (LM head) for MI355X / gfx950.
 *
 * C ABI of libfldce.so.  Every pointer argument is caller-owned device memory
 * (HIP / PyTorch allocations) unless stated otherwise; the library never
 * allocates, frees or synchronises inside a call.  All work is enqueued on the
 * caller's HIP stream (`stream`, a hipStream_t passed as void*; NULL = the
 * null stream of the current device) and is asynchronous with respect to the
 * host.  Every pointer of a call must be memory of that stream's device.
 *
 * What is computed (model page "fused_linear_diffusion_cross_entropy.py",
 * functions fused_linear_cross_entropy_forward, logsumexp_fwd and
 * cross_entropy_kernel, steps 4-6):
 *
 *   z      = s * (h W^T [+ b])                       logits, s = logit_scale
 *   lse_i  = log sum_j exp(z_ij)                     stable row logsumexp
 *   l_i    = [(1-eps)(lse_i - z_{i,y_i}) + eps(lse_i - mean_j z_ij)] / p_i
 *            (0 when y_i == ignore_index)            eps = label_smoothing
 *   loss   = sum_i l_i / D                           D = 1 (sum) or total (mean)
 *   g_ij   = s/(p_i D) (softmax_ij - eps/V - (1-eps)[j == y_i])   (0 if ignored)
 *   dH     = g W,   dW = g^T h                       gradients for d(loss) = 1
 *
 * Reading taken where the page is inconsistent: the whole label-smoothed CE of
 * a row is divided by p_i (the page's gradient divides every term by p_mask;
 * its printed loss leaves the smoothing term undivided).
 *
 * The vocabulary-shard entry points follow the tensor-parallel tutorial page
 * (daliqc.cn developer article 673292621566021), section 4 "output-layer
 * embedding": each shard produces per-row softmax partials, the partials are
 * combined across shards, and each shard then forms its own slice of the
 * gradient.
 *
 * Layouts: all matrices are dense row-major with no padding: h [N,H],
 * W [V,H] (nn.Linear layout), dH [N,H], dW [V,H].  target is int64 [N];
 * p_mask is float32 [N] (NULL means all ones).  h, W, dH, dW share one dtype:
 * FLDCE_DTYPE_F32 or FLDCE_DTYPE_BF16.  Accumulation is float32 in both cases.
 *
 * Preconditions not checked on the device (undefined results otherwise):
 * 0 <= target[i] < V or target[i] == ignore_index; p_mask[i] > 0 on rows that
 * are not ignored (p_mask of ignored rows is never read as a divisor).
 *
 * Error behaviour: every entry point returns FLDCE_OK (0) or a negative
 * status.  Argument errors are found before anything is enqueued (no output
 * is touched); FLDCE_ERR_HIP reports a failed launch, after which outputs
 * may be partly written.
 * fldce_status_string() gives a static description.  No exception crosses the
 * ABI.  Results are deterministic: no floating-point atomics are used, every
 * reduction has a fixed order.
 *
 * Thread safety: calls are re-entrant; concurrent calls need distinct
 * workspaces and outputs.
 */
#ifndef FLDCE_H
#define FLDCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLDCE_VERSION 2

enum fldce_dtype { FLDCE_DTYPE_F32 = 0, FLDCE_DTYPE_BF16 = 1 };

/* Page 1: reduction "mean" divides by total, "sum" does not. */
enum fldce_reduction { FLDCE_REDUCTION_SUM = 0, FLDCE_REDUCTION_MEAN = 1 };

enum fldce_status {
  FLDCE_OK = 0,
  FLDCE_ERR_NULL_POINTER = -1,   /* a required pointer is NULL                */
  FLDCE_ERR_BAD_SHAPE = -2,      /* N, H or V out of range, shard outside V   */
  FLDCE_ERR_BAD_DTYPE = -3,      /* dtype not one of fldce_dtype              */
  FLDCE_ERR_BAD_ARGUMENT = -4,   /* reduction, label_smoothing or logit_scale */
  FLDCE_ERR_WORKSPACE = -5,      /* workspace NULL or smaller than required   */
  FLDCE_ERR_ALIGNMENT = -6,      /* a pointer is not 16-byte aligned          */
  FLDCE_ERR_HIP = -7,            /* a kernel launch failed                    */
  FLDCE_ERR_UNSUPPORTED = -8,    /* shape the kernels do not handle: bf16 with
                                    H not a multiple of 64, V >= 2^23 or a GEMM
                                    grid of 2^32 work-items or more; fp32 with
                                    V >= 2^30 */
  FLDCE_ERR_SCRATCH_TOO_SMALL = -9 /* fldce_fwd_noalloc: the call needs more
                                    than FLDCE_NOALLOC_SCRATCH_BYTES */
};

/* Device memory fldce_fwd_noalloc may use (64 MiB per device). */
#define FLDCE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Library version (FLDCE_VERSION of the build). */
int fldce_version(void);

/* Static, human-readable text for a status code. */
const char* fldce_status_string(int status);

/* Token rows processed per chunk when chunk_rows == 0 is passed with bf16
 * inputs: all N rows while twice the chunk's [C, V] bf16 buffer of the
 * backward operand stays within 16 GiB, else the largest multiple of 256
 * that fits, and at most 2^22 (fp32 inputs keep two 4-byte buffers, so half
 * as many rows when that bound binds).  Page 1 chunks rows to bound the [C, V] logits buffer;
 * 288 GB of HBM lets one chunk cover every workload here.  H is unused. */
int64_t fldce_default_chunk_rows(int64_t N, int64_t H, int64_t V);

/* Bytes of device workspace fldce_fwd_bwd needs for these sizes (chunk_rows 0
 * = default).  Returns 0 for invalid sizes. */
size_t fldce_workspace_size(int64_t N, int64_t H, int64_t V, int dtype,
                            int64_t chunk_rows);

/*
 * Loss and gradients of the fused LM-head cross-entropy (page 1,
 * fused_linear_cross_entropy_forward: the forward pass computes the loss and
 * both gradients in one go).
 *
 *   h            [N,H] dtype       hidden states (row-major, H contiguous)
 *   W            [V,H] dtype       LM-head weight
 *   target       [N]   int64       class index or ignore_index
 *   p_mask       [N]   float32     masking probability per token; NULL = 1
 *   ignore_index                   rows with this target contribute nothing
 *   label_smoothing  0 <= eps <= 1
 *   logit_scale      s > 0, finite
 *   reduction        FLDCE_REDUCTION_SUM or FLDCE_REDUCTION_MEAN
 *   total            divisor for "mean" when > 0; <= 0 counts the rows whose
 *                    target != ignore_index on the device (no host sync)
 *   loss         [1]   float32     out: loss (overwritten)
 *   dH           [N,H] dtype       out: d loss / d h (overwritten)
 *   dW           [V,H] dtype       out: d loss / d W (overwritten; float32
 *                                  accumulation, rounded once to dtype)
 *   row_lse      [N]   float32     optional out (NULL ok): per-row lse
 *                                  (0 on rows whose target is ignore_index)
 *   row_loss     [N]   float32     optional out (NULL ok): per-row l_i
 *   chunk_rows       rows per chunk, 0 = fldce_default_chunk_rows
 *   workspace        device scratch of at least fldce_workspace_size bytes
 *
 * Rows whose target is ignore_index contribute exactly nothing (page 1,
 * cross_entropy_kernel step 2), so the bf16 path never multiplies them: the
 * valid rows are compacted on the device and only they go through the three
 * GEMMs; their dH rows are written as +0.
 *
 * Sizes: 0 <= N < 2^28, 0 < V < 2^31, 0 < H <= 2^20 (FLDCE_ERR_BAD_SHAPE
 * otherwise, and the workspace queries return 0); the same range holds for
 * every entry point below (V_local in place of V for the shard calls).
 * bf16 requires H % 64 == 0 and V < 2^23 (FLDCE_ERR_UNSUPPORTED otherwise;
 * the same bound applies to V_local below); all pointers must be 16-byte
 * aligned.  bf16 chunks hold at most 2^22 rows (a larger chunk_rows is
 * lowered to it).
 */
int fldce_fwd_bwd(const void* h, const void* W, const int64_t* target,
                  const float* p_mask, int64_t N, int64_t H, int64_t V,
                  int dtype, int64_t ignore_index, float label_smoothing,
                  float logit_scale, int reduction, int64_t total,
                  float* loss, void* dH, void* dW, float* row_lse,
                  float* row_loss, int64_t chunk_rows, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * fldce_fwd_bwd with the rest of page 1's interface: the optional bias of
 * fused_linear_cross_entropy_forward (F.linear(x, weight, bias)) and its
 * gradient db, and the end-of-block weight of the module's forward
 * (FusedLinearDiffusionCrossEntropyLoss.forward).
 *
 *   bias         [V]   dtype       optional (NULL = none): the logits become
 *                                  z = s (h W^T + b)
 *   db           [V]   dtype       optional out (NULL = not computed):
 *                                  sum_i g_i, float32 accumulation over the
 *                                  rows in a fixed order, rounded once;
 *                                  allowed without a bias
 *   eob_token_id     rows whose target equals it get their loss and
 *                    gradient multiplied by eob_weight (the page divides
 *                    their p_mask by the weight); < 0 = no such weighting
 *   eob_weight       finite and >= 0 (checked only when eob_token_id >= 0)
 *   dH, dW           may be NULL here (not in fldce_fwd_bwd): that gradient
 *                    is not computed and its GEMM is skipped (for instance
 *                    a frozen LM-head weight); with dH, dW and db all NULL
 *                    only the loss (and row statistics) is computed
 *
 * Every other argument is as in fldce_fwd_bwd, which equals this call with
 * bias = db = NULL and eob_token_id = -1; whatever is computed is bit for
 * bit what the full call computes.  Workspace: fldce_workspace_size.
 */
int fldce_fwd_bwd_ex(const void* h, const void* W, const void* bias,
                     const int64_t* target, const float* p_mask, int64_t N,
                     int64_t H, int64_t V, int dtype, int64_t ignore_index,
                     float label_smoothing, float logit_scale, int reduction,
                     int64_t total, int64_t eob_token_id, float eob_weight,
                     float* loss, void* dH, void* dW, void* db,
                     float* row_lse, float* row_loss, int64_t chunk_rows,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace fldce_fwd needs. */
size_t fldce_fwd_workspace_size(int64_t N, int64_t H, int64_t V, int dtype);

/*
 * Forward only (evaluation): the loss and optionally the per-row lse and
 * loss, no gradient -- the forward half of page 1's chunk loop (F.linear,
 * logsumexp_fwd and the loss part of cross_entropy_kernel).  The [N, V]
 * logits are never written to memory on the bf16 path, which also skips
 * rows whose target is ignore_index (their row_lse and row_loss are 0).
 * Arguments as in fldce_fwd_bwd_ex.
 */
int fldce_fwd(const void* h, const void* W, const void* bias,
              const int64_t* target, const float* p_mask, int64_t N, int64_t H,
              int64_t V, int dtype, int64_t ignore_index,
              float label_smoothing, float logit_scale, int reduction,
              int64_t total, int64_t eob_token_id, float eob_weight,
              float* loss, float* row_lse, float* row_loss, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * fldce_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument; the call uses a device array inside the library of
 * FLDCE_NOALLOC_SCRATCH_BYTES, which each device holds from the library's
 * load until the process ends.  It calls no allocating routine.
 *
 * Arguments, results and errors as in fldce_fwd (the same kernels; results
 * are bit for bit those of fldce_fwd), except:
 *   - FLDCE_ERR_SCRATCH_TOO_SMALL, before anything is enqueued, when
 *     fldce_fwd_workspace_size(N, H, V, dtype) > FLDCE_NOALLOC_SCRATCH_BYTES
 *     (bf16 at H = 2560, V = 151936: N <= 3378 rows);
 *   - the array is looked up on the calling thread's current device, which
 *     must be the device of `stream` and of every pointer;
 *   - every call on one device shares that device's array: calls that
 *     overlap in time on one device (other streams, other threads) race and
 *     give undefined results; calls one after another on a stream are fine
 *     (nothing in the array has to start at any value).
 */
int fldce_fwd_noalloc(const void* h, const void* W, const void* bias,
                      const int64_t* target, const float* p_mask, int64_t N,
                      int64_t H, int64_t V, int dtype, int64_t ignore_index,
                      float label_smoothing, float logit_scale, int reduction,
                      int64_t total, int64_t eob_token_id, float eob_weight,
                      float* loss, float* row_lse, float* row_loss,
                      void* stream);

/*
 * Upstream-gradient scaling (page 1, fused_linear_cross_entropy_backward):
 * the gradients above are for d(loss) = 1; a caller that receives the
 * upstream gradient `do` later multiplies them by it, in place.  *grad_out
 * is read on the device (no host sync): when it equals 1 the kernels return
 * without touching the gradients (the page skips the multiply too),
 * otherwise every element becomes dtype(float(x) * do), rounded to nearest
 * even for bf16.
 *
 *   grad_out     [1]   float32     do, device memory
 *   dH, dW, db         dtype       n_dH, n_dW, n_db elements each, scaled in
 *                                  place; a NULL pointer (with n = 0) is
 *                                  skipped
 *
 * Pointers must be 16-byte aligned; counts >= 0.
 */
int fldce_scale_grads(const float* grad_out, int dtype, void* dH, int64_t n_dH,
                      void* dW, int64_t n_dW, void* db, int64_t n_db,
                      void* stream);

/* Bytes of workspace fldce_shard_partials needs. */
size_t fldce_shard_partials_workspace_size(int64_t N, int64_t H,
                                           int64_t V_local, int dtype);

/*
 * Per-row softmax partials of one vocabulary shard W_local = rows
 * [vocab_start, vocab_start + V_local) of the full weight (tutorial page,
 * section 4: each shard sums exp of its own logits; the per-shard maximum is
 * kept alongside, as in page 1's two-stage logsumexp).  The [N, V_local]
 * logits are never written to memory.
 *
 *   row_max      [N] float32 out   m_i = max_{j in shard} z_ij
 *   row_sumexp   [N] float32 out   S_i = sum_{j in shard} exp(z_ij - m_i)
 *   target_logit [N] float32 out   z_{i,y_i} if y_i is in the shard and the
 *                                  row is not ignored, else 0
 *   row_sumlogit [N] float32 out   sum_{j in shard} z_ij (NULL ok: skipped;
 *                                  only needed when label_smoothing > 0)
 *
 * Combining over shards: M = max_k m_k, lse = M + log sum_k S_k e^{m_k - M},
 * z_target = sum_k target_logit_k, sum_j z_ij = sum_k row_sumlogit_k.
 *
 * Rows whose target is ignore_index are skipped (a training step needs no
 * softmax for them): for them row_max = -INFINITY and row_sumexp =
 * target_logit = row_sumlogit = 0, the identity of the combine.  A caller
 * that needs every row's partials (evaluation: every row's lse) passes an
 * ignore_index that no target equals (e.g. INT64_MIN): then every row is
 * computed, and a row whose target lies outside [0, V) of every shard (such
 * as -100) simply has target_logit = 0 in each shard.
 */
int fldce_shard_partials(const void* h, const void* W_local,
                         const int64_t* target, int64_t N, int64_t H,
                         int64_t V_local, int64_t vocab_start, int dtype,
                         int64_t ignore_index, float logit_scale,
                         float* row_max, float* row_sumexp,
                         float* target_logit, float* row_sumlogit,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* Bytes of workspace fldce_shard_bwd needs (chunk_rows 0 = default). */
size_t fldce_shard_bwd_workspace_size(int64_t N, int64_t H, int64_t V_local,
                                      int dtype, int64_t chunk_rows);

/*
 * Gradient slices of one vocabulary shard given every row's GLOBAL lse
 * (combined from all shards' partials).  eps/V uses V_global; the target
 * entry is corrected only when y_i falls inside the shard.
 *
 *   lse          [N]         float32 in   global row logsumexp
 *   total        as fldce_fwd_bwd (the count, when done on the device, is
 *                over all N rows, which every shard sees)
 *   dH_partial   [N,H]       float32 out  g[:, shard] W_local; the sum over
 *                                         shards is dH (tutorial page,
 *                                         section 1.1: row-split product
 *                                         summed across devices)
 *   dW_local     [V_local,H] dtype out    g[:, shard]^T h (complete)
 */
int fldce_shard_bwd(const void* h, const void* W_local, const int64_t* target,
                    const float* p_mask, const float* lse, int64_t N,
                    int64_t H, int64_t V_local, int64_t vocab_start,
                    int64_t V_global, int dtype, int64_t ignore_index,
                    float label_smoothing, float logit_scale, int reduction,
                    int64_t total, float* dH_partial, void* dW_local,
                    int64_t chunk_rows, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Stage profiling (diagnostics).  While enabled, every call above records a
 * pair of HIP events on its own stream around each stage, so stage times are
 * those of the launches on the caller's stream.  fldce_profile_begin()
 * enables recording and clears the totals; fldce_profile_end() disables it.
 * fldce_profile_read() sums the elapsed times of the stage's launches since
 * begin; call it after the stream has been synchronised.  Creating the event
 * pool is the only resource the library ever creates itself, and only while
 * profiling.  Not thread-safe: profile one thread at a time.
 *
 * Stages: 0 prep (divisor, W^T, column sums, target/row-sum dots),
 * 1 h^T, 2 logits GEMM (+ softmax partials), 3 row combine, 4 dlogits,
 * 5 dH GEMM, 6 dH split-K reduction, 7 dW GEMM, 8 loss reduction,
 * 9 flagged rows (redone relative to their lse), 10 db, 11 dH and dW GEMMs
 * in one launch (bf16 with several row chunks).
 */
int fldce_profile_num_stages(void);
const char* fldce_profile_stage_name(int stage);
int fldce_profile_begin(void);
int fldce_profile_end(void);
/* total_ms: summed duration; launches: number of timed launches (either may
 * be NULL).  Returns FLDCE_OK, FLDCE_ERR_BAD_ARGUMENT for a bad stage, or
 * FLDCE_ERR_HIP if an event query fails (stream not synchronised). */
int fldce_profile_read(int stage, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* FLDCE_H */
