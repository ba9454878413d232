/*
 * libpop: POP (Partition-guided Online Pruning) channel-pruned gated-MLP path
 * for AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes.
 *
 * The method (cited by page title and section):
 *   "POP: Online Structural Pruning Enables Efficient Inference of Large
 *   Foundation Models" (paper notes), "Key design 1": during prefill, every
 *   intermediate channel i of the FFN gets an importance from the whole prompt,
 *   I_i = || W_up[i,:] * s ||_2 with s_k = || X[:,:,k] ||_2, and the channels are
 *   split by the quantile thresholds q_{r-delta} and q_{r+delta} into Retained
 *   (R), Candidate (C) and Pruned (P) regions.  "Key design 2": in every decode
 *   step the input goes through W_gate / W_up restricted to R u C, the
 *   candidates are scored and the best k of them top R up to the live count that
 *   r requires, and W_down is applied to R plus the selected candidates.
 *   The gated MLP itself is equation (1) of "Batch-wise adaptive pruning ... for
 *   language reasoning models", section 3.1: z = SiLU(W_g x) * (W_1 x),
 *   y = W_2 z.
 *
 * Readings taken where the pages leave a step open:
 *   - delta = gamma; cut ranks c = round(p * d_ff) with p clamped to [0, 1]
 *     and round half away from zero; live = round((1 - r) * d_ff);
 *     k = clamp(live - |R|, 0, |C|).
 *   - one total order for every selection: a larger value is more important;
 *     on equal values the lower index is more important.
 *   - decode candidate score = max over the batch rows of |SiLU(g_i) * u_i|
 *     (a batch shares one mask).
 *   - no biases.
 *
 * Conventions shared by every entry point:
 *   - Every call returns pop_status.  Arguments are validated before anything is
 *     enqueued; on an error nothing is enqueued, outputs are untouched and
 *     pop_last_error() holds a message for this thread.
 *   - POP_OK means the work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream).  The host never waits for the device and never reads device
 *     memory, so every call may be captured in a HIP graph.
 *   - The caller allocates and owns every buffer: inputs, outputs and the
 *     workspace.  The library keeps no pointer after it returns.  Its only
 *     host-side state is per thread (the last error message and the trace
 *     events of pop_set_trace_events) or a per-device cache of device
 *     attributes (compute units, occupancy); no call's result depends on it.
 *     Calls on different streams need distinct workspaces.
 *   - A workspace starts zero-filled (the first call on it must see zeros).
 *     Decode workspaces carry control words between calls: every call that
 *     completes leaves them zero again, so a workspace stays valid for any
 *     later call, of any shape, ordered after it on one stream.
 *   - Device buffers are contiguous, row-major and 16-byte aligned.
 *     dtype POP_BF16 needs d % 8 == 0, POP_F32 needs d % 4 == 0.
 *   - Index lists (R, C) are int32, strictly ascending, in [0, d_ff) and
 *     mutually disjoint (unchecked in release builds).
 *   - Outputs are fp32 whatever the input dtype; accumulation is fp32.
 */
#ifndef POP_H_
#define POP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  POP_OK = 0,
  POP_ERR_INVALID_ARGUMENT = 1,   /* r, gamma out of range; null pointer; count mismatch */
  POP_ERR_UNSUPPORTED_DTYPE = 2,
  POP_ERR_BAD_SHAPE = 3,          /* sizes negative, too large, or d not a vector multiple */
  POP_ERR_MISALIGNED = 4,         /* a device pointer not 16-byte aligned */
  POP_ERR_WORKSPACE_TOO_SMALL = 5,
  POP_ERR_HIP = 6                 /* a HIP launch failed; see pop_last_error() */
} pop_status;

typedef enum { POP_F32 = 0, POP_BF16 = 1 } pop_dtype;

/* Region sizes of one partition and the per-step top-k count. */
typedef struct {
  int32_t d_ff;
  int32_t c_low;   /* cut rank at r - delta: |P| */
  int32_t c_high;  /* cut rank at r + delta: |P| + |C| */
  int32_t n_P, n_C, n_R;
  int32_t n_live;  /* round((1 - r) * d_ff) */
  int32_t k;       /* candidates selected per decode step; n_R + k == n_live when feasible */
} pop_counts;

/* Largest d_ff a single partition or a single decode call accepts. */
#define POP_MAX_D_FF 32768
/* Largest d (model width) accepted. */
#define POP_MAX_D 16384
/* Largest decode batch that shares one mask. */
#define POP_MAX_BATCH 256
/* Largest prompt routed by one MoE call, and the expert count range. */
#define POP_MAX_MOE_TOKENS (1 << 22)
#define POP_MAX_EXPERTS 64

/* Human-readable name of a status code (static storage). */
const char* pop_status_string(pop_status s);
/* Detail of the last error raised on the calling thread ("" if none). */
const char* pop_last_error(void);

/*
 * pop_partition_counts — pure host function, no device work.
 * The sizes of P, C, R and the top-k count for d_ff channels at pruning rate
 * r and partition width gamma (POP notes, "Key design 1" thresholds
 * q_{r-delta}, q_{r+delta}; "Key design 2" exact live count).
 * Requires 1 <= d_ff <= POP_MAX_D_FF, 0 <= r < 1, 0 <= gamma < 1.
 */
pop_status pop_partition_counts(int32_t d_ff, double r, double gamma, pop_counts* out);

/*
 * pop_decode_topk_count — pure host function, no device work.
 * *k = the number of candidates one decode step selects for an existing
 * partition (n_R retained, n_C candidates) at pruning rate r: k =
 * clamp(round((1 - r) d_ff) - n_R, 0, n_C), so that n_R + k is the live count
 * exactly whenever the partition allows it (POP notes, "Key design 2").  The
 * size of pop_decode_ffn's `selected` output.
 * Errors: BAD_SHAPE for d_ff outside [1, POP_MAX_D_FF]; INVALID_ARGUMENT for
 * r outside [0, 1), negative counts, n_R + n_C > d_ff or k == NULL.
 */
pop_status pop_decode_topk_count(int32_t d_ff, double r, int32_t n_R, int32_t n_C, int32_t* k);

/*
 * pop_check_lists — pure host function, no device work: a debug aid.
 * Checks host copies of a partition's index lists against what every entry
 * point taking R, C (or P) assumes: counts >= 0 with n_R + n_C + n_P <= d_ff;
 * each list strictly ascending within [0, d_ff); no channel in two lists.
 * The device code does not check these (it clamps channel ids into [0, d_ff),
 * so a bad list gives wrong results, not a fault).  A library built with
 * POP_DEBUG defined (libpop_debug.so) runs this check on copies of R and C
 * inside pop_decode_ffn (and so pop_decode_ffn_noalloc), pop_decode_gateup,
 * pop_decode_ffn_periodic and pop_layer_decode before anything is enqueued:
 * a device-to-host copy on the call's stream, waited for, and a host
 * allocation, so such a build can not be captured into a graph.
 *   R, C, P    host int32 arrays (each may be NULL when its count is 0).
 * Errors: BAD_SHAPE for d_ff outside [1, POP_MAX_D_FF]; INVALID_ARGUMENT for
 * negative counts, counts summing past d_ff, a NULL list with a nonzero
 * count, or the first violation found (pop_last_error() names the list, the
 * position and the value).
 */
pop_status pop_check_lists(const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C, const int32_t* P,
                           int32_t n_P, int32_t d_ff);

/* Workspace bytes pop_prefill_partition needs for these sizes. */
size_t pop_prefill_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff);

/*
 * pop_prefill_partition — POP notes, "Key design 1".
 *   X          device, [n_tokens, d] in dt: the FFN inputs of every prompt token
 *              of every sequence (B*L rows; n_tokens may be 0).
 *   W_up       device, [d_ff, d] in dt (nn.Linear layout: row i = channel i).
 *   r, gamma   pruning rate and partition width (delta = gamma).
 *   R, C, P    device int32 outputs of n_R, n_C, n_P entries (sizes from
 *              pop_partition_counts), each written in ascending order.
 *   importance optional device fp32 [d_ff]: I_i (NULL to skip).
 *   ws         device workspace of at least pop_prefill_workspace_bytes().
 * Kernels: column sums of squares of X (one pass per column slice, or
 * partial sums and their fixed-order reduction for long prompts); the weighted
 * sums of squares of W_up over pieces of each row, in equal shares per wave;
 * one workgroup that adds each row's pieces in a fixed order, takes I and
 * splits the rows (histogram select of the two cut keys, ordered compaction).
 * Deterministic: identical inputs give bit-identical outputs.
 */
pop_status pop_prefill_partition(const void* X, int64_t n_tokens, int32_t d, const void* W_up,
                                  int32_t d_ff, pop_dtype dt, double r, double gamma, int32_t* R,
                                  int32_t* C, int32_t* P, float* importance, void* ws,
                                  size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Stages of pop_prefill_partition, callable on their own.
 * ------------------------------------------------------------------------- */

/* Workspace bytes pop_prefill_importance needs (the same as
 * pop_prefill_workspace_bytes). */
size_t pop_prefill_importance_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff);

/*
 * pop_prefill_importance — POP notes, "Key design 1", importance equation
 * (read with row i of W_up; the Wanda-style |W| * ||X||_2 metric named in
 * "Loss / training strategy").
 *   importance  device fp32 [d_ff] output: I_i = sqrt(sum_k W_up[i,k]^2 s_k^2),
 *               s_k^2 = sum over the n_tokens rows of X[:,k]^2.
 * Other arguments as for pop_prefill_partition.
 */
pop_status pop_prefill_importance(const void* X, int64_t n_tokens, int32_t d, const void* W_up,
                                  int32_t d_ff, pop_dtype dt, float* importance, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * pop_partition_select — POP notes, "Key design 1", three-region split.
 * Splits d_ff channels by their importance (device fp32 [d_ff], values >= 0)
 * at the cut ranks of pop_partition_counts: P = the c_low least important,
 * C = the next n_C, R = the rest (larger value more important; on equal values
 * the lower index more important).  R, C, P: device int32, ascending.
 * One workgroup; needs no workspace.
 */
pop_status pop_partition_select(const float* importance, int32_t d_ff, double r, double gamma,
                                int32_t* R, int32_t* C, int32_t* P, void* stream);

/* Workspace bytes pop_decode_ffn / pop_dense_ffn_decode need. */
size_t pop_decode_workspace_bytes(int32_t batch, int32_t d, int32_t d_ff);

/* Byte offset of z in a decode workspace.  The bytes before it are control
 * and hand-over words of the single-launch batch-1 step, zero between calls;
 * the 32-bit word at offset 0 is a sticky error code: nonzero after a batch-1
 * step whose bounded in-kernel wait ran out (that step's y is then not
 * valid).  The library never clears it. */
#define POP_DECODE_WS_Z_OFFSET 70656

/*
 * pop_decode_ffn — POP notes, "Key design 2" and "Overall framework".
 *   x          device, [batch, d] in dt: this step's FFN inputs; the batch
 *              rows share one mask (0 <= batch <= POP_MAX_BATCH).
 *   W_gate     device, [d_ff, d] in dt.
 *   W_up       device, [d_ff, d] in dt.
 *   W_downT    device, [d_ff, d] in dt: the TRANSPOSE of the nn.Linear down
 *              weight [d, d_ff], so channel i's down column is a contiguous row.
 *   R, n_R     device int32 retained channels (ascending).
 *   C, n_C     device int32 candidate channels (ascending).
 *   r          pruning rate; k = clamp(round((1 - r) d_ff) - n_R, 0, n_C).
 *   y          device fp32 [batch, d] output.
 *   selected   optional device int32 [k]: the selected candidates, ascending.
 *   ws         device workspace >= pop_decode_workspace_bytes(batch, d, d_ff),
 *              zero-filled before its first use.  After the call completes,
 *              byte offset POP_DECODE_WS_Z_OFFSET holds the intermediate z
 *              (fp32 [batch, n_R + n_C], R columns first, then C) and byte
 *              offset POP_DECODE_WS_Z_OFFSET + align_up(4 * batch * d_ff + 16,
 *              256) the candidate scores (fp32 [n_C]).
 * Kernels at batch 1 with a candidate top-k (n_C >= 1, k >= 1, n_C <= 4096,
 * d <= 2048 vectors of 16 bytes): two launches.  In the first (512-thread
 * workgroups, at most one per CU), workgroup 0 is the candidate top-k and
 * every other workgroup (a worker) streams an even share of the candidates'
 * gate/up rows (handing each |z| to the top-k through a valid-tagged word),
 * then of the retained channels' gate, up and W_downT rows (z and its down
 * contribution in one pass); the top-k publishes the cut, then the selected
 * candidates as valid-tagged (channel, z) words, and each worker adds the
 * W_downT rows of an equal share of them by rank (their loads issued with its
 * last retained rows when its share is in by then, else after its rows), then
 * stores its partial y.  The second adds the partials in a fixed order into y and clears
 * the hand-over words.  The grid never exceeds what the device holds at once
 * and every in-kernel wait is bounded (see POP_DECODE_WS_Z_OFFSET for the
 * error word).  Batch 1 without a top-k (no candidates, k = 0): the retained
 * rows' gate, up and W_downT rows in one stream, then the fixed-order sum.
 * Other batch-1 shapes: three launches (candidate rows; the one-workgroup
 * top-k beside the retained stream; the selected rows and the sum).
 * Batches 2-64 in bf16: the matrix-core kernels (16-token tiles): gate/up
 * over R u C with fused SiLU*up and the batch-max score; the down-projection
 * over the retained rows with the candidate top-k as one of its workgroups;
 * the down-projection over the selected rows; a fixed-order sum.  fp32 and
 * wider batches: gate/up GEMV, one-workgroup radix top-k, gathered
 * down-projection, fixed-order sum.  Deterministic (the same bits on every
 * call with the same inputs).
 */
pop_status pop_decode_ffn(const void* x, int32_t batch, int32_t d, const void* W_gate,
                          const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                          const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C,
                          double r, float* y, int32_t* selected, void* ws, size_t ws_bytes,
                          void* stream);

/* Workspace bytes of pop_decode_ffn_periodic (independent of r and the lists). */
size_t pop_decode_periodic_workspace_bytes(int32_t batch, int32_t d, int32_t d_ff);

/* Bytes of the device array pop_decode_ffn_noalloc uses as its workspace. */
#define POP_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * pop_decode_ffn_noalloc — pop_decode_ffn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same step, inputs, outputs and result, with the
 * workspace taken from a library-owned device array of
 * POP_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU instead of a caller buffer.  The
 * call allocates nothing.  The array is held by each GPU the library runs on
 * until the process ends; its address is looked up, and its control words
 * cleared (a kernel on `stream`), at the first call on each device.  Every
 * call on one GPU shares that GPU's array and finds the last call's contents:
 * calls that overlap on one GPU (different streams, or graphs replayed
 * concurrently) race and give wrong results; order them.  The sticky error
 * word of POP_DECODE_WS_Z_OFFSET lives in the array too.
 * Errors: as pop_decode_ffn, plus WORKSPACE_TOO_SMALL when
 * pop_decode_workspace_bytes(batch, d, d_ff) exceeds POP_NOALLOC_SCRATCH_BYTES
 * (nothing is enqueued), and HIP_ERROR when the array cannot be found.
 */
pop_status pop_decode_ffn_noalloc(const void* x, int32_t batch, int32_t d, const void* W_gate,
                                  const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                  const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C, double r,
                                  float* y, int32_t* selected, void* stream);

/*
 * pop_decode_ffn_periodic — an alternative decode mode: the candidate
 * selection refreshed only every `period` steps, with an activation memory
 * ("Batch-wise adaptive pruning ... for language reasoning models", figure 1
 * and figure 2(b); its definition is cut off in the pages and is read into
 * POP's candidate set).  Step `step` (0-based) refreshes when
 * step % period == 0: gate/up over R u C, each candidate's score (max over
 * the batch of |z|) is added to memory[position], the k candidates of highest
 * memory (ties: lower position) become the selection, written to
 * positions [k] (into C, ascending) and selected [k] (channels), and memory is
 * cleared; rows [n_R + k] receives R followed by the selection.  Any other
 * step computes the retained rows `rows` (those of the last refresh) with no
 * candidates, and adds the selected candidates' scores to their memory at
 * `positions`.  y [batch, d] fp32 as pop_decode_ffn.  memory [n_C] fp32 is
 * caller-owned state (zero before the first step); positions, selected and
 * rows are state too.  k, x, weights and lists as pop_decode_ffn;
 * period >= 1, step >= 0.  ws: at least
 * pop_decode_periodic_workspace_bytes(batch, d, d_ff) bytes, 16-byte aligned.
 * Kernels at batch 1 (when pop_decode_ffn's single launch applies): a
 * refresh is that launch with each candidate ranked by memory + |z| (the
 * workers clear the memory they read), then one small launch writing rows; a
 * kept step is the retained-row stream whose last launch also updates the
 * memory.  Other batches compose the stage entry points.
 * Errors as pop_decode_ffn and INVALID_ARGUMENT for period < 1 or step < 0.
 * Calls that share memory or ws must be ordered on one stream.
 */
pop_status pop_decode_ffn_periodic(const void* x, int32_t batch, int32_t d, const void* W_gate,
                                   const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                   const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C, double r,
                                   int32_t step, int32_t period, float* memory, int32_t* positions,
                                   int32_t* selected, int32_t* rows, float* y, void* ws, size_t ws_bytes,
                                   void* stream);

/* ---------------------------------------------------------------------------
 * Stages of pop_decode_ffn, callable on their own (also the building blocks of
 * the static-mask and full re-evaluation variants of the POP notes' ablation
 * table).
 * ------------------------------------------------------------------------- */

/*
 * pop_decode_gateup — POP notes, "Key design 2": H_t = f(X_t; R u C), with f the
 * gated MLP's first half (equation (1) of the batch-wise pruning page):
 * z[b, p] = SiLU(W_gate[ch_p] . x_b) * (W_up[ch_p] . x_b) for the positions
 * p < n_R + n_C, where ch_p = R[p] for p < n_R and C[p - n_R] after.
 *   R == NULL means R = 0, 1, ..., n_R - 1 (then n_C must be 0): the dense
 *   first half over all channels when n_R == d_ff.
 *   z      device fp32 [batch, n_R + n_C] output.
 *   score  optional device fp32 [n_C] output: max over b of |z[b, n_R + j]|.
 */
pop_status pop_decode_gateup(const void* x, int32_t batch, int32_t d, const void* W_gate,
                             const void* W_up, int32_t d_ff, pop_dtype dt, const int32_t* R,
                             int32_t n_R, const int32_t* C, int32_t n_C, float* z, float* score,
                             void* stream);

/*
 * pop_decode_select — POP notes, "Key design 2": the candidates sorted by their
 * step score, highest first (equal scores: lower position first), and the first
 * k kept.
 *   score      device fp32 [n_C], values >= 0.
 *   C          device int32 [n_C]: the candidate channels.
 *   positions  device int32 [k] output: the kept positions into C, ascending.
 *   selected   device int32 [k] output: C[positions[j]].
 * One workgroup; 0 <= k <= n_C <= POP_MAX_D_FF.
 */
pop_status pop_decode_select(const float* score, int32_t n_C, const int32_t* C, int32_t k,
                             int32_t* positions, int32_t* selected, void* stream);

/* Workspace bytes pop_decode_down needs for n_live = n_R + k rows. */
size_t pop_decode_down_workspace_bytes(int32_t batch, int32_t d, int32_t n_live);

/*
 * pop_decode_down — POP notes, "Overall framework": the FFN finished on R plus
 * the selected candidates: y[b, :] = sum over live rows of z[b, col] * W_downT[ch, :]
 * with (ch, col) = (R[q], q) for q < n_R and (selected[j], n_R + positions[j])
 * for j < k (the pop_decode_select outputs).  R == NULL means R = 0, ...,
 * n_R - 1 (valid with k == 0).
 *   z   device fp32 [batch, n_A] (the pop_decode_gateup output, n_A columns).
 *   y   device fp32 [batch, d] output.
 * The partial sums of row chunks are reduced in a fixed order: deterministic.
 */
pop_status pop_decode_down(const float* z, int32_t batch, int32_t n_A, const void* W_downT,
                           int32_t d, int32_t d_ff, pop_dtype dt, const int32_t* R, int32_t n_R,
                           const int32_t* selected, const int32_t* positions, int32_t k, float* y,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * pop_dense_ffn_decode — the unpruned gated MLP (equation (1) of the
 * batch-wise pruning page, section 3.1) for one decode step over all d_ff
 * channels: the dense baseline the pruned step is compared with.  Same
 * layouts and workspace as pop_decode_ffn; after the call, byte offset
 * POP_DECODE_WS_Z_OFFSET of the workspace holds z (fp32 [batch, d_ff]).
 */
pop_status pop_dense_ffn_decode(const void* x, int32_t batch, int32_t d, const void* W_gate,
                                const void* W_up, const void* W_downT, int32_t d_ff,
                                pop_dtype dt, float* y, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Dense prompt FFN (the prefill forward).
 * ------------------------------------------------------------------------- */

/* Workspace bytes of pop_dense_ffn_prefill (0 for invalid arguments). */
size_t pop_dense_ffn_prefill_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff, pop_dtype dt);

/*
 * pop_dense_ffn_prefill — the dense gated MLP over every prompt token, the
 * prefill forward whose input the partition is computed from (POP notes,
 * "Loss / training strategy": the online masking starts from the second step,
 * so the prompt itself runs through all d_ff channels).  Gated MLP of
 * equation (1), section 3.1 of the batch-wise pruning page:
 *   Z = SiLU(X W_gate^T) * (X W_up^T),   Y = Z W_down^T = Z W_downT.
 *
 *   X        [n_tokens, d] row-major, dtype dt
 *   W_gate, W_up, W_downT   [d_ff, d] row-major, dtype dt (W_downT is the
 *            transpose of the nn.Linear weight W_down [d, d_ff])
 *   Y        [n_tokens, d] fp32, written
 *   ws       pop_dense_ffn_prefill_workspace_bytes(n_tokens, d, d_ff, dt)
 *            bytes; holds Z for up to 4096 tokens at a time (the call works
 *            through the prompt in passes of 4096 tokens).
 * POP_BF16 multiplies on the matrix cores (bf16 x bf16, fp32 accumulation) and
 * keeps Z in bf16 (round to nearest even); POP_F32 computes in fp32 FMA.
 * n_tokens = 0 enqueues nothing.  Errors: BAD_SHAPE (d, d_ff or n_tokens out
 * of range, d not a multiple of the vector width), INVALID_ARGUMENT (NULL
 * buffers), MISALIGNED, WORKSPACE_TOO_SMALL, HIP (launch failure).
 */
pop_status pop_dense_ffn_prefill(const void* X, int64_t n_tokens, int32_t d, const void* W_gate,
                                 const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                 float* Y, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of pop_prefill_ffn_partition (0 for invalid arguments). */
size_t pop_prefill_ffn_partition_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff, pop_dtype dt);

/*
 * pop_prefill_ffn_partition — the whole prefill of one FFN layer in one call:
 * the dense prompt FFN (as pop_dense_ffn_prefill) and the three-region
 * partition of POP notes, "Key design 1" (as pop_prefill_partition), with the
 * importance I_i = || W_up[i, :] * s ||_2 computed inside the gate/up pass from
 * the W_up tiles it already reads, so W_up is swept once instead of twice.
 * The column norms s (over all n_tokens rows of X) are computed first.
 *
 *   X, W_gate, W_up, W_downT, Y   as for pop_dense_ffn_prefill
 *   r, gamma, R, C, P             as for pop_prefill_partition
 *   importance  optional device fp32 [d_ff] output (NULL: kept in ws)
 *   ws          pop_prefill_ffn_partition_workspace_bytes(n_tokens, d, d_ff, dt)
 * The sums behind I run in another order than pop_prefill_importance's, so
 * the two I agree to fp32 rounding, and the partitions agree except where a
 * channel's I lies within that rounding of a cut.  n_tokens = 0: Y is not
 * touched, I = 0 and the partition goes by index.  Errors: as for the two
 * calls it combines.
 */
pop_status pop_prefill_ffn_partition(const void* X, int64_t n_tokens, int32_t d, const void* W_gate,
                                     const void* W_up, const void* W_downT, int32_t d_ff, pop_dtype dt,
                                     double r, double gamma, float* Y, int32_t* R, int32_t* C, int32_t* P,
                                     float* importance, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Mixture of experts.
 *
 * The POP notes ("Key experimental data") apply the method to MoE models; the
 * pages give no routing detail.  Readings taken: a token goes to the experts
 * of its two largest router logits (on equal logits the lower expert id
 * first), weighted by the softmax of those two logits; every expert keeps its
 * own R/C/P partition, built from the prompt tokens routed to it; in a decode
 * step every expert runs the POP step on the tokens routed to it (candidate
 * score = max over those tokens), and a token's output is the weighted sum of
 * its two experts' outputs, lower expert id first.  An expert no token reaches
 * does nothing.
 *
 * Expert tensors are stacked: W_gate, W_up, W_downT are [E, d_ff, d] (expert
 * e's [d_ff, d] matrix at offset e * d_ff * d); R, C, P are [E, n_R], [E, n_C],
 * [E, n_P] with the sizes of pop_partition_counts (equal for every expert);
 * router logits are fp32 [n_tokens, E].  2 <= E <= POP_MAX_EXPERTS.
 * ------------------------------------------------------------------------- */

/*
 * pop_moe_route_top2 — the routing alone.  experts [n_tokens, 2] (best expert
 * first), weights [n_tokens, 2] (fp32), offsets [E + 1], tokens [2 n_tokens],
 * slots [n_tokens, 2]: the pairs of expert e are tokens[offsets[e] ..
 * offsets[e + 1]) in ascending token order, and pair (t, experts[t, j]) sits at
 * tokens[slots[t, j]].  0 <= n_tokens <= POP_MAX_MOE_TOKENS.
 */
pop_status pop_moe_route_top2(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t* experts,
                              float* weights, int32_t* offsets, int32_t* tokens, int32_t* slots, void* stream);

size_t pop_moe_prefill_workspace_bytes(int64_t n_tokens, int32_t d, int32_t d_ff, int32_t n_experts);

/*
 * pop_moe_prefill_partition — "Key design 1" per expert: for every expert,
 * s over the prompt tokens routed to it, I = ||W_up[e][i, :] * s||_2, and its
 * R/C/P.  X [n_tokens, d] and W_up [E, d_ff, d] in dtype dt; logits fp32
 * [n_tokens, E]; importance [E, d_ff] (optional).  bf16 supports E <= 32
 * (the per-expert accumulators live in LDS).  Errors as
 * pop_prefill_partition, and BAD_SHAPE for E or n_tokens out of range.
 */
pop_status pop_moe_prefill_partition(const void* X, int64_t n_tokens, int32_t d, const float* logits,
                                     int32_t n_experts, const void* W_up, int32_t d_ff, pop_dtype dt, double r,
                                     double gamma, int32_t* R, int32_t* C, int32_t* P, float* importance,
                                     void* ws, size_t ws_bytes, void* stream);

size_t pop_moe_decode_workspace_bytes(int32_t n_tokens, int32_t d, int32_t d_ff, int32_t n_experts);

/*
 * pop_moe_decode_ffn — one MoE decode step over n_tokens tokens
 * (0 <= n_tokens <= POP_MAX_BATCH): routing, then per expert the POP step of
 * pop_decode_ffn on its routed tokens, then y = the weighted sum (fp32
 * [n_tokens, d], every row written).  selected (optional) is [E, k]: expert
 * e's selected candidates, ascending, written only for experts that received
 * a token.  k = clamp(round((1 - r) d_ff) - n_R, 0, n_C) as for one layer.
 * Deterministic: the same inputs give the same bits.  Errors as
 * pop_decode_ffn, and BAD_SHAPE for E out of range.
 * After the call the workspace holds, each region starting on a 256-byte
 * boundary in this order (P = 2 n_tokens routed pairs): experts [P] int32,
 * weights [P] fp32, offsets [E + 1] int32, tokens [P] int32, slots [P] int32,
 * z fp32 with rows of n_R + n_C values (row p: pair p's z over its expert's R
 * then C; the region is sized for P rows of d_ff), scores fp32 [E][n_C]
 * (region sized for E * d_ff).
 */
pop_status pop_moe_decode_ffn(const void* x, int32_t n_tokens, int32_t d, const float* logits, int32_t n_experts,
                              const void* W_gate, const void* W_up, const void* W_downT, int32_t d_ff,
                              pop_dtype dt, const int32_t* R, int32_t n_R, const int32_t* C, int32_t n_C,
                              double r, float* y, int32_t* selected, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * A whole decoder layer around the pruned FFN.
 *
 * "POP: Online Structural Pruning ..." (paper notes), "Key design 3" and
 * "Limitations": attention keeps every parameter and runs dense; only the FFN
 * is pruned (at the rate the global budget gives it: 20% global is 29.9% of
 * LLaMA-2-7B's FFN).  The layer is the pre-norm LLaMA decoder layer of the
 * model family the notes evaluate:
 *   h   = x + Attn(RMSNorm(x; attn_norm)) Wo_T
 *   out = h + FFN(RMSNorm(h; ffn_norm))
 * with RMSNorm(v) = v / sqrt(mean(v^2) + eps) * gain (Zhang & Sennrich 2019,
 * eq. 4); [q | k | v] = RMSNorm(x) Wqkv_T; q and k turned by the rotary
 * embedding of RoFormer (Su et al. 2021, eqs. 14-15): pair (2i, 2i+1) of each
 * head by the angle pos * theta^(-2i/hd), evaluated in double precision;
 * causal scaled dot-product attention (Vaswani et al. 2017, sec. 3.2.1), scale
 * 1/sqrt(hd), query head h reading key/value head h / (H / H_kv).
 * With POP_BF16 the layer stores bf16 (round to nearest even) where a bf16
 * model stores its values: both RMSNorm outputs, the key/value cache and the
 * attention output.  q, every sum and the residual stream x stay fp32.
 * Key/value caches: device [batch, H_kv, cache_len, hd] in dt each, caller-owned.
 * ------------------------------------------------------------------------- */
typedef struct pop_layer_shape {
  int32_t d;           /* model width D: D % 64 == 0, D <= POP_MAX_D */
  int32_t n_heads;     /* H, 1..1024 */
  int32_t n_kv_heads;  /* H_kv >= 1, dividing H */
  int32_t head_dim;    /* hd: 64 or 128 */
  int32_t d_ff;        /* FFN width, 1..POP_MAX_D_FF */
  int32_t cache_len;   /* positions one sequence's cache holds, 1..2^20 */
  double eps;          /* RMSNorm epsilon, >= 0 */
  double rope_theta;   /* rotary base, > 0 */
} pop_layer_shape;

typedef struct pop_layer_weights {
  const float* attn_norm; /* device fp32 [D]: gain of the attention's RMSNorm */
  const void* Wqkv_T;     /* device [D, (H + 2 H_kv) hd] in dt: the q, k, v column blocks */
  const void* Wo_T;       /* device [H hd, D] in dt */
  const float* ffn_norm;  /* device fp32 [D]: gain of the FFN's RMSNorm */
  const void* W_gate;     /* device [d_ff, D] in dt */
  const void* W_up;       /* device [d_ff, D] in dt */
  const void* W_downT;    /* device [d_ff, D] in dt (transpose of W_down) */
} pop_layer_weights;

/* Workspace bytes of pop_layer_prefill; 0 for an invalid shape. */
size_t pop_layer_prefill_workspace_bytes(int32_t batch, int32_t n_tokens, const pop_layer_shape* s, pop_dtype dt);

/*
 * pop_layer_prefill — the prompt's pass through one layer: dense attention,
 * the dense FFN, and the FFN's partition from its input ("Key design 1"; the
 * prompt runs dense, masking starts at the first decode step).
 *   x          device fp32 [batch, n_tokens, D], updated in place to the
 *              layer's output.  1 <= n_tokens <= cache_len,
 *              batch * n_tokens <= 2^22.
 *   s, w, dt   shape (host struct), weights (host struct of device pointers).
 *   K_cache, V_cache  positions 0 .. n_tokens - 1 of every sequence written.
 *   r, gamma, R, C, P, importance  as pop_prefill_partition, over the FFN
 *              inputs of all batch * n_tokens tokens (one partition).
 *   ws         >= pop_layer_prefill_workspace_bytes; after the call byte 0
 *              holds the FFN's input RMSNorm(h) (dt, [batch * n_tokens, D]).
 * Kernels: RMSNorm; the q|k|v GEMM and the output GEMM on the prompt FFN's
 * matrix-core kernel (bf16) or LDS-tiled FMA (fp32); the rotation and cache
 * write; causal attention, for bf16 on the matrix cores over 64-query x 64-key
 * tiles (q and the softmax weights enter as bf16 hi + lo parts, keeping
 * fp32-level error), for fp32 over 16 x 32 LDS tiles; the fused prompt FFN
 * and partition of pop_prefill_ffn_partition; residual adds.
 * Errors: BAD_SHAPE / UNSUPPORTED_DTYPE / INVALID_ARGUMENT / MISALIGNED /
 * WORKSPACE_TOO_SMALL as the other calls; nothing is enqueued on an error.
 */
pop_status pop_layer_prefill(float* x, int32_t batch, int32_t n_tokens, const pop_layer_shape* s,
                             const pop_layer_weights* w, pop_dtype dt, void* K_cache, void* V_cache, double r,
                             double gamma, int32_t* R, int32_t* C, int32_t* P, float* importance, void* ws,
                             size_t ws_bytes, void* stream);

/* Workspace bytes of pop_layer_decode (1 <= batch <= 64); 0 for an invalid shape. */
size_t pop_layer_decode_workspace_bytes(int32_t batch, const pop_layer_shape* s, pop_dtype dt);

/*
 * pop_layer_decode — one decode step of one layer: dense attention over the
 * cache, then POP's FFN step ("Key design 2") on R u C, or the dense FFN.
 *   x          device fp32 [batch, D] (1 <= batch <= 64): this step's token of
 *              every sequence, updated in place to the layer's output.
 *   pos        device int32 [1]: the token's position (= tokens already in the
 *              cache), read on the device so that a captured graph can be
 *              replayed as it advances.  The call writes cache entry pos and
 *              attends to entries 0 .. pos.  A value outside [0, cache_len)
 *              writes no cache entry and leaves x undefined; no memory outside
 *              the buffers is touched.
 *   R, n_R, C, n_C, r, selected   as pop_decode_ffn (unused with dense_ffn).
 *   dense_ffn  0: POP's step; 1: every FFN channel (pop_dense_ffn_decode).
 *   ws         >= pop_layer_decode_workspace_bytes; after the call byte 0
 *              holds the FFN's input RMSNorm(h) (dt, [batch, D]).
 * Kernels, in three batch regimes:
 *   - batch <= 2: the q|k|v projection as a K-major GEMV (one wave per 512
 *     bf16 or 256 fp32 columns and a chunk of rows, fp32 partial sums) with the
 *     RMSNorm computed inside its waves; the chunk sums with the rotation and
 *     cache write; attention split into 64-key slices; the output projection
 *     GEMV, whose waves merge the slices (log-sum-exp) on the fly;
 *   - batch 3-11, and fp32 at any batch above 2: a separate RMSNorm launch, the
 *     same GEMV projections, and the attention slices merged by a kernel of
 *     their own before a plain output projection;
 *   - bf16 from 12 tokens: both projections on a matrix-core GEMM (16 tokens
 *     as the A operand, 256-column W tiles; each 16-token group streams W
 *     again), split into reduction slices whose partial products the rotation
 *     kernel and the residual kernel add; the workspace grows with the slice
 *     count.
 * Then the residual, the FFN's RMSNorm, and pop_decode_ffn or
 * pop_dense_ffn_decode, whose last kernel adds its output into x at batch 1
 * (a residual add launch above).  Deterministic.  Errors as pop_layer_prefill
 * and pop_decode_ffn; nothing is enqueued on an error.
 */
pop_status pop_layer_decode(float* x, int32_t batch, const pop_layer_shape* s, const pop_layer_weights* w,
                            pop_dtype dt, void* K_cache, void* V_cache, const int32_t* pos, const int32_t* R,
                            int32_t n_R, const int32_t* C, int32_t n_C, double r, int32_t dense_ffn,
                            int32_t* selected, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Kernel tracing (measurement hook).
 * ------------------------------------------------------------------------- */

/*
 * pop_set_trace_events — arms kernel tracing on the calling thread: every
 * later libpop call on this thread records the next unused event of `events`
 * (hipEvent_t handles created by the caller) on its stream before its first
 * kernel and right after each kernel it launches, until n_events are used.
 * pop_set_trace_events(NULL, 0) disarms.  This thread-local list is the only
 * state the library keeps between calls; it is never touched unless armed.
 */
pop_status pop_set_trace_events(void* const* events, int32_t n_events);
/* Events recorded since the last pop_set_trace_events call on this thread. */
int32_t pop_trace_recorded(void);

/*
 * pop_hbm_read_probe — a measurement aid, not part of the path: reads the
 * first bytes / 16 16-byte vectors of src once (device memory, 16-byte
 * aligned), as `blocks` workgroups of 256 threads each streaming one
 * contiguous chunk with non-temporal loads, eight in flight per thread (the
 * decode streams' access pattern), and writes one folded word per thread to
 * sink (device uint32 [blocks * 256]).  Timing it gives the HBM read rate the
 * decode kernels can be held to.  Errors: INVALID_ARGUMENT, MISALIGNED,
 * HIP_ERROR.
 */
pop_status pop_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* POP_H_ */
