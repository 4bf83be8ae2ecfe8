/* dllm.h — C ABI of libdllm.so: the dLLM denoise step (LowConfidence), mixed-state packing and
 * first-done-first-out compaction on AMD Instinct MI355X (gfx950).
 *
 * Citation key (page titles):
 *   [FDFO]       "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」"
 *   [BlockServe] "BlockServe: 块粒度连续批处理实现高吞吐扩散大语言模型服务"
 *   [DiLaServe]  "DiLaServe: High SLO Attainment Serving for Diffusion Language Models"
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers unless stated otherwise; the dllm_reqs / dllm_queue structs
 *     themselves are passed by host pointer and their fields are device pointers.
 *   - Calls are stream-ordered and asynchronous: they enqueue work on `stream` (a hipStream_t;
 *     NULL = the default stream) and never synchronise it.
 *   - Problems the host can see return synchronously as a dllm_status, with text available from
 *     dllm_last_error().  Data-dependent problems found on the device are written to *status,
 *     a device int32: the library only ever stores a nonzero code there (the first one wins), so
 *     the caller zeroes it once and may check it after many calls.
 *   - The caller owns every buffer.  The library allocates nothing and keeps no state besides a
 *     per-device cache of the compute-unit count.
 *   - Calls that share a workspace, request table or queue must not overlap in time.
 */
#ifndef DLLM_H
#define DLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DLLM_OK = 0,
    DLLM_ERR_ARG = 1,       /* null pointer, bad size or id, workspace too small */
    DLLM_ERR_SHAPE = 2,     /* shape outside the supported limits, or a row that does not fit the box */
    DLLM_ERR_DTYPE = 3,     /* unknown logits dtype */
    DLLM_ERR_CAPACITY = 4,  /* a queued request cannot be admitted even into an empty batch; queue too long */
    DLLM_ERR_HIP = 5        /* a HIP call failed (text from dllm_last_error) */
} dllm_status;

/* Logits element types.  Entry points take the value as an int32_t `dtype` (the size of a C enum is
 * the compiler's choice, and any other value must be rejected, not assumed away): anything but these
 * two returns DLLM_ERR_DTYPE, or 0 from dllm_step_workspace_bytes. */
typedef enum { DLLM_FP32 = 0, DLLM_BF16 = 1 } dllm_dtype;

/* Limits (checked synchronously). */
#define DLLM_MAX_L 1024            /* block length */
#define DLLM_MAX_ROWS 4096         /* rows of a box / row capacity */
#define DLLM_MAX_POSITIONS 262144  /* rows * L */
#define DLLM_MAX_QUEUE 8192        /* queue capacity */
#define DLLM_MAX_SHARDS 1024       /* vocabulary shards */

/* Request table, indexed by request id ([BlockServe] §II-A: prompt length p_i, K_i = ceil(g_i/L)
 * blocks, current block index b_i).  All arrays are device memory of length n_req (blk_mask:
 * n_req * L bytes, row-major).  arena holds, for request q starting at arena_off[q], its
 * p[q] prompt tokens followed by K[q] blocks of L tokens (block k at arena_off[q] + p[q] + k*L);
 * blk_mask[q] is the mask of its current block (1 = masked): the half-finished block a request
 * carries between rounds ([FDFO] §工程设计二, dllm_incomplete_ids).  The caller guarantees that
 * every region lies inside the arena's allocation: the table carries no arena length, so the
 * library cannot check it, and a region past the end makes dllm_pack and dllm_compact access
 * memory outside the arena.  Ids, b and state are checked (DLLM_ERR_ARG in *status). */
typedef struct {
    int32_t n_req;
    const int32_t *p;          /* prompt length */
    const int32_t *K;          /* blocks to generate */
    int32_t *b;                /* current block index (updated by dllm_compact) */
    int32_t *state;            /* 0 queued, 1 active, 2 finished (updated by dllm_compact) */
    const float *threshold;    /* per-request confidence threshold ([DiLaServe] §四 4.1) */
    const int64_t *arena_off;  /* start of each request's token region */
    int32_t *arena;            /* token storage */
    uint8_t *blk_mask;         /* [n_req, L] */
} dllm_reqs;

/* Pending queue ([BlockServe] §II-D: kept sorted by prompt length; here ascending (p, id)).
 * ids: device int32 [cap]; the first *len entries are the queued request ids in order.
 * len: device int32.  cap: host value, <= DLLM_MAX_QUEUE.  dllm_compact removes admitted
 * entries and keeps the rest in order. */
typedef struct {
    int32_t *ids;
    int32_t *len;
    int32_t cap;
} dllm_queue;

/* Layout summary written by dllm_compact (device memory, 32 bytes). */
typedef struct {
    int32_t rows;        /* active rows after the call (dense: rows 0 .. rows-1) */
    int32_t W;           /* box width max_i (p_i + (b_i + 1) L), 0 if no rows ([BlockServe] Eq.(1)) */
    int32_t n_evicted;   /* requests finished by this call */
    int32_t n_admitted;  /* requests admitted by this call */
    int32_t n_queued;    /* requests still queued */
    int32_t reserved;
    int64_t cost;        /* rows * W: Cost(A) of [BlockServe] Eq.(1) */
} dllm_meta;

/* dllm_step — one denoise step, LowConfidence rule.
 *
 * Defined by [FDFO] §工程设计一 (step(forward_batch, full_logits, states) -> done_flags; LowConfidence:
 * unmask masked slots whose confidence exceeds the threshold, else at least the single most
 * confident one), [DiLaServe] §三 3.1 (the confidence is the softmax probability; slots below the
 * threshold stay masked), [FDFO] §工程设计二 (accept length 0 = continue, block_size = commit) and
 * [BlockServe] §II-E (left padding puts every row's active block in the last L box columns).
 *
 * For every row r < rows and slot j < L with mask_in[r, j] != 0, with x = logits[r, j, 0:V]:
 *   argmax a = the lowest v with x_v = max x;  conf c = 1 / sum_v exp(x_v - max x)  (float32
 *   arithmetic; c is the softmax probability of token a).
 * Per row: U = {masked j : c_j > threshold[r]}; if U is empty and the row has a masked slot,
 *   U = {the masked j with the largest c_j, lowest j on ties}.  For j in U:
 *   input_ids[r, W - L + j] = a_j.  mask_out[r, j] = mask_in[r, j] && j not in U.
 *   done[r] = no masked slot left; accept_len[r] = done ? L : 0.  A row with no masked slot on
 *   entry is left unchanged and reports done = 1, accept_len = L.
 *
 * logits     : element (r, j, v) at r*row_stride + j*pos_stride + v (strides in elements);
 *              fp32 or bf16; must be finite.  Only masked slots are read.  16-byte aligned rows
 *              (base and both strides) take the vector path; others a slower element path.
 * input_ids  : int32 [rows, W], row-major; only active-block columns of unmasked slots are written.
 * mask_in    : uint8 [rows, L]; mask_out: uint8 [rows, L], every entry written; may be mask_in
 *              itself (in-place update), but must not overlap it otherwise.
 * threshold  : float32 [rows].   p, b: int32 [rows] or both NULL; when given, a row with
 *              p + (b + 1) L > W sets *status = DLLM_ERR_SHAPE (the step still completes).
 * conf, argmax: float32 / int32 [rows, L] outputs, or NULL; -1 where a slot was not scored.
 * done       : uint8 [rows]; accept_len: int32 [rows].
 * workspace  : device scratch of at least dllm_step_workspace_bytes(rows, L, V, dtype) bytes,
 *              16-byte aligned, any contents: it holds per-chunk partial results, each written
 *              before it is read.  Serves calls of any shape that fits.  Not shared by
 *              overlapping calls.
 * status     : device int32 (see conventions).
 * Errors: DLLM_ERR_ARG (null required pointer, rows < 0, V < 1, strides too small, mask_out
 * overlapping mask_in without being it, workspace too small or misaligned), DLLM_ERR_SHAPE (L outside [1, DLLM_MAX_L], W < L,
 * rows > DLLM_MAX_ROWS, rows*L > DLLM_MAX_POSITIONS), DLLM_ERR_DTYPE, DLLM_ERR_HIP.
 * rows == 0 is a no-op returning DLLM_OK.  Work: two kernels on `stream` (scoring, then the
 * per-row decision); the call returns after enqueueing both. */
dllm_status dllm_step(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                      int64_t row_stride, int32_t rows, int32_t L, int32_t V, int32_t *input_ids,
                      int32_t W, const uint8_t *mask_in, uint8_t *mask_out, const float *threshold,
                      const int32_t *p, const int32_t *b, float *conf, int32_t *argmax, uint8_t *done,
                      int32_t *accept_len, void *workspace, size_t workspace_bytes, int32_t *status);

/* dllm_step_timed — dllm_step with its device time measured: start_event takes the start of the
 * scoring kernel and stop_event the end of the deciding kernel (hipEvent_t handles created with
 * timing enabled, owned by the caller), so hipEventElapsedTime gives the step from the first
 * kernel's start to the second's end, without the dispatch latency an event pair recorded around
 * the call also holds.  Outputs, status and errors as for dllm_step, plus DLLM_ERR_ARG for a null
 * event.  With rows == 0 nothing is launched and the events are not recorded. */
dllm_status dllm_step_timed(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                            int64_t row_stride, int32_t rows, int32_t L, int32_t V, int32_t *input_ids,
                            int32_t W, const uint8_t *mask_in, uint8_t *mask_out, const float *threshold,
                            const int32_t *p, const int32_t *b, float *conf, int32_t *argmax, uint8_t *done,
                            int32_t *accept_len, void *workspace, size_t workspace_bytes, int32_t *status,
                            void *start_event, void *stop_event);

/* Bytes of workspace dllm_step (or the pair below) needs for this shape (0 for invalid
 * arguments). */
size_t dllm_step_workspace_bytes(int32_t rows, int32_t L, int32_t V, int32_t dtype);

/* dllm_step_noalloc — dllm_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid hipMalloc.  It takes no workspace
 * and allocates nothing: its per-chunk partials live in a fixed device array of
 * DLLM_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held until the process ends; its
 * address is looked up once per device, on the first call on that device).  Arguments, outputs,
 * status and errors as for dllm_step, plus DLLM_ERR_CAPACITY, before anything is launched, when the
 * shape needs more workspace than that (dllm_step_workspace_bytes(rows, L, V, dtype) >
 * DLLM_NOALLOC_SCRATCH_BYTES: at V = 152064 bf16, rows * L up to 27594 slots fit, so 256 rows of
 * L = 64 do).  The
 * array keeps whatever the last call left; the step writes every partial before reading it, so
 * it needs no clearing.  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (on different streams, or from different host threads without ordering) race
 * and give wrong results.  Results are bit for bit those of dllm_step. */
#define DLLM_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
dllm_status dllm_step_noalloc(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                              int64_t row_stride, int32_t rows, int32_t L, int32_t V, int32_t *input_ids,
                              int32_t W, const uint8_t *mask_in, uint8_t *mask_out, const float *threshold,
                              const int32_t *p, const int32_t *b, float *conf, int32_t *argmax, uint8_t *done,
                              int32_t *accept_len, int32_t *status);

/* dllm_step_score and dllm_step_decide — dllm_step in its two halves, for callers that time,
 * overlap or schedule them apart.  Calling dllm_step_score, then dllm_step_decide on the same
 * stream with the same dtype, rows, L, V, mask_in and workspace, equals one dllm_step call
 * bit for bit.
 *
 * dllm_step_score: for every masked slot (mask_in != 0), reduces its logits row ([DiLaServe] §三
 * 3.1: the confidence is a softmax probability; [FDFO] §工程设计一: only masked slots are
 * predicted) to per-chunk partial results (max, sum of exp(x - max), first index at the max) in
 * the workspace.  Arguments as for dllm_step; writes only the workspace (and *status).
 * dllm_step_decide: merges those partials in a fixed order into conf and argmax and applies the
 * LowConfidence rule, with the outputs and conditions of dllm_step.  It reads no logits.  Two
 * optional per-row outputs (device arrays of `rows` entries, or NULL) report how the rule went,
 * the per-request result of a step ([FDFO] §工程设计二) beside the accept length:
 *   unmasked[r] (int32) = the number of slots the step unmasked in row r;
 *   fallback[r] (uint8) = 1 if row r had masked slots and none exceeded its threshold (so the
 *   single most confident one was unmasked), else 0.
 * Errors: those of dllm_step that concern each half's own arguments. */
dllm_status dllm_step_score(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                            int64_t row_stride, int32_t rows, int32_t L, int32_t V, const uint8_t *mask_in,
                            void *workspace, size_t workspace_bytes, int32_t *status);
/* dllm_step_score_timed — dllm_step_score with its scoring kernel's execution timed: the two
 * events (hipEvent_t handles created with timing enabled, owned by the caller) take the start and
 * the end of that kernel itself, so hipEventElapsedTime gives its duration without the dispatch
 * latency that an event pair recorded around the call also holds.  Partials, status and errors as
 * for dllm_step_score, plus DLLM_ERR_ARG for a null event.  With rows == 0 nothing is launched and
 * the events are not recorded. */
dllm_status dllm_step_score_timed(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                                  int64_t row_stride, int32_t rows, int32_t L, int32_t V,
                                  const uint8_t *mask_in, void *workspace, size_t workspace_bytes,
                                  int32_t *status, void *start_event, void *stop_event);
dllm_status dllm_step_decide(void *stream, int32_t dtype, int32_t rows, int32_t L, int32_t V,
                             int32_t *input_ids, int32_t W, const uint8_t *mask_in, uint8_t *mask_out,
                             const float *threshold, const int32_t *p, const int32_t *b, float *conf,
                             int32_t *argmax, uint8_t *done, int32_t *accept_len, void *workspace,
                             size_t workspace_bytes, int32_t *status, int32_t *unmasked, uint8_t *fallback);

/* dllm_step_quota and dllm_step_decide_quota — the step (and its deciding half) with the fixed
 * per-step quota of [BlockServe] §II-E (向量化混合调度执行: the per-step transfer quota spreads a
 * block's masked tokens evenly over S diffusion steps; §III-A: S = 32 for L = 32) in place of the
 * threshold.  Confidence and predicted token are those of dllm_step.  Per row with m masked slots:
 *   base = L / S, rem = L % S; step t of a block takes base + (t < rem) tokens;
 *   t = the last step whose running total t*base + min(t, rem) does not exceed L - m;
 *   k = m if t >= S, else min(m, base + (t < rem));
 *   U = the k masked slots with the largest confidence, the lowest j on ties.
 * Write-back, done and accept_len as for dllm_step.  steps_per_block >= 1 (DLLM_ERR_ARG
 * otherwise); no threshold.  Other arguments and errors as for dllm_step / dllm_step_decide. */
dllm_status dllm_step_quota(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                            int64_t row_stride, int32_t rows, int32_t L, int32_t V, int32_t *input_ids,
                            int32_t W, const uint8_t *mask_in, uint8_t *mask_out, int32_t steps_per_block,
                            const int32_t *p, const int32_t *b, float *conf, int32_t *argmax, uint8_t *done,
                            int32_t *accept_len, void *workspace, size_t workspace_bytes, int32_t *status);
dllm_status dllm_step_decide_quota(void *stream, int32_t dtype, int32_t rows, int32_t L, int32_t V,
                                   int32_t *input_ids, int32_t W, const uint8_t *mask_in, uint8_t *mask_out,
                                   int32_t steps_per_block, const int32_t *p, const int32_t *b, float *conf,
                                   int32_t *argmax, uint8_t *done, int32_t *accept_len, void *workspace,
                                   size_t workspace_bytes, int32_t *status);

/* dllm_step_score_shard and dllm_step_decide_shards — the step over a vocabulary split into
 * n_shards contiguous column ranges (a tensor-parallel language-model head: [DiLaServe] §三 3.2 ②
 * and §四 4.5 serve every step on tensor-parallel instances).
 *
 * dllm_step_score_shard scores shard `shard` (columns vocab_offset .. vocab_offset + V_shard - 1)
 * of every masked slot: logits point at that shard's column 0 with the given strides (as for
 * dllm_step, with V = V_shard).  For each masked slot it writes one record {float m, float S,
 * int32 a, int32 0} = (max of the shard, sum of exp(x - m) over the shard, global index of the
 * shard's first max) to triples[(r*L + j)*n_shards + shard]; other records are untouched.  The
 * workspace is that of dllm_step for V_shard.
 * dllm_step_decide_shards combines the n_shards records of every masked slot in shard order:
 * m = max m_t, a = the smallest a_t with m_t = m, S = sum_t S_t exp(m_t - m), c = 1/S, by the fixed
 * merge tree dllm_step uses for its chunks, and then applies the LowConfidence rule with the
 * outputs and conditions of dllm_step (V = the whole vocabulary, for the argmax range check).
 * Every rank of a tensor-parallel group that holds the same records reaches the same decisions.
 * triples: device memory of dllm_shard_triples_bytes(rows, L, n_shards) bytes, 16-byte aligned.
 * Errors: as dllm_step_score / dllm_step_decide, plus DLLM_ERR_ARG for a shard outside
 * [0, n_shards), n_shards outside [1, DLLM_MAX_SHARDS], a negative vocab_offset or null triples. */
size_t dllm_shard_triples_bytes(int32_t rows, int32_t L, int32_t n_shards);
dllm_status dllm_step_score_shard(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                                  int64_t row_stride, int32_t rows, int32_t L, int32_t V_shard,
                                  int32_t vocab_offset, int32_t shard, int32_t n_shards,
                                  const uint8_t *mask_in, void *workspace, size_t workspace_bytes,
                                  void *triples, int32_t *status);
dllm_status dllm_step_decide_shards(void *stream, int32_t n_shards, const void *triples, int32_t rows,
                                    int32_t L, int32_t V, int32_t *input_ids, int32_t W,
                                    const uint8_t *mask_in, uint8_t *mask_out, const float *threshold,
                                    const int32_t *p, const int32_t *b, float *conf, int32_t *argmax,
                                    uint8_t *done, int32_t *accept_len, int32_t *status);

/* dllm_step_features — per-request inputs of a remaining-step predictor, after a step.
 *
 * Defined by [DiLaServe] §四 4.2 ③ (paper §3.2.3, Step Prediction): progress features (the
 * fraction of tokens already unmasked) and confidence features (quantiles of the output tokens'
 * confidences); the page names the threshold, output length, full and block progress and the
 * min / q25 / median / mean / q75 confidence (it counts 11, these 9 are the ones it names).  The
 * predictor itself (a trained model) is not part of this library.
 *
 * For row r holding request q = row_req[r]:
 *   features[r, 0..8] (float32) = { threshold[q], K[q]*L, (b[q]*L + u)/(K[q]*L), u/L,
 *                                   min c, q25 c, median c, mean c, q75 c }
 * with u = slots of the row's block unmasked after the step (L minus the nonzero mask_out bytes)
 * and c the confidences the step scored (conf >= 0; conf as written by dllm_step).  Quantiles
 * interpolate linearly between order statistics at position q*(n-1); with no scored slot the five
 * confidence features are NaN.  b[q] is the current block (call before dllm_compact).
 * row_req: int32 [rows]; conf: float32 [rows, L]; mask_out: uint8 [rows, L]; features: float32
 * [rows, 9].  Errors: DLLM_ERR_ARG (null pointer, incomplete table; on the device *status for a
 * bad request id, whose row reads NaN), DLLM_ERR_SHAPE (L or rows out of range). */
dllm_status dllm_step_features(void *stream, int32_t rows, int32_t L, const int32_t *row_req,
                               const dllm_reqs *reqs, const float *conf, const uint8_t *mask_out,
                               float *features, int32_t *status);

/* dllm_pack — materialise the left-padded bounding box for the active rows.
 *
 * Defined by [BlockServe] §II-D Eq.(1) (row width p_i + (b_i + 1) L) and §II-E 逻辑位置对齐 (a dense
 * |A| x W tensor, left padded; position ids count real tokens so the first is position 0) and
 * 向量化混合调度执行 (gather of each request's active block for denoising).
 *
 * For row r < rows holding request q = row_req[r], with w = p[q] + (b[q] + 1) L, pad = W - w:
 *   box_ids[r, c] = pad_id for c < pad, else arena[arena_off[q] + c - pad];
 *   box_valid[r, c] = c >= pad;  box_pos[r, c] = c >= pad ? c - pad : 0;
 *   mask[r, :] = blk_mask[q, :];  threshold[r] = reqs->threshold[q];  p[r] = p[q];  b[r] = b[q].
 * box_ids: int32 [rows, W]; box_valid (uint8) and box_pos (int32) [rows, W] may be NULL.
 * W is normally dllm_meta.W from the preceding dllm_compact.  Device errors: request id out of
 * range, not active, or with b outside [0, K) -> DLLM_ERR_ARG (that row is written as all pads
 * with an empty mask); w > W -> DLLM_ERR_SHAPE (that row is written as all pads).
 * Synchronous errors: null required pointer, rows < 0, L outside [1, DLLM_MAX_L], W < L when
 * rows > 0, rows > DLLM_MAX_ROWS.  rows == 0 is a no-op. */
dllm_status dllm_pack(void *stream, int32_t rows, int32_t L, int32_t W, int32_t pad_id,
                      const int32_t *row_req, const dllm_reqs *reqs, int32_t *box_ids,
                      uint8_t *box_valid, int32_t *box_pos, uint8_t *mask, float *threshold,
                      int32_t *p, int32_t *b, int32_t *status);

/* dllm_compact — block-boundary commit, eviction and token-budget refill.
 *
 * Defined by [FDFO] §FDFO 的核心思想 and §工程设计二 (a finished block is committed and its request
 * leaves or moves on; an unfinished one keeps its partial block), §工程设计四 (unfinished blocks keep
 * their slot in place), [BlockServe] §II-C Algorithm 1 (admit under Cost <= beta; advance b_i; evict
 * when b_i >= K_i or at end of sequence) and §II-D (queue sorted by prompt length; "sand-fill"
 * refill with a candidate whose p + L fits the current box; Cost of Eq.(1)).
 *
 * In order:
 *  1. (box given) for every row r < rows holding q = row_req[r]: block b[q] of q's arena <-
 *     box_ids[r, W-L : W]; blk_mask[q, :] <- mask[r, :].
 *  2. (box given) for every row with done[r]: b[q] += 1; if b[q] >= K[q], or eos_id >= 0 and the
 *     committed block contains eos_id, q is finished (state 2) and row r is freed; otherwise q keeps
 *     row r with a fresh block of L mask_id tokens and an all-ones mask.
 *  3. admission, while fewer than rows_cap rows are active and the queue is not empty: with W_A
 *     the current box width (0 if empty), the candidate is the queued request with the largest p
 *     such that p + L <= W_A (lowest id on ties), else the one with the smallest p; it is admitted
 *     (state 1, b = 0, fresh masked block 0) iff budget <= 0 or (active + 1) * max(W_A, p + L) <=
 *     budget; the first rejection ends admission.  A rejection with no active row sets *status =
 *     DLLM_ERR_CAPACITY.
 *  4. rows: admissions take the freed rows in ascending order, then rows after the old last row;
 *     remaining holes are filled by moving the highest-index active rows into the lowest holes, so
 *     rows 0 .. n-1 are dense; every other request keeps its row.  row_req[n .. rows_cap) = -1.
 *  5. meta <- {rows, W, n_evicted, n_admitted, n_queued, cost}.
 * box_ids (int32 [rows, W]), mask (uint8 [rows, L]) and done (uint8 [rows]) are either all given
 * or all NULL; with all NULL only steps 3-5 run (the start of a run).  row_req: int32 [rows_cap],
 * entries >= rows ignored on entry.  meta: device dllm_meta.
 * Synchronous errors: null required pointer, rows < 0, rows > rows_cap, rows_cap > DLLM_MAX_ROWS,
 * L outside [1, DLLM_MAX_L], queue->cap outside [0, DLLM_MAX_QUEUE], box given with W < L; and
 * DLLM_ERR_CAPACITY when rows_cap * 21 + queue->cap * 9 + 16 bytes (the row map and the queue's
 * prompt lengths, held in LDS) plus 4 KiB exceed the device's LDS per workgroup: on MI355X
 * (160 KiB) 4096 rows leave room for a queue of 8190.
 * Device errors: a row holding an id out of range, not active, or with b outside [0, K) ->
 * DLLM_ERR_ARG (the row is dropped); a queue entry out of range, not queued, or with K < 1 ->
 * DLLM_ERR_ARG (nothing is admitted and the queue is left as it is); *queue->len outside
 * [0, cap] -> DLLM_ERR_CAPACITY.  Preconditions: the queue is sorted by (p, id); arena regions
 * do not overlap. */
dllm_status dllm_compact(void *stream, int32_t rows, int32_t L, int32_t W, int32_t mask_id,
                         int32_t eos_id, const int32_t *box_ids, const uint8_t *mask,
                         const uint8_t *done, int32_t *row_req, int32_t rows_cap,
                         const dllm_reqs *reqs, const dllm_queue *queue, int64_t budget,
                         dllm_meta *meta, int32_t *status);

/* Text for the last non-OK status returned on the calling host thread ("" if none). */
const char *dllm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DLLM_H */
