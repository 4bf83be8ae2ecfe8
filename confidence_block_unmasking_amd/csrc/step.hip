// dllm_step: one LowConfidence denoise step over a packed box.
//
// What is computed ([FDFO] = page "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」",
// [DiLaServe] = page "DiLaServe: High SLO Attainment Serving for Diffusion Language Models"):
//   [FDFO] §工程设计一 — step() reads the logits, updates input_ids by the LowConfidence rule
//   (unmask masked slots whose confidence exceeds the threshold, else the single most confident
//   one) and returns per-block done flags; [DiLaServe] §三 3.1 — the confidence is the softmax
//   probability of the predicted token; [FDFO] §工程设计二 — accept length is 0 or block_size.
//
// How (gfx950).  The work is a streaming reduction over M masked slots x V logits, bound by HBM,
// done in two launches on the caller's stream:
//   1. score_kernel streams every masked slot's vocabulary row once.  Each row is cut into NC
//      chunks of 64*kVPL 16-byte vectors (the last one shorter); the cut depends on V only, so a
//      slot's result never depends on the rest of the batch.  The M*NC chunks are split evenly
//      over the workgroups (four per compute unit, two resident at a time; fewer for small boxes).
//      Inside a workgroup the waves take chunks one at a time from an LDS counter: the sequencer
//      favours older waves when they compete for the memory pipe, so a fixed split per wave
//      leaves the young ones finishing last, while a shared counter lets every wave of the unit
//      finish within about one chunk of the others.  (Global atomics would do the same across
//      units but cost a memory round trip each and serialise on one address.)
//      One wavefront reduces one chunk: 64 lanes issue kVPL coalesced 16-byte non-temporal loads
//      each (1 KiB per wave instruction), the next chunk's loads go out before this chunk's
//      arithmetic, each element costs an unpack, a share of a max3, one FMA, one v_exp and one add
//      (sum of exp2(x*log2e - max*log2e)),
//      and lanes combine through DPP.  The chunk partial (max, sum, first element index at the
//      max) stays in a lane register until the wave has 64 of them or runs out of chunks, then
//      they leave in one store: a store between the loads of consecutive chunks would hold back
//      every later load until it completed.
//   2. decide_kernel, one workgroup per row, merges each masked slot's NC partials in chunk order
//      (a fixed tree, so the bits are reproducible), and applies the unmask rule to the row.
//   The launch boundary is what makes the partials of kernel 1 visible to kernel 2.  A one-launch
//   variant (the last workgroup to finish a row decides it) needs an agent-scope release (an L2
//   write-back) in every scoring workgroup and an acquire in the deciding one; the release alone
//   costs more than the whole second launch on this part.  With device-coherent stores and loads
//   standing in for those fences it read stale partials.  No MFMA: there is no contraction here.
//
// This file holds the argument checks and the C entry points; the kernels are in score.hip and
// decide.hip, their shared definitions in step_common.h.
#include <mutex>

#include "step_common.h"

// The workspace of dllm_step_noalloc: a fixed device array (one copy per GPU, allocated by the
// runtime with the code object and held until the process ends).  In host code its name is only a
// stand-in; the device address comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed on.
static __device__ __align__(256) unsigned char scratch[DLLM_NOALLOC_SCRATCH_BYTES];

namespace dllm {
// decide.hip: launch_decide with an event bound to the deciding kernel's end (nullptr: none)
dllm_status launch_decide_ev(const StepParams &P, hipStream_t st, int mode, hipEvent_t ev_stop);
}  // namespace dllm

namespace {

using namespace dllm;

// Checks shared by the three entry points; fills P's shape fields.  `who` names the caller.
dllm_status check_shape(const char *who, int32_t dtype, int32_t rows, int32_t L, int32_t V, void *workspace,
                        StepParams &P) {
    if (dtype != DLLM_FP32 && dtype != DLLM_BF16) return fail(DLLM_ERR_DTYPE, "%s: unknown dtype %d", who, (int)dtype);
    if (rows < 0) return fail(DLLM_ERR_ARG, "%s: rows < 0", who);
    if (L < 1 || L > DLLM_MAX_L) return fail(DLLM_ERR_SHAPE, "%s: L=%d outside [1, %d]", who, L, DLLM_MAX_L);
    if (V < 1) return fail(DLLM_ERR_ARG, "%s: V < 1", who);
    if (rows > DLLM_MAX_ROWS || (int64_t)rows * L > DLLM_MAX_POSITIONS)
        return fail(DLLM_ERR_SHAPE, "%s: rows=%d, L=%d exceed the limits", who, rows, L);
    int NV, NC;
    size_t need;
    shape_of(rows, L, V, dtype, NV, NC, need);
    if ((int64_t)rows * L * NC >= (int64_t)1 << 31) return fail(DLLM_ERR_SHAPE, "%s: rows*L*chunks too large", who);
    P.rows = rows; P.L = L; P.V = V; P.NV = NV; P.NC = NC;
    P.partials = (float4 *)workspace;
    return DLLM_OK;
}

// The workspace check, after every other argument check.
dllm_status check_workspace(const char *who, int32_t dtype, const void *workspace, size_t workspace_bytes,
                            const StepParams &P) {
    if (P.rows == 0) return DLLM_OK;
    int NV, NC;
    size_t need;
    shape_of(P.rows, P.L, P.V, dtype, NV, NC, need);
    if (!workspace) return fail(DLLM_ERR_ARG, "%s: null workspace", who);
    if (workspace_bytes < need)
        return fail(DLLM_ERR_ARG, "%s: workspace %zu bytes < %zu needed", who, workspace_bytes, need);
    if (((uintptr_t)workspace & 15) != 0) return fail(DLLM_ERR_ARG, "%s: workspace not 16-byte aligned", who);
    return DLLM_OK;
}

dllm_status check_score(const char *who, const void *logits, int32_t dtype, int64_t pos_stride, int64_t row_stride,
                        const uint8_t *mask_in, int32_t *status, StepParams &P) {
    if (pos_stride < P.V || row_stride < (int64_t)P.L * pos_stride)
        return fail(DLLM_ERR_ARG, "%s: strides too small (pos %lld, row %lld)", who, (long long)pos_stride,
                    (long long)row_stride);
    if (P.rows > 0 && (!logits || !mask_in || !status)) return fail(DLLM_ERR_ARG, "%s: null required pointer", who);
    const int es = dtype == DLLM_BF16 ? 2 : 4;
    P.logits = (const char *)logits;
    P.pos_stride_b = pos_stride * es;
    P.row_stride_b = row_stride * es;
    P.mask_in = mask_in;
    P.status = status;
    return DLLM_OK;
}

// steps = 0: the threshold rule (threshold required); steps >= 1: the quota rule with that many
// diffusion steps per block (threshold unused).
dllm_status check_decide(const char *who, int32_t *input_ids, int32_t W, const uint8_t *mask_in, uint8_t *mask_out,
                         const float *threshold, int32_t steps, const int32_t *p, const int32_t *b, float *conf,
                         int32_t *argmax, uint8_t *done, int32_t *accept_len, int32_t *status, StepParams &P) {
    if (W < P.L) return fail(DLLM_ERR_SHAPE, "%s: W=%d < L=%d", who, W, P.L);
    if ((p == nullptr) != (b == nullptr)) return fail(DLLM_ERR_ARG, "%s: p and b must be both given or both NULL", who);
    if (steps < 0) return fail(DLLM_ERR_ARG, "%s: steps_per_block < 1", who);
    P.S = steps;
    if (P.rows == 0) return DLLM_OK;
    if (!input_ids || !mask_in || !mask_out || (steps == 0 && !threshold) || !done || !accept_len || !status)
        return fail(DLLM_ERR_ARG, "%s: null required pointer", who);
    if (!threshold) threshold = (const float *)accept_len;   // never read for its value
    const int64_t S = (int64_t)P.rows * P.L;
    if (mask_out != mask_in && (uintptr_t)mask_out < (uintptr_t)mask_in + (uintptr_t)S &&
        (uintptr_t)mask_in < (uintptr_t)mask_out + (uintptr_t)S)
        return fail(DLLM_ERR_ARG, "%s: mask_out partly overlaps mask_in", who);
    P.W = W;
    P.ids = input_ids; P.mask_in = mask_in; P.mask_out = mask_out; P.tau = threshold;
    P.check_fit = p != nullptr;
    P.p = p ? p : (const int32_t *)threshold;  // a readable array of `rows` 4-byte entries
    P.b = b ? b : (const int32_t *)threshold;
    P.conf_out = conf; P.arg_out = argmax; P.done = done; P.accept = accept_len;
    P.status = status;
    return DLLM_OK;
}


constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call on each device).
dllm_status scratch_address(const char *who, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return check_hip(e, who);
    if (dev < 0 || dev >= kMaxDevices) return fail(DLLM_ERR_ARG, "%s: device %d beyond the %d this library tracks", who,
                                                   dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        void *addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return check_hip(e, "dllm_step_noalloc: hipGetSymbolAddress");
        if (addr == nullptr) return fail(DLLM_ERR_HIP, "%s: no device address for the scratch array", who);
        g_scratch_addr[dev] = addr;
    }
    *out = g_scratch_addr[dev];
    return DLLM_OK;
}

}  // namespace


extern "C" size_t dllm_step_workspace_bytes(int32_t rows, int32_t L, int32_t V, int32_t dtype) {
    int NV, NC;
    size_t bytes;
    if (!shape_of(rows, L, V, dtype, NV, NC, bytes)) return 0;
    return bytes;
}

extern "C" dllm_status dllm_step(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                                 int64_t row_stride, int32_t rows, int32_t L, int32_t V, int32_t *input_ids,
                                 int32_t W, const uint8_t *mask_in, uint8_t *mask_out, const float *threshold,
                                 const int32_t *p, const int32_t *b, float *conf, int32_t *argmax,
                                 uint8_t *done, int32_t *accept_len, void *workspace, size_t workspace_bytes,
                                 int32_t *status) {
    StepParams P{};
    dllm_status rc = check_shape("dllm_step", dtype, rows, L, V, workspace, P);
    if (rc == DLLM_OK) rc = check_score("dllm_step", logits, dtype, pos_stride, row_stride, mask_in, status, P);
    if (rc == DLLM_OK)
        rc = check_decide("dllm_step", input_ids, W, mask_in, mask_out, threshold, 0, p, b, conf, argmax, done,
                          accept_len, status, P);
    if (rc == DLLM_OK) rc = check_workspace("dllm_step", dtype, workspace, workspace_bytes, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    rc = launch_score(P, dtype, (hipStream_t)stream);
    if (rc != DLLM_OK) return rc;
    return launch_decide(P, (hipStream_t)stream, P.S > 0 ? kRuleQuota : kRuleThreshold);
}

extern "C" dllm_status dllm_step_noalloc(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                                         int64_t row_stride, int32_t rows, int32_t L, int32_t V, int32_t *input_ids,
                                         int32_t W, const uint8_t *mask_in, uint8_t *mask_out, const float *threshold,
                                         const int32_t *p, const int32_t *b, float *conf, int32_t *argmax,
                                         uint8_t *done, int32_t *accept_len, int32_t *status) {
    const char *who = "dllm_step_noalloc";
    StepParams P{};
    dllm_status rc = check_shape(who, dtype, rows, L, V, nullptr, P);
    if (rc == DLLM_OK) rc = check_score(who, logits, dtype, pos_stride, row_stride, mask_in, status, P);
    if (rc == DLLM_OK)
        rc = check_decide(who, input_ids, W, mask_in, mask_out, threshold, 0, p, b, conf, argmax, done, accept_len,
                          status, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    int NV, NC;
    size_t need;
    shape_of(rows, L, V, dtype, NV, NC, need);
    if (need > DLLM_NOALLOC_SCRATCH_BYTES)
        return fail(DLLM_ERR_CAPACITY, "%s: rows=%d, L=%d, V=%d need %zu bytes of workspace; the fixed scratch "
                    "holds %zu (use dllm_step with a caller workspace)", who, rows, L, V, need,
                    (size_t)DLLM_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    rc = scratch_address(who, &ws);
    if (rc != DLLM_OK) return rc;
    P.partials = (float4 *)ws;
    rc = launch_score(P, dtype, (hipStream_t)stream);
    if (rc != DLLM_OK) return rc;
    return launch_decide(P, (hipStream_t)stream, kRuleThreshold);
}

extern "C" dllm_status dllm_step_timed(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                                       int64_t row_stride, int32_t rows, int32_t L, int32_t V, int32_t *input_ids,
                                       int32_t W, const uint8_t *mask_in, uint8_t *mask_out, const float *threshold,
                                       const int32_t *p, const int32_t *b, float *conf, int32_t *argmax,
                                       uint8_t *done, int32_t *accept_len, void *workspace, size_t workspace_bytes,
                                       int32_t *status, void *start_event, void *stop_event) {
    if (!start_event || !stop_event) return fail(DLLM_ERR_ARG, "dllm_step_timed: null event");
    StepParams P{};
    dllm_status rc = check_shape("dllm_step_timed", dtype, rows, L, V, workspace, P);
    if (rc == DLLM_OK) rc = check_score("dllm_step_timed", logits, dtype, pos_stride, row_stride, mask_in, status, P);
    if (rc == DLLM_OK)
        rc = check_decide("dllm_step_timed", input_ids, W, mask_in, mask_out, threshold, 0, p, b, conf, argmax, done,
                          accept_len, status, P);
    if (rc == DLLM_OK) rc = check_workspace("dllm_step_timed", dtype, workspace, workspace_bytes, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    rc = launch_score(P, dtype, (hipStream_t)stream, (hipEvent_t)start_event, nullptr);
    if (rc != DLLM_OK) return rc;
    return launch_decide_ev(P, (hipStream_t)stream, kRuleThreshold, (hipEvent_t)stop_event);
}

extern "C" dllm_status dllm_step_score(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                                       int64_t row_stride, int32_t rows, int32_t L, int32_t V,
                                       const uint8_t *mask_in, void *workspace, size_t workspace_bytes,
                                       int32_t *status) {
    StepParams P{};
    dllm_status rc = check_shape("dllm_step_score", dtype, rows, L, V, workspace, P);
    if (rc == DLLM_OK) rc = check_score("dllm_step_score", logits, dtype, pos_stride, row_stride, mask_in, status, P);
    if (rc == DLLM_OK) rc = check_workspace("dllm_step_score", dtype, workspace, workspace_bytes, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    return launch_score(P, dtype, (hipStream_t)stream);
}

extern "C" dllm_status dllm_step_score_timed(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                                             int64_t row_stride, int32_t rows, int32_t L, int32_t V,
                                             const uint8_t *mask_in, void *workspace, size_t workspace_bytes,
                                             int32_t *status, void *start_event, void *stop_event) {
    if (!start_event || !stop_event) return fail(DLLM_ERR_ARG, "dllm_step_score_timed: null event");
    StepParams P{};
    dllm_status rc = check_shape("dllm_step_score_timed", dtype, rows, L, V, workspace, P);
    if (rc == DLLM_OK)
        rc = check_score("dllm_step_score_timed", logits, dtype, pos_stride, row_stride, mask_in, status, P);
    if (rc == DLLM_OK) rc = check_workspace("dllm_step_score_timed", dtype, workspace, workspace_bytes, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    return launch_score(P, dtype, (hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event);
}

extern "C" dllm_status dllm_step_decide(void *stream, int32_t dtype, int32_t rows, int32_t L, int32_t V,
                                        int32_t *input_ids, int32_t W, const uint8_t *mask_in, uint8_t *mask_out,
                                        const float *threshold, const int32_t *p, const int32_t *b, float *conf,
                                        int32_t *argmax, uint8_t *done, int32_t *accept_len, void *workspace,
                                        size_t workspace_bytes, int32_t *status, int32_t *unmasked,
                                        uint8_t *fallback) {
    StepParams P{};
    dllm_status rc = check_shape("dllm_step_decide", dtype, rows, L, V, workspace, P);
    if (rc == DLLM_OK)
        rc = check_decide("dllm_step_decide", input_ids, W, mask_in, mask_out, threshold, 0, p, b, conf, argmax,
                          done, accept_len, status, P);
    if (rc == DLLM_OK) rc = check_workspace("dllm_step_decide", dtype, workspace, workspace_bytes, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    P.unmasked_out = unmasked;
    P.fallback_out = fallback;
    return launch_decide(P, (hipStream_t)stream, P.S > 0 ? kRuleQuota : kRuleThreshold);
}

extern "C" dllm_status dllm_step_quota(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                                       int64_t row_stride, int32_t rows, int32_t L, int32_t V, int32_t *input_ids,
                                       int32_t W, const uint8_t *mask_in, uint8_t *mask_out,
                                       int32_t steps_per_block, const int32_t *p, const int32_t *b, float *conf,
                                       int32_t *argmax, uint8_t *done, int32_t *accept_len, void *workspace,
                                       size_t workspace_bytes, int32_t *status) {
    StepParams P{};
    if (steps_per_block < 1) return fail(DLLM_ERR_ARG, "dllm_step_quota: steps_per_block < 1");
    dllm_status rc = check_shape("dllm_step_quota", dtype, rows, L, V, workspace, P);
    if (rc == DLLM_OK) rc = check_score("dllm_step_quota", logits, dtype, pos_stride, row_stride, mask_in, status, P);
    if (rc == DLLM_OK)
        rc = check_decide("dllm_step_quota", input_ids, W, mask_in, mask_out, nullptr, steps_per_block, p, b, conf,
                          argmax, done, accept_len, status, P);
    if (rc == DLLM_OK) rc = check_workspace("dllm_step_quota", dtype, workspace, workspace_bytes, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    rc = launch_score(P, dtype, (hipStream_t)stream);
    if (rc != DLLM_OK) return rc;
    return launch_decide(P, (hipStream_t)stream, P.S > 0 ? kRuleQuota : kRuleThreshold);
}

extern "C" dllm_status dllm_step_decide_quota(void *stream, int32_t dtype, int32_t rows, int32_t L, int32_t V,
                                              int32_t *input_ids, int32_t W, const uint8_t *mask_in,
                                              uint8_t *mask_out, int32_t steps_per_block, const int32_t *p,
                                              const int32_t *b, float *conf, int32_t *argmax, uint8_t *done,
                                              int32_t *accept_len, void *workspace, size_t workspace_bytes,
                                              int32_t *status) {
    StepParams P{};
    if (steps_per_block < 1) return fail(DLLM_ERR_ARG, "dllm_step_decide_quota: steps_per_block < 1");
    dllm_status rc = check_shape("dllm_step_decide_quota", dtype, rows, L, V, workspace, P);
    if (rc == DLLM_OK)
        rc = check_decide("dllm_step_decide_quota", input_ids, W, mask_in, mask_out, nullptr, steps_per_block, p, b,
                          conf, argmax, done, accept_len, status, P);
    if (rc == DLLM_OK) rc = check_workspace("dllm_step_decide_quota", dtype, workspace, workspace_bytes, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    return launch_decide(P, (hipStream_t)stream, P.S > 0 ? kRuleQuota : kRuleThreshold);
}

extern "C" size_t dllm_shard_triples_bytes(int32_t rows, int32_t L, int32_t n_shards) {
    if (rows < 0 || L < 1 || n_shards < 1) return 0;
    return (size_t)rows * (size_t)L * (size_t)n_shards * sizeof(float4);
}

extern "C" dllm_status dllm_step_score_shard(void *stream, const void *logits, int32_t dtype, int64_t pos_stride,
                                             int64_t row_stride, int32_t rows, int32_t L, int32_t V_shard,
                                             int32_t vocab_offset, int32_t shard, int32_t n_shards,
                                             const uint8_t *mask_in, void *workspace, size_t workspace_bytes,
                                             void *triples, int32_t *status) {
    StepParams P{};
    dllm_status rc = check_shape("dllm_step_score_shard", dtype, rows, L, V_shard, workspace, P);
    if (rc == DLLM_OK)
        rc = check_score("dllm_step_score_shard", logits, dtype, pos_stride, row_stride, mask_in, status, P);
    if (rc != DLLM_OK) return rc;
    if (n_shards < 1 || n_shards > DLLM_MAX_SHARDS || shard < 0 || shard >= n_shards)
        return fail(DLLM_ERR_ARG, "dllm_step_score_shard: shard %d of %d", shard, n_shards);
    if (vocab_offset < 0 || (int64_t)vocab_offset + V_shard > INT32_MAX)
        return fail(DLLM_ERR_ARG, "dllm_step_score_shard: vocab_offset %d", vocab_offset);
    if (rows > 0 && !triples) return fail(DLLM_ERR_ARG, "dllm_step_score_shard: null triples");
    rc = check_workspace("dllm_step_score_shard", dtype, workspace, workspace_bytes, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    P.triples = (float4 *)triples;
    P.shard = shard;
    P.n_shards = n_shards;
    P.vocab_offset = vocab_offset;
    rc = launch_score(P, dtype, (hipStream_t)stream);
    if (rc != DLLM_OK) return rc;
    return launch_decide(P, (hipStream_t)stream, kEmitTriples);
}

extern "C" dllm_status dllm_step_decide_shards(void *stream, int32_t n_shards, const void *triples, int32_t rows,
                                               int32_t L, int32_t V, int32_t *input_ids, int32_t W,
                                               const uint8_t *mask_in, uint8_t *mask_out, const float *threshold,
                                               const int32_t *p, const int32_t *b, float *conf, int32_t *argmax,
                                               uint8_t *done, int32_t *accept_len, int32_t *status) {
    StepParams P{};
    if (n_shards < 1 || n_shards > DLLM_MAX_SHARDS)
        return fail(DLLM_ERR_ARG, "dllm_step_decide_shards: n_shards=%d outside [1, %d]", n_shards, DLLM_MAX_SHARDS);
    dllm_status rc = check_shape("dllm_step_decide_shards", DLLM_FP32, rows, L, V, nullptr, P);
    if (rc == DLLM_OK)
        rc = check_decide("dllm_step_decide_shards", input_ids, W, mask_in, mask_out, threshold, 0, p, b, conf, argmax,
                          done, accept_len, status, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    if (!triples) return fail(DLLM_ERR_ARG, "dllm_step_decide_shards: null triples");
    P.partials = (float4 *)triples;            // the shards play the part of a slot's chunks
    P.NC = n_shards;
    return launch_decide(P, (hipStream_t)stream, kRuleThreshold);
}
