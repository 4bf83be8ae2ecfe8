// dllm_pack: materialise the left-padded bounding box of the active rows.
//
// [BlockServe] = page "BlockServe: 块粒度连续批处理实现高吞吐扩散大语言模型服务".
//   §II-D Eq.(1): a request at block index b has row width p + (b + 1) L; the box is the active set
//   times the widest row.  §II-E 逻辑位置对齐: the box is a dense tensor with left padding, prompts
//   contiguous and followed by their generated region; position ids count real tokens from 0.
//   §II-E 向量化混合调度执行: gather of each request's active block into the batch.
//
// One workgroup per row; lanes stride over the W columns with coalesced 4-byte stores.  Integer
// gather only: O(rows * W) bytes written (a few MB at the largest shapes).
#include "common.h"

namespace {

using namespace dllm;

constexpr int kThreads = 256;

constexpr int kUnroll = 8;   // box columns per thread whose loads go out together

// Latency-bound (a few kilobytes per row): three dependent memory round trips per row, the row's
// request id, then every field of that request at once, then the arena gather and the block mask,
// each thread issuing all its loads before any of its stores.
__global__ __launch_bounds__(kThreads) void pack_kernel(int32_t L, int32_t W, int32_t pad_id,
                                                        const int32_t *__restrict__ row_req, dllm_reqs R,
                                                        int32_t *__restrict__ box_ids, uint8_t *__restrict__ box_valid,
                                                        int32_t *__restrict__ box_pos, uint8_t *__restrict__ mask,
                                                        float *__restrict__ tau, int32_t *__restrict__ p_out,
                                                        int32_t *__restrict__ b_out, int32_t *status) {
    fetch_args(row_req, R.n_req, R.p, R.K, R.b, R.state, R.threshold, R.arena_off, R.arena, R.blk_mask, box_ids,
               box_valid, box_pos, mask, tau, p_out, b_out, status, L, W, pad_id);
    const int r = blockIdx.x;
    const int q = row_req[r];
    const bool in_range = q >= 0 && q < R.n_req;
    int st = 0, bq = -1, Kq = 0, pq = 0;
    int64_t off = 0;
    float th = 0.0f;
    if (in_range) {                            // one branch: the six loads go out together
        st = R.state[q];
        bq = R.b[q];
        Kq = R.K[q];
        pq = R.p[q];
        off = R.arena_off[q];
        th = R.threshold[q];
    }
    const bool ok_id = in_range && st == 1 && bq >= 0 && bq < Kq;
    int64_t pad = W;
    if (ok_id) pad = W - ((int64_t)pq + ((int64_t)bq + 1) * L);
    const bool fits = ok_id && pad >= 0;
    if (threadIdx.x == 0) {
        if (!ok_id) set_status(status, DLLM_ERR_ARG);
        else if (!fits) set_status(status, DLLM_ERR_SHAPE);
        tau[r] = ok_id ? th : 0.0f;
        p_out[r] = ok_id ? pq : 0;
        b_out[r] = ok_id ? bq : 0;
    }
    // the block mask (L <= 4 * kThreads) and the first kUnroll strides of columns: loads first
    uint8_t mv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = threadIdx.x + u * kThreads;
        mv[u] = 0;
        if (ok_id && j < L) mv[u] = R.blk_mask[(int64_t)q * L + j];
    }
    const int64_t rb = (int64_t)r * W;
    for (int c0 = threadIdx.x; c0 < W; c0 += kUnroll * kThreads) {
        int v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = c0 + u * kThreads;
            v[u] = pad_id;
            if (fits && c < W && c >= pad) v[u] = R.arena[off + (c - pad)];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = c0 + u * kThreads;
            if (c < W) {
                const bool valid = fits && c >= pad;
                box_ids[rb + c] = v[u];
                if (box_valid) box_valid[rb + c] = valid ? 1 : 0;
                if (box_pos) box_pos[rb + c] = valid ? (int32_t)(c - pad) : 0;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = threadIdx.x + u * kThreads;
        if (j < L) mask[(int64_t)r * L + j] = mv[u];
    }
}

}  // namespace

extern "C" dllm_status dllm_pack(void *stream, int32_t rows, int32_t L, int32_t W, int32_t pad_id,
                                 const int32_t *row_req, const dllm_reqs *reqs, int32_t *box_ids,
                                 uint8_t *box_valid, int32_t *box_pos, uint8_t *mask, float *threshold,
                                 int32_t *p, int32_t *b, int32_t *status) {
    if (rows < 0) return fail(DLLM_ERR_ARG, "dllm_pack: rows < 0");
    if (L < 1 || L > DLLM_MAX_L) return fail(DLLM_ERR_SHAPE, "dllm_pack: L=%d outside [1, %d]", L, DLLM_MAX_L);
    if (rows > DLLM_MAX_ROWS) return fail(DLLM_ERR_SHAPE, "dllm_pack: rows=%d > %d", rows, DLLM_MAX_ROWS);
    if (rows == 0) return DLLM_OK;
    if (W < L) return fail(DLLM_ERR_SHAPE, "dllm_pack: W=%d < L=%d", W, L);
    if (!row_req || !reqs || !box_ids || !mask || !threshold || !p || !b || !status)
        return fail(DLLM_ERR_ARG, "dllm_pack: null required pointer");
    if (!reqs->p || !reqs->K || !reqs->b || !reqs->state || !reqs->threshold || !reqs->arena_off || !reqs->arena ||
        !reqs->blk_mask || reqs->n_req < 0)
        return fail(DLLM_ERR_ARG, "dllm_pack: incomplete request table");
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream, L, W, pad_id,
                       row_req, *reqs, box_ids, box_valid, box_pos, mask, threshold, p, b, status);
    return check_hip(hipGetLastError(), "dllm_pack launch");
}
