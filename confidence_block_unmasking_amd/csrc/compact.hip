// dllm_compact: block-boundary commit, eviction and token-budget refill (first-done-first-out).
//
// [FDFO] = page "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」":
//   §FDFO 的核心思想 — a request whose block finishes leaves the batch at once and its resources are
//   reused; §工程设计二 — unfinished: keep the partial block; finished: commit it, update the finish
//   state; §工程设计四 — unfinished blocks keep their slot in place.
// [BlockServe] = page "BlockServe: 块粒度连续批处理实现高吞吐扩散大语言模型服务":
//   §II-C Algorithm 1 — admit while Cost(A ∪ {r_cand}) <= beta, advance b_i, evict at b_i >= K_i or
//   end of sequence; §II-D — queue sorted by prompt length, refill with a candidate whose p + L
//   fits the current box ("sand filling"), Cost of Eq.(1); §II-E — each block starts fully masked.
//
// One workgroup of 1024 threads: the O(rows * L) scatter, commits and fills run in parallel; the
// greedy admission is inherently sequential (each choice changes the box width) and runs on one
// thread over LDS copies of the queue's prompt lengths, with a binary search for the best fit.
// The queue is compacted in place (in order) with a parallel prefix scan.
#include "common.h"

namespace {

using namespace dllm;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

struct CompactParams {
    int32_t rows, L, W, mask_id, eos_id, rows_cap;
    const int32_t *box_ids;
    const uint8_t *mask;
    const uint8_t *done;
    int32_t *row_req;
    dllm_reqs R;
    int32_t *q_ids;
    int32_t *q_len;
    int32_t q_cap;
    int64_t budget;
    dllm_meta *meta;
    int32_t *status;
};

__device__ __forceinline__ int64_t block_start(const dllm_reqs &R, int q, int blk, int L) {
    return R.arena_off[q] + (int64_t)R.p[q] + (int64_t)blk * L;
}

__device__ int block_reduce_max(int v, int *scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max_i(v);
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    int r = scratch[0];
    for (int w = 1; w < kWaves; ++w) r = max(r, scratch[w]);
    return r;
}
__device__ int block_reduce_sum(int v, int *scratch) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum_i(v);
    __syncthreads();
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    int r = 0;
    for (int w = 0; w < kWaves; ++w) r += scratch[w];
    return r;
}

__global__ __launch_bounds__(kThreads) void compact_kernel(CompactParams P) {
    extern __shared__ int32_t lds[];
    __shared__ int red[kWaves];
    __shared__ int sh_nadm, sh_nnew, sh_qlen, sh_bad, sh_badid;
    const int tid = threadIdx.x;
    const int rows = P.rows, L = P.L, cap = P.rows_cap;
    const dllm_reqs &R = P.R;
    int32_t *s_row = lds;                        // [cap]   row -> request (-1 free)
    int32_t *s_adm = s_row + cap;                // [cap]   admitted queue indices, in order
    int32_t *s_qp = s_adm + cap;                 // [q_cap] prompt length of queue entries
    int32_t *s_qid = s_qp + P.q_cap;             // [q_cap] queue ids
    uint8_t *s_flag = (uint8_t *)(s_qid + P.q_cap);   // [cap] 1 = fresh block needed
    uint8_t *s_taken = s_flag + cap;             // [q_cap]

    if (tid == 0) {
        int ql = *P.q_len;
        sh_bad = (ql < 0 || ql > P.q_cap);
        sh_qlen = sh_bad ? 0 : ql;
        sh_badid = 0;
        if (sh_bad) set_status(P.status, DLLM_ERR_CAPACITY);
    }
    for (int r = tid; r < cap; r += kThreads) {
        int q = -1;
        if (r < rows) {
            q = P.row_req[r];
            if (q < 0 || q >= R.n_req || R.state[q] != 1 || R.b[q] < 0 || R.b[q] >= R.K[q]) {
                set_status(P.status, DLLM_ERR_ARG);
                q = -1;
            }
        }
        s_row[r] = q;
        s_flag[r] = 0;
    }
    __syncthreads();
    for (int i = tid; i < sh_qlen; i += kThreads) {
        const int id = P.q_ids[i];
        const bool ok = id >= 0 && id < R.n_req && R.state[id] == 0 && R.K[id] >= 1;
        s_qid[i] = id;
        s_qp[i] = ok ? R.p[id] : 0;
        s_taken[i] = 0;
        if (!ok) sh_badid = 1;
    }
    __syncthreads();
    if (sh_badid && tid == 0) set_status(P.status, DLLM_ERR_ARG);
    // a queue holding an invalid or non-queued id is left untouched and admits nothing
    const int qlen = sh_badid ? 0 : sh_qlen;
    const bool touch_queue = !sh_bad && !sh_badid;

    int n_evicted = 0;
    if (P.box_ids) {
        // 1. scatter active blocks (the last L box columns) and masks back to their requests
        for (int idx = tid; idx < rows * L; idx += kThreads) {
            const int r = idx / L, j = idx - (idx / L) * L;
            const int q = s_row[r];
            if (q < 0) continue;
            R.arena[block_start(R, q, R.b[q], L) + j] = P.box_ids[(int64_t)r * P.W + (P.W - L) + j];
            R.blk_mask[(int64_t)q * L + j] = P.mask[(int64_t)r * L + j];
        }
        __syncthreads();
        // 2. commit finished blocks: advance; evict, or open a fresh block in the same row
        int ev = 0;
        for (int r = tid; r < rows; r += kThreads) {
            const int q = s_row[r];
            if (q < 0 || !P.done[r]) continue;
            bool eos = false;
            if (P.eos_id >= 0)
                for (int j = 0; j < L; ++j) eos |= P.box_ids[(int64_t)r * P.W + (P.W - L) + j] == P.eos_id;
            const int nb = R.b[q] + 1;
            R.b[q] = nb;
            if (nb >= R.K[q] || eos) {
                R.state[q] = 2;
                s_row[r] = -1;
                ++ev;
            } else {
                s_flag[r] = 1;
            }
        }
        n_evicted = block_reduce_sum(ev, red);     // includes a barrier
        for (int idx = tid; idx < rows * L; idx += kThreads) {
            const int r = idx / L, j = idx - (idx / L) * L;
            if (!s_flag[r]) continue;
            const int q = s_row[r];
            R.arena[block_start(R, q, R.b[q], L) + j] = P.mask_id;
            R.blk_mask[(int64_t)q * L + j] = 1;
        }
    }
    __syncthreads();

    // 3. admission (sequential, one thread): current width and survivor count first
    int wloc = 0, nloc = 0;
    for (int r = tid; r < rows; r += kThreads) {
        const int q = s_row[r];
        if (q >= 0) {
            wloc = max(wloc, R.p[q] + (R.b[q] + 1) * L);
            ++nloc;
        }
    }
    const int W_A0 = block_reduce_max(wloc, red);
    const int n_act0 = block_reduce_sum(nloc, red);
    if (tid == 0) {
        int n_act = n_act0, W_A = W_A0, n_adm = 0, lo = 0;
        while (n_act < cap) {
            while (lo < qlen && s_taken[lo]) ++lo;
            if (lo >= qlen) break;
            int cand = -1;
            const int lim = W_A - L;               // best fit: largest p <= W_A - L
            if (lim >= 0 && s_qp[lo] <= lim) {
                int a = lo, bnd = qlen;             // first index with p > lim
                while (a < bnd) {
                    const int mid = (a + bnd) >> 1;
                    if (s_qp[mid] <= lim) a = mid + 1; else bnd = mid;
                }
                int i = a - 1;
                while (i >= lo && s_taken[i]) --i;
                if (i >= lo) {
                    const int ps = s_qp[i];
                    int best = i;
                    for (int k = i - 1; k >= lo && s_qp[k] == ps; --k)
                        if (!s_taken[k]) best = k;  // lowest id among equal p
                    cand = best;
                }
            }
            if (cand < 0) cand = lo;               // none fits: smallest p widens the least
            const int newW = max(W_A, s_qp[cand] + L);
            if (P.budget > 0 && (int64_t)(n_act + 1) * newW > P.budget) {
                if (n_act == 0) set_status(P.status, DLLM_ERR_CAPACITY);
                break;
            }
            s_taken[cand] = 1;
            s_adm[n_adm++] = cand;
            ++n_act;
            W_A = newW;
        }
        // 4. rows: freed rows ascending, then rows after the old end (every free row below `rows`
        //    was freed by this call); then fill holes from the tail
        int k = 0;
        for (int r = 0; r < cap && k < n_adm; ++r)
            if (s_row[r] < 0) s_row[r] = s_qid[s_adm[k++]];
        const int n_new = n_act;
        int h = 0, t = cap - 1;
        while (true) {
            while (h < n_new && s_row[h] >= 0) ++h;
            while (t >= n_new && s_row[t] < 0) --t;
            if (h >= n_new || t < n_new) break;
            s_row[h] = s_row[t];
            s_row[t] = -1;
            ++h;
            --t;
        }
        sh_nadm = n_adm;
        sh_nnew = n_new;
    }
    __syncthreads();
    const int n_adm = sh_nadm;
    const int n_new = sh_nnew;

    // 5. write the layout; open block 0 of admitted requests
    for (int r = tid; r < cap; r += kThreads) P.row_req[r] = s_row[r];
    for (int idx = tid; idx < n_adm * L; idx += kThreads) {
        const int a = idx / L, j = idx - (idx / L) * L;
        const int q = s_qid[s_adm[a]];
        if (j == 0) {
            R.state[q] = 1;
            R.b[q] = 0;
        }
        R.arena[block_start(R, q, 0, L) + j] = P.mask_id;
        R.blk_mask[(int64_t)q * L + j] = 1;
    }
    // 6. compact the queue in place, keeping order
    int keep_prefix = 0;
    {
        const int per = (qlen + kThreads - 1) / kThreads;
        const int i0 = min(qlen, tid * per), i1 = min(qlen, i0 + per);
        int loc = 0;
        for (int i = i0; i < i1; ++i) loc += !s_taken[i];
        const int lane = tid & 63, wave = tid >> 6;
        const int incl = wave_incl_scan(loc);
        __syncthreads();
        if (lane == 63) red[wave] = incl;
        __syncthreads();
        int off = 0;
        for (int w = 0; w < wave; ++w) off += red[w];
        keep_prefix = off + incl - loc;
        if (touch_queue)
            for (int i = i0; i < i1; ++i)
                if (!s_taken[i]) P.q_ids[keep_prefix++] = s_qid[i];
    }
    __syncthreads();
    // 7. meta (b of every active request is final now)
    int wl = 0;
    for (int r = tid; r < n_new; r += kThreads) {
        const int q = s_row[r];
        wl = max(wl, R.p[q] + (R.b[q] + 1) * L);
    }
    const int W_new = block_reduce_max(wl, red);
    if (tid == 0) {
        if (touch_queue) *P.q_len = qlen - n_adm;
        dllm_meta m;
        m.rows = n_new;
        m.W = W_new;
        m.n_evicted = n_evicted;
        m.n_admitted = n_adm;
        m.n_queued = touch_queue ? qlen - n_adm : sh_qlen;
        m.reserved = 0;
        m.cost = (int64_t)n_new * W_new;
        *P.meta = m;
    }
}

}  // namespace

extern "C" dllm_status dllm_compact(void *stream, int32_t rows, int32_t L, int32_t W, int32_t mask_id,
                                    int32_t eos_id, const int32_t *box_ids, const uint8_t *mask,
                                    const uint8_t *done, int32_t *row_req, int32_t rows_cap,
                                    const dllm_reqs *reqs, const dllm_queue *queue, int64_t budget,
                                    dllm_meta *meta, int32_t *status) {
    if (rows < 0) return fail(DLLM_ERR_ARG, "dllm_compact: rows < 0");
    if (rows > rows_cap) return fail(DLLM_ERR_ARG, "dllm_compact: rows=%d > rows_cap=%d", rows, rows_cap);
    if (rows_cap > DLLM_MAX_ROWS) return fail(DLLM_ERR_SHAPE, "dllm_compact: rows_cap=%d > %d", rows_cap, DLLM_MAX_ROWS);
    if (L < 1 || L > DLLM_MAX_L) return fail(DLLM_ERR_SHAPE, "dllm_compact: L=%d outside [1, %d]", L, DLLM_MAX_L);
    const int given = (box_ids != nullptr) + (mask != nullptr) + (done != nullptr);
    if (given != 0 && given != 3) return fail(DLLM_ERR_ARG, "dllm_compact: box_ids, mask, done must be all given or all NULL");
    if (given == 3 && rows > 0 && W < L) return fail(DLLM_ERR_SHAPE, "dllm_compact: W=%d < L=%d", W, L);
    if (!row_req || !reqs || !queue || !meta || !status) return fail(DLLM_ERR_ARG, "dllm_compact: null required pointer");
    if (!reqs->p || !reqs->K || !reqs->b || !reqs->state || !reqs->arena_off || !reqs->arena || !reqs->blk_mask ||
        reqs->n_req < 0)
        return fail(DLLM_ERR_ARG, "dllm_compact: incomplete request table");
    if (queue->cap < 0 || queue->cap > DLLM_MAX_QUEUE)
        return fail(DLLM_ERR_CAPACITY, "dllm_compact: queue cap %d outside [0, %d]", queue->cap, DLLM_MAX_QUEUE);
    if (!queue->len || (queue->cap > 0 && !queue->ids)) return fail(DLLM_ERR_ARG, "dllm_compact: queue pointers");
    if (rows_cap < 1) return fail(DLLM_ERR_ARG, "dllm_compact: rows_cap < 1");

    CompactParams P;
    P.rows = rows; P.L = L; P.W = W; P.mask_id = mask_id; P.eos_id = eos_id; P.rows_cap = rows_cap;
    P.box_ids = given ? box_ids : nullptr;
    P.mask = mask; P.done = done; P.row_req = row_req; P.R = *reqs;
    P.q_ids = queue->ids; P.q_len = queue->len; P.q_cap = queue->cap;
    P.budget = budget; P.meta = meta; P.status = status;
    const size_t lds = (size_t)rows_cap * 8 + (size_t)queue->cap * 8 + (size_t)rows_cap + (size_t)queue->cap + 16;
    int dev = 0, max_lds = 65536;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        max_lds = 65536;
    if (lds + 4096 > (size_t)max_lds)
        return fail(DLLM_ERR_CAPACITY, "dllm_compact: rows_cap=%d and queue cap=%d need %zu bytes of LDS (max %d)",
                    rows_cap, queue->cap, lds, max_lds);
    hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(kThreads), lds, (hipStream_t)stream, P);
    return check_hip(hipGetLastError(), "dllm_compact launch");
}
