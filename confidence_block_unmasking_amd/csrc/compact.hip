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
// One workgroup of 1024 threads.  The kernel is latency-bound (kilobytes of data, a chain of
// dependent reads), so it is laid out to pay few memory round trips: the request fields of every
// row and every queue entry are loaded once, up front (the queue ids speculatively up to the queue
// capacity, so they need not wait for the queue length), and all later phases work from registers
// and LDS.  The scatter of the finished step, the commit and the fresh-block fill are one pass that
// writes every arena and mask element once.  The greedy admission is inherently sequential (each
// choice changes the box width) and runs on one thread over LDS copies of the queue's prompt
// lengths, with a binary search for the best fit.  The queue is compacted in place (in order) with a
// parallel prefix scan.
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

constexpr int kRowsPerThread = DLLM_MAX_ROWS / kThreads;   // rows owned by one thread (registers)
constexpr int kQPerThread = DLLM_MAX_QUEUE / kThreads;      // queue entries loaded by one thread

// Row actions decided in phase 2 (s_act).
constexpr uint8_t kKeep = 0;      // unfinished block: scatter it back, keep the row
constexpr uint8_t kAdvance = 1;   // finished, blocks left: commit, then a fresh masked block
constexpr uint8_t kEvict = 2;     // finished, last block (or end of sequence): commit, free the row
constexpr uint8_t kNone = 3;      // no (valid) request in this row

__global__ __launch_bounds__(kThreads) void compact_kernel(CompactParams P) {
    extern __shared__ int64_t lds64[];
    __shared__ int red3[kWaves][3];
    __shared__ int sh_qlen, sh_bad, sh_badid;
    const int tid = threadIdx.x;
    const int rows = P.rows, L = P.L, cap = P.rows_cap, qcap = P.q_cap;
    const dllm_reqs &R = P.R;
    int64_t *s_old = lds64;                      // [cap]   arena start of the row's current block
    int32_t *s_row = (int32_t *)(s_old + cap);   // [cap]   row -> request (-1 free); the new layout
    int32_t *s_q0 = s_row + cap;                 // [cap]   row -> request on entry (read by the scatter
                                                 //         while wave 0 rewrites s_row)
    int32_t *s_adm = s_q0 + cap;                 // [cap]   admitted queue indices, in order
    int32_t *s_qp = s_adm + cap;                 // [qcap]  prompt length of queue entries
    int32_t *s_qid = s_qp + qcap;                // [qcap]  queue ids
    uint8_t *s_act = (uint8_t *)(s_qid + qcap);  // [cap]   row action
    uint8_t *s_taken = s_act + cap;              // [qcap]

    // 1. every load that does not depend on another one: queue length, the rows' request ids and
    //    done flags, the queue ids (up to its capacity); then the request fields they point to
    fetch_args(P.rows, P.L, P.W, P.mask_id, P.eos_id, P.rows_cap, P.box_ids, P.mask, P.done, P.row_req, R.n_req, R.p,
               R.K, R.b, R.state, R.arena_off, R.arena, R.blk_mask, P.q_ids, P.q_len, P.q_cap, P.budget, P.meta,
               P.status);
    int qlen_raw = 0;
    if (tid == 0) qlen_raw = __builtin_nontemporal_load(P.q_len);   // a vector load: no wait until used
    int rq[kRowsPerThread], rdone[kRowsPerThread];
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
        const int r = tid + k * kThreads;
        rq[k] = r < rows ? P.row_req[r] : -1;
        rdone[k] = (r < rows && P.box_ids) ? P.done[r] : 0;
    }
    int qi[kQPerThread];
#pragma unroll
    for (int k = 0; k < kQPerThread; ++k) {
        const int i = tid + k * kThreads;
        qi[k] = i < qcap ? P.q_ids[i] : -1;
    }
    int rp[kRowsPerThread], rb[kRowsPerThread], rK[kRowsPerThread], rst[kRowsPerThread];
    int64_t roff[kRowsPerThread];
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
        const int q = rq[k];
        const bool in = q >= 0 && q < R.n_req;
        rp[k] = in ? R.p[q] : 0;
        rb[k] = in ? R.b[q] : 0;
        rK[k] = in ? R.K[q] : 0;
        rst[k] = in ? R.state[q] : -1;
        roff[k] = in ? R.arena_off[q] : 0;
    }
    int qp[kQPerThread];
    bool qok[kQPerThread];
#pragma unroll
    for (int k = 0; k < kQPerThread; ++k) {
        const int id = qi[k];
        const bool in = id >= 0 && id < R.n_req;
        qp[k] = in ? R.p[id] : 0;
        qok[k] = in && R.state[id] == 0 && R.K[id] >= 1;
    }
    if (tid == 0) {
        sh_bad = (qlen_raw < 0 || qlen_raw > qcap);
        sh_qlen = sh_bad ? 0 : qlen_raw;
        sh_badid = 0;
        if (sh_bad) set_status(P.status, DLLM_ERR_CAPACITY);
    }
    __syncthreads();
    const int qlen0 = sh_qlen;

    // 2. validate; per row: its action and its blocks' arena starts
    int ev = 0, wloc = 0, nloc = 0;
#pragma unroll
    for (int k = 0; k < kRowsPerThread; ++k) {
        const int r = tid + k * kThreads;
        if (r >= cap) continue;
        int q = rq[k];
        if (r < rows && (q < 0 || q >= R.n_req || rst[k] != 1 || rb[k] < 0 || rb[k] >= rK[k])) {
            set_status(P.status, DLLM_ERR_ARG);
            q = -1;
        }
        uint8_t act = q < 0 ? kNone : kKeep;
        int b = rb[k];
        if (q >= 0 && P.box_ids && rdone[k]) {
            bool eos = false;
            if (P.eos_id >= 0)
                for (int j = 0; j < L; ++j) eos |= P.box_ids[(int64_t)r * P.W + (P.W - L) + j] == P.eos_id;
            act = (b + 1 >= rK[k] || eos) ? kEvict : kAdvance;
            R.b[q] = b + 1;
            if (act == kEvict) {
                R.state[q] = 2;
                ++ev;
            } else {
                ++b;
            }
        }
        s_old[r] = roff[k] + rp[k] + (int64_t)rb[k] * L;
        s_q0[r] = q;
        s_act[r] = act;
        s_row[r] = (act == kNone || act == kEvict) ? -1 : q;
        if (act == kKeep || act == kAdvance) {
            wloc = max(wloc, rp[k] + (b + 1) * L);
            ++nloc;
        }
    }
#pragma unroll
    for (int k = 0; k < kQPerThread; ++k) {
        const int i = tid + k * kThreads;
        if (i < qlen0) {
            s_qid[i] = qi[k];
            s_qp[i] = qok[k] ? qp[k] : 0;
            s_taken[i] = 0;
            if (!qok[k]) sh_badid = 1;
        }
    }
    {   // this wave's part of the counts wave 0 needs; one barrier publishes them with phase 2
        const int e = wave_sum_i(ev), wm = wave_max_i(wloc), n = wave_sum_i(nloc);
        if ((tid & 63) == 0) { red3[tid >> 6][0] = e; red3[tid >> 6][1] = wm; red3[tid >> 6][2] = n; }
    }
    __syncthreads();
    // a queue holding an invalid or non-queued id is left untouched and admits nothing
    const int qlen = sh_badid ? 0 : qlen0;
    const bool touch_queue = !sh_bad && !sh_badid;
    const int wave = tid >> 6, lane = tid & 63;

    // 3. waves 1..: the step's block back to its request, in one pass: the finished block (or the
    //    unfinished one with its mask) goes to the arena; an advancing request's next block opens
    //    fully masked.  Then these waves are done.
    if (wave != 0) {
        if (P.box_ids) {
            for (int idx = tid - 64; idx < rows * L; idx += kThreads - 64) {
                const int r = idx / L, j = idx - (idx / L) * L;
                const uint8_t act = s_act[r];
                if (act == kNone) continue;
                const int q = s_q0[r];
                const int32_t tok = P.box_ids[(int64_t)r * P.W + (P.W - L) + j];
                const uint8_t m = P.mask[(int64_t)r * L + j];
                const int64_t old = s_old[r];
                R.arena[old + j] = tok;
                if (act == kAdvance) {
                    R.arena[old + L + j] = P.mask_id;
                    R.blk_mask[(int64_t)q * L + j] = 1;
                } else {
                    // kept, or evicted (its last block committed, its all-zero mask stored as well)
                    R.blk_mask[(int64_t)q * L + j] = m;
                }
            }
        }
        return;
    }

    // 4.. wave 0 alone from here: every step below is wave-synchronous (no workgroup barrier).  LDS
    //    accesses of one wave take effect in program order, so lanes see each other's writes.
    int n_evicted = 0, W_A0 = 0, n_act0 = 0;
    for (int w = 0; w < kWaves; ++w) {
        n_evicted += red3[w][0];
        W_A0 = max(W_A0, red3[w][1]);
        n_act0 += red3[w][2];
    }
    if (sh_badid && lane == 0) set_status(P.status, DLLM_ERR_ARG);

    // 4. admission (sequential, lane 0)
    int n_adm = 0, n_new = n_act0, W_new = W_A0;
    if (lane == 0) {
        int n_act = n_act0, W_A = W_A0, lo = 0;
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
        n_new = n_act;
        W_new = W_A;                               // widest row of the new active set
    }
    n_adm = __builtin_amdgcn_readfirstlane(n_adm);
    n_new = __builtin_amdgcn_readfirstlane(n_new);
    W_new = __builtin_amdgcn_readfirstlane(W_new);

    // 5. open block 0 of admitted requests
    for (int idx = lane; idx < n_adm * L; idx += 64) {
        const int a = idx / L, j = idx - (idx / L) * L;
        const int ai = s_adm[a];
        const int q = s_qid[ai];
        if (j == 0) {
            R.state[q] = 1;
            R.b[q] = 0;
        }
        R.arena[R.arena_off[q] + s_qp[ai] + j] = P.mask_id;
        R.blk_mask[(int64_t)q * L + j] = 1;
    }

    // 6. rows.  Lane l looks after rows l*per .. l*per + per - 1.
    //    (a) the k-th admitted request takes the k-th free row in ascending order: freed rows
    //    first, then rows past the old end (every free row below `rows` was freed by this call);
    //    (b) the rows left free below n_new (holes, ascending) take the requests of the occupied
    //    rows at or above n_new (movers, descending); survivors otherwise stay where they are.
    {
        const int per = (cap + 63) / 64;
        const int r0 = min(cap, lane * per), r1 = min(cap, r0 + per);
        int nf = 0;
        for (int r = r0; r < r1; ++r) nf += s_row[r] < 0;
        int ef = wave_incl_scan(nf) - nf;
        for (int r = r0; r < r1; ++r) {
            if (s_row[r] < 0) {
                if (ef < n_adm) s_row[r] = s_qid[s_adm[ef]];
                ++ef;
            }
        }
        int nh = 0, nm = 0;
        for (int r = r0; r < r1; ++r) {
            const bool occ = s_row[r] >= 0;
            nh += (r < n_new && !occ);
            nm += (r >= n_new && occ);
        }
        int eh = wave_incl_scan(nh) - nh;
        const int im = wave_incl_scan(nm);
        const int tm = __builtin_amdgcn_readlane(im, 63);
        int em = im - nm;
        int *s_mv = s_adm;                         // the admitted list is placed: movers by rank
        for (int r = r0; r < r1; ++r)
            if (r >= n_new && s_row[r] >= 0) s_mv[tm - 1 - em++] = r;   // descending rank
        for (int r = r0; r < r1; ++r)
            if (r < n_new && s_row[r] < 0) s_row[r] = s_row[s_mv[eh++]];   // holes < n_new <= movers
        for (int r = r0; r < r1; ++r)
            if (r >= n_new && s_row[r] >= 0) s_row[r] = -1;
        for (int r = r0; r < r1; ++r) P.row_req[r] = s_row[r];
    }

    // 7. compact the queue in place, keeping order (lane l: entries l*per .. l*per + per - 1)
    {
        const int per = (qlen + 63) / 64;
        const int i0 = min(qlen, lane * per), i1 = min(qlen, i0 + per);
        int loc = 0;
        for (int i = i0; i < i1; ++i) loc += !s_taken[i];
        int keep = wave_incl_scan(loc) - loc;
        if (touch_queue)
            for (int i = i0; i < i1; ++i)
                if (!s_taken[i]) P.q_ids[keep++] = s_qid[i];
    }
    // 8. meta
    if (lane == 0) {
        if (touch_queue) *P.q_len = qlen - n_adm;
        dllm_meta m;
        m.rows = n_new;
        m.W = n_new > 0 ? W_new : 0;
        m.n_evicted = n_evicted;
        m.n_admitted = n_adm;
        m.n_queued = touch_queue ? qlen - n_adm : sh_qlen;
        m.reserved = 0;
        m.cost = (int64_t)n_new * m.W;
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
    const size_t lds = (size_t)rows_cap * 21 + (size_t)queue->cap * 9 + 16;
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
