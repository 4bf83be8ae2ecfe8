// dllm_step: one LowConfidence denoise step over a packed box, in a single launch.
//
// What is computed ([FDFO] = page "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」",
// [DiLaServe] = page "DiLaServe: High SLO Attainment Serving for Diffusion Language Models"):
//   [FDFO] §工程设计一 — step() reads the logits, updates input_ids by the LowConfidence rule
//   (unmask masked slots whose confidence exceeds the threshold, else the single most confident
//   one) and returns per-block done flags; [DiLaServe] §三 3.1 — the confidence is the softmax
//   probability of the predicted token; [FDFO] §工程设计二 — accept length is 0 or block_size.
//
// How (gfx950): the work is a streaming reduction over M masked slots x V logits, bound by HBM.
//   * Every vocabulary row is cut into NC fixed chunks of <= 64*kVPL 16-byte vectors.  The cut
//     depends on V only, so each slot's result is independent of the rest of the batch.
//   * One wavefront reduces one chunk: 64 lanes issue kVPL coalesced 16-byte loads each (1 KiB per
//     wave instruction), take a per-lane max, then sum exp2((x - max) * log2 e) with one v_exp per
//     element, then combine lanes with a fixed butterfly.  The partial (max, sum, first vector
//     holding the max) goes to the workspace.
//   * The M*NC chunks are split statically and evenly over all waves of the grid.  The wave that
//     completes a slot's last chunk (per-slot arrival counter) merges its NC partials in chunk
//     order and resolves the exact argmax from one 16-byte re-read; the wave that completes a
//     row's last slot (per-row counter) applies the unmask rule for the row.  Everything happens
//     in one launch; every workspace word is returned to zero by its last user, so the workspace
//     is all zeros between calls whatever the shapes.
//   * Each workgroup first builds an LDS bitmap of mask_in and a per-row prefix of masked counts,
//     which maps chunk indices to (row, slot).  mask_in is never written, so late workgroups see
//     the same mask; the new mask goes to mask_out.
//   * No MFMA: there is no contraction here.  Loads are non-temporal (each byte is read once).
#include "common.h"

namespace {

using namespace dllm;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kVPL = 8;                       // 16-byte vectors per lane per chunk
constexpr float kLog2e = 1.4426950408889634f;

struct StepParams {
    const char *logits;
    int64_t pos_stride_b, row_stride_b;       // strides in bytes
    int32_t rows, L, V, NV, NC, W;
    int32_t *ids;
    const uint8_t *mask_in;
    uint8_t *mask_out;
    const float *tau;
    const int32_t *p, *b;
    float *conf_out;
    int32_t *arg_out;
    uint8_t *done;
    int32_t *accept;
    float4 *partials;                         // [rows*L*NC] {max, sum, vector index, -}
    float *conf_ws;                           // [rows*L]
    int32_t *arg_ws;                          // [rows*L]
    int32_t *pos_cnt;                         // [rows*L] chunk arrivals
    int32_t *row_cnt;                         // [rows] slot arrivals
    int32_t *status;
};

// ---- bitmap helpers (LDS) --------------------------------------------------------------------
__device__ __forceinline__ uint64_t bits_at(const uint64_t *bm, int start, int n) {
    // n in [1, 64]; returns bits start .. start+n-1 in the low n bits
    const int wi = start >> 6, sh = start & 63;
    uint64_t w = bm[wi] >> sh;
    if (sh != 0 && sh + n > 64) w |= bm[wi + 1] << (64 - sh);
    return n == 64 ? w : (w & ((1ull << n) - 1));
}
__device__ __forceinline__ int count_row(const uint64_t *bm, int row, int L) {
    int c = 0;
    for (int off = 0; off < L; off += 64) c += __popcll(bits_at(bm, row * L + off, min(64, L - off)));
    return c;
}
// slot of the k-th (0-based) masked position of the row
__device__ __forceinline__ int select_in_row(const uint64_t *bm, int row, int L, int k) {
    for (int off = 0; off < L; off += 64) {
        uint64_t w = bits_at(bm, row * L + off, min(64, L - off));
        const int pc = __popcll(w);
        if (k < pc) {
            for (int t = 0; t < k; ++t) w &= w - 1;
            return off + __builtin_ctzll(w);
        }
        k -= pc;
    }
    return -1;
}

// ---- element access ----------------------------------------------------------------------------
template <bool BF16>
struct Fmt {
    static constexpr int E = BF16 ? 8 : 4;    // elements per 16-byte vector
    static constexpr int S = BF16 ? 2 : 4;    // bytes per element
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Load vector vi (E elements) of a row; elements at or beyond V read as -inf.  Full vectors of an
// aligned row use one 16-byte non-temporal load; the partial last vector and unaligned rows use
// element loads.
template <bool BF16, bool ALIGNED>
__device__ __forceinline__ void load_vec(const char *row, int vi, int V, float *x) {
    constexpr int E = Fmt<BF16>::E;
    const int e0 = vi * E;
    if (ALIGNED && e0 + E <= V) {
        const u32x4 u = __builtin_nontemporal_load((const u32x4 *)(row + (int64_t)vi * 16));
        if (BF16) {
            x[0] = bf16_lo(u[0]); x[1] = bf16_hi(u[0]); x[2] = bf16_lo(u[1]); x[3] = bf16_hi(u[1]);
            x[4] = bf16_lo(u[2]); x[5] = bf16_hi(u[2]); x[6] = bf16_lo(u[3]); x[7] = bf16_hi(u[3]);
        } else {
            x[0] = __uint_as_float(u[0]); x[1] = __uint_as_float(u[1]);
            x[2] = __uint_as_float(u[2]); x[3] = __uint_as_float(u[3]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int v = e0 + e;
            if (v < V) {
                if (BF16) x[e] = __uint_as_float((uint32_t)((const uint16_t *)row)[v] << 16);
                else x[e] = ((const float *)row)[v];
            } else {
                x[e] = -INFINITY;
            }
        }
    }
}

// Reduce vectors [vb, ve) of one row with the whole wave.  Returns, uniform over the wave:
// M = max, S = sum exp(x - M), vidx = lowest vector index holding M.
template <bool BF16, bool ALIGNED>
__device__ __forceinline__ void chunk_reduce(const char *row, int vb, int ve, int V, float &M, float &S,
                                             int &vidx) {
    constexpr int E = Fmt<BF16>::E;
    const int lane = lane_id();
    float x[kVPL][E];
#pragma unroll
    for (int k = 0; k < kVPL; ++k) {
        const int vi = vb + k * 64 + lane;
        if (vi < ve) {
            load_vec<BF16, ALIGNED>(row, vi, V, x[k]);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) x[k][e] = -INFINITY;
        }
    }
    // per-lane max and the first of this lane's vectors that holds it
    float m = -INFINITY;
    int kb = -1;
#pragma unroll
    for (int k = 0; k < kVPL; ++k) {
        float vm = x[k][0];
#pragma unroll
        for (int e = 1; e < E; ++e) vm = fmaxf(vm, x[k][e]);
        if (vm > m) { m = vm; kb = k; }
    }
    // per-lane sum of exp(x - m) = exp2(x*log2e - m*log2e)
    const float nml = (m == -INFINITY) ? 0.0f : -m * kLog2e;
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int k = 0; k < kVPL; ++k) {
#pragma unroll
        for (int e = 0; e < E; e += 2) {
            s0 += __builtin_amdgcn_exp2f(fmaf(x[k][e], kLog2e, nml));
            s1 += __builtin_amdgcn_exp2f(fmaf(x[k][e + 1], kLog2e, nml));
        }
    }
    const float sl = s0 + s1;
    // wave combine: common max, rescaled sums, lowest vector index at the max
    M = wave_max(m);
    const float scale = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m - M) * kLog2e);
    S = wave_sum(sl * scale);
    const int cand = (kb >= 0 && m == M) ? vb + kb * 64 + lane : 0x7FFFFFFF;
    vidx = wave_min(cand);
}

// Merge the NC chunk partials of slot (row, j) in chunk order; resolve the exact argmax.
template <bool BF16, bool ALIGNED>
__device__ void merge_slot(const StepParams &P, int row, int j) {
    constexpr int E = Fmt<BF16>::E;
    const int lane = lane_id();
    const int q = row * P.L + j;
    float4 *part = P.partials + (int64_t)q * P.NC;
    float Mr = -INFINITY, Sr = 0.0f;
    int vr = 0x7FFFFFFF;
    for (int base = 0; base < P.NC; base += 64) {
        const int c = base + lane;
        float mc = -INFINITY, sc = 0.0f;
        int vc = 0x7FFFFFFF;
        if (c < P.NC) {
            const float4 t = part[c];
            mc = t.x; sc = t.y; vc = __float_as_int(t.z);
            part[c] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);   // leave the workspace zeroed
        }
        const float Mb = wave_max(mc);
        const int vb = wave_min(mc == Mb ? vc : 0x7FFFFFFF);
        const float Sb = wave_sum(mc == -INFINITY ? 0.0f : sc * __builtin_amdgcn_exp2f((mc - Mb) * kLog2e));
        if (base == 0) {
            Mr = Mb; Sr = Sb; vr = vb;
        } else {
            const float Mn = fmaxf(Mr, Mb);
            Sr = Sr * __builtin_amdgcn_exp2f((Mr - Mn) * kLog2e) + Sb * __builtin_amdgcn_exp2f((Mb - Mn) * kLog2e);
            if (Mb > Mr) vr = vb;
            Mr = Mn;
        }
    }
    // exact index of the first maximum inside vector vr (vr is out of range only for non-finite
    // logits, which break the precondition; then no re-read is made and the argmax reads 0)
    int arg = 0;
    if (vr >= 0 && vr < P.NV) {
        const char *rowp = P.logits + (int64_t)row * P.row_stride_b + (int64_t)j * P.pos_stride_b;
        float x[E];
        load_vec<BF16, ALIGNED>(rowp, vr, P.V, x);
        int e_first = 0;
#pragma unroll
        for (int e = E - 1; e >= 0; --e)
            if (x[e] == Mr) e_first = e;
        arg = vr * E + e_first;
    }
    if (lane == 0) {
        P.conf_ws[q] = 1.0f / Sr;
        P.arg_ws[q] = arg;
        P.pos_cnt[q] = 0;
    }
}

// LowConfidence rule for one row whose masked slots are all scored.
__device__ void decide_row(const StepParams &P, const uint64_t *bm, int row, int nmasked) {
    const int lane = lane_id();
    const int L = P.L;
    const float tau = P.tau[row];
    bool any_above = false;
    float best_c = -INFINITY;
    int best_j = 0x7FFFFFFF;
    for (int g = 0; g < L; g += 64) {
        const int j = g + lane;
        const bool masked = j < L && ((bits_at(bm, row * L + g, min(64, L - g)) >> lane) & 1ull);
        const float c = masked ? P.conf_ws[row * L + j] : -INFINITY;
        any_above |= __ballot(masked && c > tau) != 0;
        const float gm = wave_max(c);
        const int gj = wave_min((masked && c == gm) ? j : 0x7FFFFFFF);
        if (gm > best_c) { best_c = gm; best_j = gj; }        // earlier groups win ties
    }
    int n_unmasked = 0;
    const int col0 = P.W - L;
    for (int g = 0; g < L; g += 64) {
        const int j = g + lane;
        const bool masked = j < L && ((bits_at(bm, row * L + g, min(64, L - g)) >> lane) & 1ull);
        const int q = row * L + j;
        const float c = masked ? P.conf_ws[q] : -1.0f;
        const bool u = masked && (any_above ? (c > tau) : (j == best_j));
        n_unmasked += __popcll(__ballot(u));
        if (j < L) {
            const int a = masked ? P.arg_ws[q] : -1;
            if (masked) {                                 // leave the workspace zeroed
                P.conf_ws[q] = 0.0f;
                P.arg_ws[q] = 0;
            }
            if (u) P.ids[(int64_t)row * P.W + col0 + j] = a;
            P.mask_out[q] = (masked && !u) ? 1 : 0;
            if (P.conf_out) P.conf_out[q] = c;
            if (P.arg_out) P.arg_out[q] = a;
        }
    }
    if (lane == 0) {
        const bool fin = nmasked == n_unmasked;
        P.done[row] = fin ? 1 : 0;
        P.accept[row] = fin ? L : 0;
        P.row_cnt[row] = 0;
    }
}

template <bool BF16, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void step_kernel(StepParams P) {
    extern __shared__ uint64_t lds[];
    __shared__ int wave_tot[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rows = P.rows, L = P.L;
    const int nbits = rows * L;
    const int nwords = (nbits + 63) >> 6;
    uint64_t *bm = lds;
    int *pre = (int *)(lds + nwords);          // [rows + 1] exclusive prefix of masked counts

    // 0a. bitmap of mask_in
    for (int w = wave; w < nwords; w += kWaves) {
        const int idx = w * 64 + lane;
        const bool m = idx < nbits && P.mask_in[idx] != 0;
        const uint64_t bits = __ballot(m);
        if (lane == 0) bm[w] = bits;
    }
    __syncthreads();
    // 0b. per-row counts -> exclusive prefix
    const int per = (rows + kThreads - 1) / kThreads;
    const int r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
    int local = 0;
    for (int r = r0; r < r1; ++r) local += count_row(bm, r, L);
    const int incl = wave_incl_scan(local);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int offset = 0;
    for (int w = 0; w < wave; ++w) offset += wave_tot[w];
    int run = offset + incl - local;
    for (int r = r0; r < r1; ++r) {
        pre[r] = run;
        run += count_row(bm, r, L);
    }
    if (tid == kThreads - 1) pre[rows] = offset + incl;
    __syncthreads();
    const int M = pre[rows];

    // 0c. rows with no masked slot, and the optional fit check
    for (int r = blockIdx.x * kThreads + tid; r < rows; r += gridDim.x * kThreads) {
        if (P.p && P.b && (int64_t)P.p[r] + ((int64_t)P.b[r] + 1) * L > P.W) set_status(P.status, DLLM_ERR_SHAPE);
        if (pre[r + 1] == pre[r]) {
            P.done[r] = 1;
            P.accept[r] = L;
            for (int j = 0; j < L; ++j) {
                P.mask_out[r * L + j] = 0;
                if (P.conf_out) P.conf_out[r * L + j] = -1.0f;
                if (P.arg_out) P.arg_out[r * L + j] = -1;
            }
        }
    }

    // 1. chunks: wave gw of Gw takes chunk indices [I*gw/Gw, I*(gw+1)/Gw) of I = M*NC
    const int NC = P.NC;
    const int64_t I = (int64_t)M * NC;
    const int64_t gw = (int64_t)blockIdx.x * kWaves + wave, Gw = (int64_t)gridDim.x * kWaves;
    const int64_t i0 = I * gw / Gw, i1 = I * (gw + 1) / Gw;
    int cur = -1, row = 0, j = 0, cnt = 0;
    const char *rowp = nullptr;
    for (int64_t i = i0; i <= i1; ++i) {
        const int qi = (i < i1) ? (int)(i / NC) : -2;
        if (qi != cur && cnt > 0) {
            // release this wave's partials of slot (row, j), count them in
            __threadfence();
            int old = 0;
            if (lane == 0) old = atomicAdd(&P.pos_cnt[row * L + j], cnt);
            old = __builtin_amdgcn_readfirstlane(old);
            if (old + cnt == NC) {
                __threadfence();
                merge_slot<BF16, ALIGNED>(P, row, j);
                __threadfence();
                int old2 = 0;
                if (lane == 0) old2 = atomicAdd(&P.row_cnt[row], 1);
                old2 = __builtin_amdgcn_readfirstlane(old2);
                const int need = pre[row + 1] - pre[row];
                if (old2 + 1 == need) {
                    __threadfence();
                    decide_row(P, bm, row, need);
                }
            }
            cnt = 0;
        }
        if (i == i1) break;
        if (qi != cur) {
            cur = qi;
            int lo = 0, hi = rows - 1;                  // last row with pre[row] <= qi
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pre[mid] <= qi) lo = mid; else hi = mid - 1;
            }
            row = lo;
            j = select_in_row(bm, row, L, qi - pre[row]);
            if (j < 0) {                                 // unreachable with a consistent bitmap
                set_status(P.status, DLLM_ERR_ARG);
                j = 0;
            }
            rowp = P.logits + (int64_t)row * P.row_stride_b + (int64_t)j * P.pos_stride_b;
        }
        const int c = (int)(i - (int64_t)qi * NC);
        const int vb = (int)((int64_t)c * P.NV / NC), ve = (int)((int64_t)(c + 1) * P.NV / NC);
        float m, s;
        int v;
        chunk_reduce<BF16, ALIGNED>(rowp, vb, ve, P.V, m, s, v);
        if (lane == 0) P.partials[(int64_t)(row * L + j) * NC + c] = make_float4(m, s, __int_as_float(v), 0.0f);
        ++cnt;
    }
}

struct Shape {
    int NV, NC;
    size_t partials_off, conf_off, arg_off, pcnt_off, rcnt_off, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline bool shape_of(int32_t rows, int32_t L, int32_t V, dllm_dtype dt, Shape &s) {
    if (rows < 0 || L < 1 || V < 1 || (dt != DLLM_FP32 && dt != DLLM_BF16)) return false;
    const int E = dt == DLLM_BF16 ? 8 : 4;
    const int64_t NV = ((int64_t)V + E - 1) / E;
    const int64_t NC = (NV + 64 * kVPL - 1) / (64 * kVPL);
    s.NV = (int)NV;
    s.NC = (int)NC;
    const size_t pos = (size_t)rows * (size_t)L;
    s.partials_off = 0;
    s.conf_off = align256(s.partials_off + pos * (size_t)NC * sizeof(float4));
    s.arg_off = align256(s.conf_off + pos * 4);
    s.pcnt_off = align256(s.arg_off + pos * 4);
    s.rcnt_off = align256(s.pcnt_off + pos * 4);
    s.total = align256(s.rcnt_off + (size_t)rows * 4);
    return true;
}

}  // namespace

extern "C" size_t dllm_step_workspace_bytes(int32_t rows, int32_t L, int32_t V, dllm_dtype dtype) {
    Shape s;
    if (!shape_of(rows, L, V, dtype, s)) return 0;
    return s.total;
}

extern "C" dllm_status dllm_step(void *stream, const void *logits, dllm_dtype dtype, int64_t pos_stride,
                                 int64_t row_stride, int32_t rows, int32_t L, int32_t V, int32_t *input_ids,
                                 int32_t W, const uint8_t *mask_in, uint8_t *mask_out, const float *threshold,
                                 const int32_t *p, const int32_t *b, float *conf, int32_t *argmax,
                                 uint8_t *done, int32_t *accept_len, void *workspace, size_t workspace_bytes,
                                 int32_t *status) {
    if (dtype != DLLM_FP32 && dtype != DLLM_BF16) return fail(DLLM_ERR_DTYPE, "dllm_step: unknown dtype %d", (int)dtype);
    if (rows < 0) return fail(DLLM_ERR_ARG, "dllm_step: rows < 0");
    if (L < 1 || L > DLLM_MAX_L) return fail(DLLM_ERR_SHAPE, "dllm_step: L=%d outside [1, %d]", L, DLLM_MAX_L);
    if (V < 1) return fail(DLLM_ERR_ARG, "dllm_step: V < 1");
    if (W < L) return fail(DLLM_ERR_SHAPE, "dllm_step: W=%d < L=%d", W, L);
    if (rows > DLLM_MAX_ROWS || (int64_t)rows * L > DLLM_MAX_POSITIONS)
        return fail(DLLM_ERR_SHAPE, "dllm_step: rows=%d, L=%d exceed the limits", rows, L);
    if (pos_stride < V || row_stride < (int64_t)L * pos_stride)
        return fail(DLLM_ERR_ARG, "dllm_step: strides too small (pos %lld, row %lld)", (long long)pos_stride,
                    (long long)row_stride);
    if ((p == nullptr) != (b == nullptr)) return fail(DLLM_ERR_ARG, "dllm_step: p and b must be both given or both NULL");
    if (rows == 0) return DLLM_OK;
    if (!logits || !input_ids || !mask_in || !mask_out || !threshold || !done || !accept_len || !workspace || !status)
        return fail(DLLM_ERR_ARG, "dllm_step: null required pointer");
    if (mask_in == mask_out) return fail(DLLM_ERR_ARG, "dllm_step: mask_out must not alias mask_in");
    Shape s;
    shape_of(rows, L, V, dtype, s);
    if (workspace_bytes < s.total)
        return fail(DLLM_ERR_ARG, "dllm_step: workspace %zu bytes < %zu needed", workspace_bytes, s.total);
    if (((uintptr_t)workspace & 15) != 0) return fail(DLLM_ERR_ARG, "dllm_step: workspace not 16-byte aligned");

    const int es = dtype == DLLM_BF16 ? 2 : 4;
    StepParams P;
    P.logits = (const char *)logits;
    P.pos_stride_b = pos_stride * es;
    P.row_stride_b = row_stride * es;
    P.rows = rows; P.L = L; P.V = V; P.NV = s.NV; P.NC = s.NC; P.W = W;
    P.ids = input_ids; P.mask_in = mask_in; P.mask_out = mask_out; P.tau = threshold;
    P.p = p; P.b = b; P.conf_out = conf; P.arg_out = argmax; P.done = done; P.accept = accept_len;
    char *ws = (char *)workspace;
    P.partials = (float4 *)(ws + s.partials_off);
    P.conf_ws = (float *)(ws + s.conf_off);
    P.arg_ws = (int32_t *)(ws + s.arg_off);
    P.pos_cnt = (int32_t *)(ws + s.pcnt_off);
    P.row_cnt = (int32_t *)(ws + s.rcnt_off);
    P.status = status;

    const bool aligned = ((uintptr_t)logits & 15) == 0 && (P.pos_stride_b & 15) == 0 && (P.row_stride_b & 15) == 0;
    // grid: enough waves for every chunk of a fully masked box, at most 4 workgroups per CU
    const int64_t max_chunks = (int64_t)rows * L * s.NC;
    int64_t grid = (max_chunks + kWaves - 1) / kWaves;
    const int64_t cap = (int64_t)cu_count() * 4;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    const int nwords = (rows * L + 63) / 64;
    const size_t lds = (size_t)nwords * 8 + (size_t)(rows + 1) * 4;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == DLLM_BF16) {
        if (aligned) hipLaunchKernelGGL((step_kernel<true, true>), dim3((unsigned)grid), dim3(kThreads), lds, st, P);
        else hipLaunchKernelGGL((step_kernel<true, false>), dim3((unsigned)grid), dim3(kThreads), lds, st, P);
    } else {
        if (aligned) hipLaunchKernelGGL((step_kernel<false, true>), dim3((unsigned)grid), dim3(kThreads), lds, st, P);
        else hipLaunchKernelGGL((step_kernel<false, false>), dim3((unsigned)grid), dim3(kThreads), lds, st, P);
    }
    return check_hip(hipGetLastError(), "dllm_step launch");
}
