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
//      over the workgroups, one workgroup per compute unit holding all of that unit's waves.
//      Inside a workgroup the waves take chunks one at a time from an LDS counter: the sequencer
//      favours older waves when they compete for the memory pipe, so a fixed split per wave
//      leaves the young ones finishing last, while a shared counter lets every wave of the unit
//      finish within about one chunk of the others.  (Global atomics would do the same across
//      units but cost a memory round trip each and serialise on one address.)
//      One wavefront reduces one chunk: 64 lanes issue kVPL coalesced 16-byte non-temporal loads
//      each (1 KiB per wave instruction), the next chunk's loads go out before this chunk's
//      arithmetic, each element costs one FMA and one v_exp (sum of exp2(x*log2e - max*log2e)),
//      and lanes combine through DPP.  The chunk partial (max, sum, first element index at the
//      max) stays in a lane register until the wave has 64 of them or runs out of chunks, then
//      they leave in one store: a store between the loads of consecutive chunks would hold back
//      every later load until it completed.
//   2. decide_kernel, one workgroup per row, merges each masked slot's NC partials in chunk order
//      (a fixed tree, so the bits are reproducible), and applies the unmask rule to the row.
//   The launch boundary is what makes the partials of kernel 1 visible to kernel 2.  A one-launch
//   variant (the last workgroup to finish a row decides it) needs a device-wide release and
//   acquire per workgroup; with device-coherent stores and loads standing in for those fences it
//   read stale partials on this part, and its in-kernel decision was no faster than the second
//   launch.  No MFMA: there is no contraction here.
#include "common.h"

namespace {

using namespace dllm;

#ifndef DLLM_STEP_VPL
#define DLLM_STEP_VPL 8
#endif
#ifndef DLLM_STEP_WAVES
#define DLLM_STEP_WAVES 8
#endif

constexpr int kWaves = DLLM_STEP_WAVES;       // waves per scoring workgroup (one workgroup per CU)
constexpr int kThreads = 64 * kWaves;
constexpr int kVPL = DLLM_STEP_VPL;           // 16-byte vectors per lane per chunk
constexpr int kCH = 64 * kVPL;                // vectors per chunk
constexpr int kTile = kThreads * 16;          // mask bytes per prologue pass (16 per thread)
constexpr int kDecideThreads = 256;
constexpr int kDecideWaves = kDecideThreads / 64;
constexpr int kGroup = 8;                     // slots whose partials one decide wave loads at once
constexpr float kLog2e = 1.4426950408889634f;

struct StepParams {
    const char *logits;
    int64_t pos_stride_b, row_stride_b;       // strides in bytes
    int32_t rows, L, V, NV, NC, W;
    int32_t *ids;
    const uint8_t *mask_in;
    uint8_t *mask_out;
    const float *tau;
    const int32_t *p, *b;                     // never NULL here (see check_fit)
    int32_t check_fit;                        // p and b were given: check p + (b+1)L <= W
    int32_t S;                                // quota rule: diffusion steps per block (0: threshold rule)
    float *conf_out;
    int32_t *arg_out;
    uint8_t *done;
    int32_t *accept;
    float4 *partials;                         // [rows*L*NC] {max, sum, element index, -}
    int32_t *status;
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ---- wave reductions: DPP within each row of 16 lanes, then the four rows through readlane ----
// A fixed network, so the result's bits do not depend on timing; every lane gets the result.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;    // row_half_mirror
constexpr int kRowMirror = 0x140;     // row_mirror
__device__ __forceinline__ float rlf(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

__device__ __forceinline__ float red_max(float v) {
    v = fmaxf(v, dppf<kQuadSwap1>(v));
    v = fmaxf(v, dppf<kQuadSwap2>(v));
    v = fmaxf(v, dppf<kHalfMirror>(v));
    v = fmaxf(v, dppf<kRowMirror>(v));
    return fmaxf(fmaxf(rlf(v, 0), rlf(v, 16)), fmaxf(rlf(v, 32), rlf(v, 48)));
}
__device__ __forceinline__ float red_sum(float v) {
    v += dppf<kQuadSwap1>(v);
    v += dppf<kQuadSwap2>(v);
    v += dppf<kHalfMirror>(v);
    v += dppf<kRowMirror>(v);
    return (rlf(v, 0) + rlf(v, 16)) + (rlf(v, 32) + rlf(v, 48));
}
__device__ __forceinline__ int red_min(int v) {
    v = min(v, dppi<kQuadSwap1>(v));
    v = min(v, dppi<kQuadSwap2>(v));
    v = min(v, dppi<kHalfMirror>(v));
    v = min(v, dppi<kRowMirror>(v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// ---- element access ----------------------------------------------------------------------------
template <bool BF16>
struct Fmt {
    static constexpr int E = BF16 ? 8 : 4;    // elements per 16-byte vector
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4 &u, float *x) {
    if (BF16) {
        x[0] = bf16_lo(u[0]); x[1] = bf16_hi(u[0]); x[2] = bf16_lo(u[1]); x[3] = bf16_hi(u[1]);
        x[4] = bf16_lo(u[2]); x[5] = bf16_hi(u[2]); x[6] = bf16_lo(u[3]); x[7] = bf16_hi(u[3]);
    } else {
        x[0] = __uint_as_float(u[0]); x[1] = __uint_as_float(u[1]);
        x[2] = __uint_as_float(u[2]); x[3] = __uint_as_float(u[3]);
    }
}

// One vector (E elements) by element loads; elements at or beyond V read as -inf.
template <bool BF16>
__device__ __forceinline__ void load_vec_elems(const char *row, int vi, int V, float *x) {
    constexpr int E = Fmt<BF16>::E;
    const int e0 = vi * E;
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

struct Part {
    float m, s;   // max and sum of exp(x - max) over the chunk
    int v;        // lowest element index (within the row) holding the max
};

// Chunk reduction over values already in registers: x[k][e] is element (vb + k*64 + lane)*E + e
// of the row; -inf marks padding.  Lane-local max and sum exp(x - max), then the wave combine.
// The lowest vector holding the max comes from a DPP min; its owner lane and slot k are then
// wave-uniform, so that one vector's E values are read with readlane and the first element equal
// to the max gives the exact index without going back to memory.
template <int E>
__device__ __forceinline__ Part reduce_lanes(float (&x)[kVPL][E], int vb) {
    const int lane = lane_id();
    float m = -INFINITY;
    int kb = -1;
#pragma unroll
    for (int k = 0; k < kVPL; ++k) {
        float vm = x[k][0];
#pragma unroll
        for (int e = 1; e < E; ++e) vm = fmaxf(vm, x[k][e]);
        if (vm > m) { m = vm; kb = k; }
    }
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
    Part r;
    r.m = red_max(m);
    const float scale = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m - r.m) * kLog2e);
    r.s = red_sum((s0 + s1) * scale);
    const int vmin = red_min((kb >= 0 && m == r.m) ? kb * 64 + lane : 0x7FFFFFFF);   // chunk-relative
    int elem = 0x7FFFFFFF;
    if (vmin != 0x7FFFFFFF) {
        const int kw = vmin >> 6, lw = vmin & 63;                   // wave-uniform
        int ef = E;
#pragma unroll
        for (int k = 0; k < kVPL; ++k) {
            if (k == kw) {
#pragma unroll
                for (int e = E - 1; e >= 0; --e)
                    if (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[k][e]), lw)) == r.m) ef = e;
            }
        }
        elem = (vb + vmin) * E + ef;
    }
    r.v = elem;
    return r;
}

// Aligned rows: the kVPL 16-byte loads of chunk [vb, vb + n) for this lane, issued back to back.
// Addresses past a short chunk's end are clamped to its last vector; convert() turns those
// values into -inf.
__device__ __forceinline__ void issue(u32x4 (&raw)[kVPL], const char *row, int vb, int n) {
    const int lane = lane_id();
    const u32x4 *base = (const u32x4 *)row + vb;
    if (n == kCH) {
#pragma unroll
        for (int k = 0; k < kVPL; ++k) raw[k] = __builtin_nontemporal_load(base + k * 64 + lane);
    } else {
#pragma unroll
        for (int k = 0; k < kVPL; ++k) raw[k] = __builtin_nontemporal_load(base + min(k * 64 + lane, n - 1));
    }
}
template <bool BF16>
__device__ __forceinline__ void convert(const u32x4 (&raw)[kVPL], float (&x)[kVPL][Fmt<BF16>::E], int n) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 0; k < kVPL; ++k) {
        unpack<BF16>(raw[k], x[k]);
        if (n < kCH && k * 64 + lane >= n) {
#pragma unroll
            for (int e = 0; e < Fmt<BF16>::E; ++e) x[k][e] = -INFINITY;
        }
    }
}
// Unaligned rows (or V not a multiple of the vector width): element loads straight into x.
template <bool BF16>
__device__ __forceinline__ void load_elems(float (&x)[kVPL][Fmt<BF16>::E], const char *row, int vb, int n, int V) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 0; k < kVPL; ++k) {
        if (k * 64 + lane < n) {
            load_vec_elems<BF16>(row, vb + k * 64 + lane, V, x[k]);
        } else {
#pragma unroll
            for (int e = 0; e < Fmt<BF16>::E; ++e) x[k][e] = -INFINITY;
        }
    }
}

// 16 mask bytes starting at slot s0 (bytes at or past S read as unmasked) -> bit k set when
// byte s0 + k is nonzero.
__device__ __forceinline__ uint32_t mask_bits16(const uint8_t *mask, int s0, int S) {
    uint32_t bits = 0;
    if (s0 + 16 <= S && (((uintptr_t)(mask + s0)) & 15) == 0) {
        const u32x4 w = *(const u32x4 *)(mask + s0);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            // high bit of each byte lane set iff the byte is nonzero
            const uint32_t nz = (((w[d] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w[d]) & 0x80808080u;
            bits |= ((nz >> 7) & 1u) << (4 * d) | ((nz >> 15) & 1u) << (4 * d + 1) |
                    ((nz >> 23) & 1u) << (4 * d + 2) | ((nz >> 31) & 1u) << (4 * d + 3);
        }
    } else if (s0 < S) {
        // unaligned or ragged: 16 byte loads from clamped addresses, all issued before any use
        uint32_t v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) v[k] = mask[min(s0 + k, S - 1)];
#pragma unroll
        for (int k = 0; k < 16; ++k) bits |= (uint32_t)((v[k] != 0) & (s0 + k < S)) << k;
    }
    return bits;
}

// Sum of v over the workgroup (every thread gets it).  `tmp` holds kWaves ints; the caller puts a
// barrier between two uses of the same `tmp`.
__device__ __forceinline__ int block_sum(int v, int *tmp) {
    const int s = wave_sum_i(v);
    if (lane_id() == 0) tmp[threadIdx.x >> 6] = s;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += tmp[w];
    return t;
}

// Kernel 1: score every chunk of every masked slot.
template <bool BF16, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void score_kernel(StepParams P, int win) {
    extern __shared__ int64_t s_off[];         // [win] byte offset of the window's logits rows
    int *s_id = (int *)(s_off + win);          // [win] slot index (row*L + j) of the same
    __shared__ int s_tmp[2][kWaves];
    __shared__ int s_next;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int L = P.L, S = P.rows * L, NC = P.NC;
    const int ntiles = (S + kTile - 1) / kTile;

    // 0. Masked slots are numbered in slot order (slot = row*L + j).  Count them, then list, in
    //    LDS, those whose chunks fall in this workgroup's share.  Thread tid covers slots
    //    tid*16 .. tid*16+15 of each tile of kTile slots.
    const uint32_t mb0 = mask_bits16(P.mask_in, tid * 16, S);
    int c0 = __popc(mb0);
    const int incl0 = wave_incl_scan(c0);
    if (lane == 63) s_tmp[0][wave] = incl0;
    int more_cnt = 0;                          // masked slots in tiles 1.. (several tiles only)
    for (int k = 1; k < ntiles; ++k) more_cnt += __popc(mask_bits16(P.mask_in, k * kTile + tid * 16, S));
    __syncthreads();
    int off0 = 0, tot0 = 0;                    // tile 0: masked slots before this wave, in all
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int v = s_tmp[0][w];
        off0 += w < wave ? v : 0;
        tot0 += v;
    }
    int M = tot0;
    if (ntiles > 1) M += block_sum(more_cnt, s_tmp[1]);
    M = uni(M);
    // share of workgroup g: I/G chunks, the first I%G workgroups one more (scalar arithmetic)
    const int I = M * NC;                      // chunk t is chunk t % NC of masked slot t / NC
    const int G = gridDim.x, g = blockIdx.x;
    const int per = I / G, rem = I - per * G;
    const int t0 = g * per + min(g, rem), t1 = t0 + per + (g < rem ? 1 : 0);
    if (t0 >= t1) return;                      // uniform over the workgroup
    const int q_lo = t0 / NC, q_hi = (t1 - 1) / NC;
    // list masked numbers q_lo..q_hi; qq = masked number of the first masked slot among mb's 16
    auto extract = [&](uint32_t mb, int qq, int s0) {
        const int c = __popc(mb);
        if (c == 0 || qq > q_hi || qq + c <= q_lo) return;
        for (; qq < q_lo; ++qq) mb &= mb - 1;
        int r = s0 / L, jb = s0 - r * L;
        int prev = 0;
        while (mb != 0 && qq <= q_hi) {
            const int bit = __builtin_ctz(mb);
            mb &= mb - 1;
            jb += bit - prev;
            prev = bit;
            while (jb >= L) { jb -= L; ++r; }
            s_off[qq - q_lo] = (int64_t)r * P.row_stride_b + (int64_t)jb * P.pos_stride_b;
            s_id[qq - q_lo] = r * L + jb;
            ++qq;
        }
    };
    extract(mb0, off0 + incl0 - c0, tid * 16);
    int base = tot0;
    for (int k = 1; k < ntiles && base <= q_hi; ++k) {
        const uint32_t mb = mask_bits16(P.mask_in, k * kTile + tid * 16, S);
        const int c = __popc(mb);
        const int incl = wave_incl_scan(c);
        __syncthreads();                       // the previous user of s_tmp[1] is done
        if (lane == 63) s_tmp[1][wave] = incl;
        __syncthreads();
        int off = base, tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int v = s_tmp[1][w];
            off += w < wave ? v : 0;
            tot += v;
        }
        extract(mb, off + incl - c, k * kTile + tid * 16);
        base += tot;
    }
    if (tid == 0) s_next = t0 + kWaves;
    __syncthreads();

    // 1. Chunks.  Wave w starts with chunk t0 + w, then takes the next untaken one from s_next.
    //    Which wave scores a chunk never changes the chunk's result.
    int t = t0 + wave;
    if (t >= t1) return;                       // no barrier follows
    constexpr int E = Fmt<BF16>::E;
    // lane k holds the wave's k-th pending chunk partial
    float pk_m = 0.0f, pk_s = 0.0f;
    int pk_v = 0, pk_at = 0;
    int nbuf = 0;
    int q = uni(t / NC), c = t - q * NC;
    const char *rowp = P.logits + s_off[q - q_lo];
    int slot = uni(s_id[q - q_lo]);
    u32x4 raw[kVPL];
    if (ALIGNED) issue(raw, rowp, c * kCH, min(kCH, P.NV - c * kCH));
    while (true) {
        int tn = 0;
        if (lane == 0) tn = atomicAdd(&s_next, 1);
        tn = uni(tn);
        const int vb = c * kCH;
        const int n = min(kCH, P.NV - vb);
        float x[kVPL][E];
        if (ALIGNED) convert<BF16>(raw, x, n);
        else load_elems<BF16>(x, rowp, vb, n, P.V);
        const int this_at = slot * NC + c;
        // the next chunk's loads go out before this chunk's math
        const bool more = tn < t1;
        int qn = q, cn = 0;
        if (more) {
            qn = uni(tn / NC);
            cn = tn - qn * NC;
            if (qn != q) {
                rowp = P.logits + s_off[qn - q_lo];
                slot = uni(s_id[qn - q_lo]);
            }
            if (ALIGNED) issue(raw, rowp, cn * kCH, min(kCH, P.NV - cn * kCH));
        }
        const Part pr = reduce_lanes<E>(x, vb);
        if (lane == nbuf) {
            pk_m = pr.m;
            pk_s = pr.s;
            pk_v = pr.v;
            pk_at = this_at;
        }
        if (++nbuf == 64 || !more) {
            if (lane < nbuf) P.partials[pk_at] = make_float4(pk_m, pk_s, __int_as_float(pk_v), 0.0f);
            nbuf = 0;
        }
        if (!more) break;
        q = qn;
        c = cn;
    }
}

// Merge of one slot's partials for chunks [base, base + 64) held one per lane: max over lanes,
// lowest element index at that max, sum rescaled to that max.  A fixed network (reproducible).
__device__ __forceinline__ void merge_lanes(const float4 &t, bool valid, float &Mb, float &Sb, int &vb) {
    const float mc = valid ? t.x : -INFINITY;
    const float sc = valid ? t.y : 0.0f;
    const int vc = valid ? __float_as_int(t.z) : 0x7FFFFFFF;
    Mb = red_max(mc);
    vb = red_min(mc == Mb ? vc : 0x7FFFFFFF);
    Sb = red_sum(mc == -INFINITY ? 0.0f : sc * __builtin_amdgcn_exp2f((mc - Mb) * kLog2e));
}

// Quota of the step at which m of a block's L slots are still masked, for S steps per block:
// step t takes floor(L/S) tokens and the first L mod S steps one more ([BlockServe] §II-E); the
// step is the last one whose running total of unmasked tokens P_t = t*base + min(t, rem) does
// not exceed L - m; past step S every remaining slot goes.
__device__ __forceinline__ int quota_for_remaining(int L, int S, int m) {
    if (m <= 0) return 0;
    const int base = L / S, rem = L - base * S, u = L - m;
    int t;
    if (u < rem * (base + 1)) t = u / (base + 1);
    else t = base > 0 ? rem + (u - rem * (base + 1)) / base : S;
    if (t >= S) return m;
    return min(m, base + (t < rem ? 1 : 0));
}

// Kernel 2: one workgroup per row.  Merge each masked slot's NC partials in chunk order (lanes =
// chunks, a fixed DPP tree, then blocks of 64 chunks in order), then the row's rule: LowConfidence
// (QUOTA false) or the fixed per-step quota (QUOTA true: the k most confident masked slots, k from
// quota_for_remaining, ties to the lowest j).
// Each wave loads the partials and mask bytes of kGroup slots before reducing any of them, so a
// row costs about one memory round trip; partials of unmasked slots are loaded but never used.
// A row's mask bytes are read before any of its outputs is written, so mask_out may be mask_in.
template <bool QUOTA>
__global__ __launch_bounds__(kDecideThreads) void decide_kernel(StepParams P) {
    extern __shared__ float s_conf[];           // [L]
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int L = P.L, NC = P.NC;
    int *s_arg = (int *)(s_conf + L);           // [L]
    uint8_t *s_mask = (uint8_t *)(s_arg + L);   // [L]
    uint8_t *s_u = s_mask + L;                  // [L] quota rule: slot unmasked this step
    const uint8_t *mrow = P.mask_in + (int64_t)row * L;
    const float4 *prow = P.partials + (int64_t)row * L * NC;
    // inputs of the rule first (lanes 0, 1, 2: tau, p, b; one vector load), so that their
    // latency overlaps that of the partials
    const int32_t *rin = lane == 1 ? P.p : lane == 2 ? P.b : (const int32_t *)P.tau;
    const int32_t rule_in = rin[row];
    for (int g0 = wave; g0 < L; g0 += kDecideWaves * kGroup) {
        // slots g0, g0 + 4, ..., g0 + 4*(kGroup-1) of this row; addresses are clamped into the
        // row so that every load is unconditional and they all go out together
        float Mr[kGroup], Sr[kGroup];
        int vr[kGroup];
        const int jm = g0 + (lane & (kGroup - 1)) * kDecideWaves;   // lane s loads slot s's mask byte
        const uint32_t mv = mrow[min(jm, L - 1)];
        uint32_t gm = 0;                                            // bit s: slot s is masked
        for (int base = 0; base < NC; base += 64) {
            float4 t[kGroup];
            const bool in = base + lane < NC;
            const int cl = min(base + lane, NC - 1);
#pragma unroll
            for (int s = 0; s < kGroup; ++s) t[s] = prow[(int64_t)min(g0 + s * kDecideWaves, L - 1) * NC + cl];
            if (base == 0) gm = (uint32_t)__ballot(lane < kGroup && jm < L && mv != 0) & ((1u << kGroup) - 1);
#pragma unroll
            for (int s = 0; s < kGroup; ++s) {
                float Mb, Sb;
                int vb;
                merge_lanes(t[s], in && ((gm >> s) & 1), Mb, Sb, vb);
                if (base == 0) {
                    Mr[s] = Mb; Sr[s] = Sb; vr[s] = vb;
                } else {
                    const float Mn = fmaxf(Mr[s], Mb);
                    Sr[s] = Sr[s] * __builtin_amdgcn_exp2f((Mr[s] - Mn) * kLog2e) +
                            Sb * __builtin_amdgcn_exp2f((Mb - Mn) * kLog2e);
                    if (Mb > Mr[s]) vr[s] = vb;
                    Mr[s] = Mn;
                }
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int s = 0; s < kGroup; ++s) {
                const int j = g0 + s * kDecideWaves;
                if (j < L) {
                    s_mask[j] = (gm >> s) & 1;
                    s_conf[j] = 1.0f / Sr[s];
                    // out of range only for non-finite logits (a broken precondition): index 0
                    s_arg[j] = (vr[s] >= 0 && vr[s] < P.V) ? vr[s] : 0;
                }
            }
        }
    }
    __syncthreads();
    int nmasked = 0;
    if (QUOTA) {
        // every thread: the masked count and k; then the rank of each of its masked slots among the
        // row's masked slots by (confidence descending, slot ascending); rank < k unmasks
        for (int g = 0; g < L; g += 64) nmasked += __popcll(__ballot(g + lane < L && s_mask[g + lane]));
        const int k = quota_for_remaining(L, P.S, nmasked);
        for (int j = tid; j < L; j += kDecideThreads) {
            bool u = false;
            if (s_mask[j]) {
                const float cj = s_conf[j];
                int rank = 0;
                for (int i = 0; i < L; ++i)
                    rank += s_mask[i] && (s_conf[i] > cj || (s_conf[i] == cj && i < j));
                u = rank < k;
            }
            s_u[j] = u;
        }
        __syncthreads();
    }
    if (wave != 0) return;
    const float tau = __int_as_float(__builtin_amdgcn_readlane(rule_in, 0));
    const int32_t p_r = __builtin_amdgcn_readlane(rule_in, 1), b_r = __builtin_amdgcn_readlane(rule_in, 2);
    if (lane == 0 && P.check_fit && (int64_t)p_r + ((int64_t)b_r + 1) * L > P.W) set_status(P.status, DLLM_ERR_SHAPE);
    // the threshold rule, on wave 0: U = {masked j : c_j > tau}; if empty, the masked j with the
    // largest c (lowest j on ties)
    bool any_above = false;
    int best_j = 0x7FFFFFFF;
    if (!QUOTA) {
        float best_c = -INFINITY;
        for (int g = 0; g < L; g += 64) {
            const int j = g + lane;
            const bool masked = j < L && s_mask[j];
            const float c = masked ? s_conf[j] : -INFINITY;
            any_above |= __ballot(masked && c > tau) != 0;
            nmasked += __popcll(__ballot(masked));
            const float gmx = wave_max(c);
            const int gj = wave_min((masked && c == gmx) ? j : 0x7FFFFFFF);
            if (gmx > best_c) { best_c = gmx; best_j = gj; }        // earlier groups win ties
        }
    }
    int n_unmasked = 0;
    const int col0 = P.W - L;
    for (int g = 0; g < L; g += 64) {
        const int j = g + lane;
        const bool masked = j < L && s_mask[j];
        const bool u = masked && (QUOTA ? s_u[j] != 0 : any_above ? (s_conf[j] > tau) : (j == best_j));
        n_unmasked += __popcll(__ballot(u));
        if (j < L) {
            const int64_t qi = (int64_t)row * L + j;
            const int a = masked ? s_arg[j] : -1;
            if (u) P.ids[(int64_t)row * P.W + col0 + j] = a;
            P.mask_out[qi] = (masked && !u) ? 1 : 0;
            if (P.conf_out) P.conf_out[qi] = masked ? s_conf[j] : -1.0f;
            if (P.arg_out) P.arg_out[qi] = a;
        }
    }
    if (lane == 0) {
        const bool fin = nmasked == n_unmasked;
        P.done[row] = fin ? 1 : 0;
        P.accept[row] = fin ? L : 0;
    }
}

inline bool shape_of(int32_t rows, int32_t L, int32_t V, dllm_dtype dt, int &NV, int &NC, size_t &bytes) {
    if (rows < 0 || L < 1 || V < 1 || (dt != DLLM_FP32 && dt != DLLM_BF16)) return false;
    const int E = dt == DLLM_BF16 ? 8 : 4;
    const int64_t nv = ((int64_t)V + E - 1) / E;
    NV = (int)nv;
    NC = (int)((nv + kCH - 1) / kCH);
    bytes = (((size_t)rows * (size_t)L * (size_t)NC * sizeof(float4)) + 255) & ~(size_t)255;
    return true;
}

// Checks shared by the three entry points; fills P's shape fields.  `who` names the caller.
dllm_status check_shape(const char *who, dllm_dtype dtype, int32_t rows, int32_t L, int32_t V, void *workspace,
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
dllm_status check_workspace(const char *who, dllm_dtype dtype, const void *workspace, size_t workspace_bytes,
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

dllm_status check_score(const char *who, const void *logits, dllm_dtype dtype, int64_t pos_stride, int64_t row_stride,
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

dllm_status launch_score(const StepParams &P, dllm_dtype dtype, hipStream_t st) {
    const int es = dtype == DLLM_BF16 ? 2 : 4;
    const int64_t S = (int64_t)P.rows * P.L;
    const int NC = P.NC;
    // vector path: 16-byte aligned rows whose length is a whole number of 16-byte vectors
    const bool aligned = ((uintptr_t)P.logits & 15) == 0 && (P.pos_stride_b & 15) == 0 &&
                         (P.row_stride_b & 15) == 0 && (P.V % (16 / es)) == 0;
    // grid: one workgroup per compute unit; more when the LDS window of masked slots would
    // exceed 2048 entries (24 KiB of dynamic LDS); fewer when a fully masked box has fewer chunks
    // than that many waves
    int64_t grid = cu_count();
    if (grid < (S + 2047) / 2048) grid = (S + 2047) / 2048;
    const int64_t most = (S * NC + kWaves - 1) / kWaves;
    if (grid > most) grid = most;
    if (grid < 1) grid = 1;
    // window: masked slots touched by one workgroup's ceil(M*NC/grid) chunks, for M <= S
    const int64_t per = (S * NC + grid - 1) / grid;
    const int win = (int)((per + NC - 1) / NC + 2);
    const size_t lds = (size_t)win * (sizeof(int64_t) + sizeof(int));
    if (dtype == DLLM_BF16) {
        if (aligned) hipLaunchKernelGGL((score_kernel<true, true>), dim3((unsigned)grid), dim3(kThreads), lds, st, P, win);
        else hipLaunchKernelGGL((score_kernel<true, false>), dim3((unsigned)grid), dim3(kThreads), lds, st, P, win);
    } else {
        if (aligned) hipLaunchKernelGGL((score_kernel<false, true>), dim3((unsigned)grid), dim3(kThreads), lds, st, P, win);
        else hipLaunchKernelGGL((score_kernel<false, false>), dim3((unsigned)grid), dim3(kThreads), lds, st, P, win);
    }
    return check_hip(hipGetLastError(), "dllm_step score launch");
}

dllm_status launch_decide(const StepParams &P, hipStream_t st) {
    const size_t lds = (size_t)P.L * 10 + 16;
    if (P.S > 0) hipLaunchKernelGGL(decide_kernel<true>, dim3((unsigned)P.rows), dim3(kDecideThreads), lds, st, P);
    else hipLaunchKernelGGL(decide_kernel<false>, dim3((unsigned)P.rows), dim3(kDecideThreads), lds, st, P);
    return check_hip(hipGetLastError(), "dllm_step decide launch");
}

}  // namespace

extern "C" size_t dllm_step_workspace_bytes(int32_t rows, int32_t L, int32_t V, dllm_dtype dtype) {
    int NV, NC;
    size_t bytes;
    if (!shape_of(rows, L, V, dtype, NV, NC, bytes)) return 0;
    return bytes;
}

extern "C" dllm_status dllm_step(void *stream, const void *logits, dllm_dtype dtype, int64_t pos_stride,
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
    return launch_decide(P, (hipStream_t)stream);
}

extern "C" dllm_status dllm_step_score(void *stream, const void *logits, dllm_dtype dtype, int64_t pos_stride,
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

extern "C" dllm_status dllm_step_decide(void *stream, dllm_dtype dtype, int32_t rows, int32_t L, int32_t V,
                                        int32_t *input_ids, int32_t W, const uint8_t *mask_in, uint8_t *mask_out,
                                        const float *threshold, const int32_t *p, const int32_t *b, float *conf,
                                        int32_t *argmax, uint8_t *done, int32_t *accept_len, void *workspace,
                                        size_t workspace_bytes, int32_t *status) {
    StepParams P{};
    dllm_status rc = check_shape("dllm_step_decide", dtype, rows, L, V, workspace, P);
    if (rc == DLLM_OK)
        rc = check_decide("dllm_step_decide", input_ids, W, mask_in, mask_out, threshold, 0, p, b, conf, argmax,
                          done, accept_len, status, P);
    if (rc == DLLM_OK) rc = check_workspace("dllm_step_decide", dtype, workspace, workspace_bytes, P);
    if (rc != DLLM_OK || rows == 0) return rc;
    return launch_decide(P, (hipStream_t)stream);
}

extern "C" dllm_status dllm_step_quota(void *stream, const void *logits, dllm_dtype dtype, int64_t pos_stride,
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
    return launch_decide(P, (hipStream_t)stream);
}

extern "C" dllm_status dllm_step_decide_quota(void *stream, dllm_dtype dtype, int32_t rows, int32_t L, int32_t V,
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
    return launch_decide(P, (hipStream_t)stream);
}
