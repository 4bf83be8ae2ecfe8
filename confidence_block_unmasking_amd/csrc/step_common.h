// Shared definitions of the step kernels (internal; not part of the C ABI): launch parameters,
// wave reductions, element access and the chunk reduction used by the scoring kernel, the mask
// scan used by its prologue, and the workspace shape.
#pragma once

#include <hip/hip_ext.h>

#include "common.h"

namespace dllm {


#ifndef DLLM_STEP_VPL
#define DLLM_STEP_VPL 8
#endif
#ifndef DLLM_STEP_WAVES
#define DLLM_STEP_WAVES 8
#endif
#ifndef DLLM_STEP_ACC
#define DLLM_STEP_ACC 4               // running sums per lane in the chunk reduction (a power of two)
#endif

#ifndef DLLM_STEP_GROUPS_PER_CU
#define DLLM_STEP_GROUPS_PER_CU 4
#endif

constexpr int kWaves = DLLM_STEP_WAVES;       // waves per scoring workgroup
// Scoring workgroups per compute unit over the launch.  Two fit a unit at a time (the kernel keeps
// to 128 VGPRs: four waves per SIMD); the hardware dispatcher hands the rest out as units free up.
constexpr int kGroupsPerCU = DLLM_STEP_GROUPS_PER_CU;
// Box sizes (rows * L * chunks per slot, per compute unit) below which the scoring grid is two
// workgroups per unit, and one.
constexpr int kSmallBoxChunksPerCU = 140;
constexpr int kTinyBoxChunksPerCU = 24;
constexpr int kThreads = 64 * kWaves;
constexpr int kVPL = DLLM_STEP_VPL;           // 16-byte vectors per lane per chunk
constexpr int kCH = 64 * kVPL;                // vectors per chunk
constexpr int kTile = kThreads * 16;          // mask bytes per prologue pass (16 per thread)
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
    float4 *triples;                          // vocabulary shards: [rows*L*n_shards] per-shard results
    int32_t shard, n_shards, vocab_offset;    // this shard, the shard count, its first global column
    float *conf_out;
    int32_t *arg_out;
    uint8_t *done;
    int32_t *accept;
    int32_t *unmasked_out;                    // per row: slots unmasked (optional)
    uint8_t *fallback_out;                    // per row: the rule's single-slot fallback applied (optional)
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
// The same reductions with the four rows combined by DPP row broadcasts (lane 15 of a row into the
// next row, then lane 31 into rows 2 and 3): lane 63 ends with the result, read once.  Rows that
// a broadcast does not write keep the identity element as their operand.
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ float dppf_rows(float idle, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(idle), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float red_max_bc(float v) {
    v = fmaxf(v, dppf<kQuadSwap1>(v));
    v = fmaxf(v, dppf<kQuadSwap2>(v));
    v = fmaxf(v, dppf<kHalfMirror>(v));
    v = fmaxf(v, dppf<kRowMirror>(v));
    v = fmaxf(v, dppf_rows<kRowBcast15, 0xA>(-INFINITY, v));
    v = fmaxf(v, dppf_rows<kRowBcast31, 0xC>(-INFINITY, v));
    return rlf(v, 63);
}
__device__ __forceinline__ float red_sum_bc(float v) {
    v += dppf<kQuadSwap1>(v);
    v += dppf<kQuadSwap2>(v);
    v += dppf<kHalfMirror>(v);
    v += dppf<kRowMirror>(v);
    v += dppf_rows<kRowBcast15, 0xA>(0.0f, v);
    v += dppf_rows<kRowBcast31, 0xC>(0.0f, v);
    return rlf(v, 63);
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
// of the row; -inf marks padding.  Per-vector maxima, the lane max, the lane sum of exp(x - max),
// then the wave combine.  The lowest vector holding the wave max is found from one ballot per
// vector slot k (vector index k*64 + lane grows with k first, then lane); its owner lane and k are
// wave-uniform, so that vector's E values are read with readlane and the first element equal to
// the max gives the exact index without going back to memory.  A chunk whose values are all -inf
// reports no index.
template <int E>
__device__ __forceinline__ Part reduce_lanes(float (&x)[kVPL][E], int vb) {
    float vm[kVPL];
#pragma unroll
    for (int k = 0; k < kVPL; ++k) {
        float a = x[k][0];
#pragma unroll
        for (int e = 1; e < E; ++e) a = fmaxf(a, x[k][e]);
        vm[k] = a;
    }
    float m = vm[0];
#pragma unroll
    for (int k = 1; k < kVPL; ++k) m = fmaxf(m, vm[k]);
    const float nml = (m == -INFINITY) ? 0.0f : -m * kLog2e;
    // DLLM_STEP_ACC independent running sums (the adds are the only serial chain of the loop)
    float acc[DLLM_STEP_ACC];
#pragma unroll
    for (int a = 0; a < DLLM_STEP_ACC; ++a) acc[a] = 0.0f;
#pragma unroll
    for (int k = 0; k < kVPL; ++k) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[(k * E + e) % DLLM_STEP_ACC] += __builtin_amdgcn_exp2f(fmaf(x[k][e], kLog2e, nml));
    }
#pragma unroll
    for (int w = DLLM_STEP_ACC / 2; w >= 1; w /= 2) {
#pragma unroll
        for (int a = 0; a < w; ++a) acc[a] += acc[a + w];
    }
    Part r;
    r.m = red_max_bc(m);
    const float scale = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((m - r.m) * kLog2e);
    r.s = red_sum_bc(acc[0] * scale);
    int elem = 0x7FFFFFFF;
    if (r.m != -INFINITY) {
        int kw = 0, lw = 0;
#pragma unroll
        for (int k = kVPL - 1; k >= 0; --k) {
            const uint64_t bal = __ballot(vm[k] == r.m);
            if (bal != 0) {
                kw = k;
                lw = __builtin_ctzll(bal);
            }
        }
        int ef = E;
#pragma unroll
        for (int k = 0; k < kVPL; ++k) {
            if (k == kw) {
#pragma unroll
                for (int e = E - 1; e >= 0; --e)
                    if (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[k][e]), lw)) == r.m) ef = e;
            }
        }
        elem = (vb + kw * 64 + lw) * E + ef;
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
// n is wave-uniform: full chunks take no masking work at all, only a row's short last chunk does.
template <bool BF16>
__device__ __forceinline__ void convert(const u32x4 (&raw)[kVPL], float (&x)[kVPL][Fmt<BF16>::E], int n) {
#pragma unroll
    for (int k = 0; k < kVPL; ++k) unpack<BF16>(raw[k], x[k]);
    if (n < kCH) {
        const int lane = lane_id();
#pragma unroll
        for (int k = 0; k < kVPL; ++k) {
            const bool pad = k * 64 + lane >= n;
#pragma unroll
            for (int e = 0; e < Fmt<BF16>::E; ++e) x[k][e] = pad ? -INFINITY : x[k][e];
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


inline bool shape_of(int32_t rows, int32_t L, int32_t V, int32_t dt, int &NV, int &NC, size_t &bytes) {
    if (rows < 0 || L < 1 || V < 1 || (dt != DLLM_FP32 && dt != DLLM_BF16)) return false;
    const int E = dt == DLLM_BF16 ? 8 : 4;
    const int64_t nv = ((int64_t)V + E - 1) / E;
    NV = (int)nv;
    NC = (int)((nv + kCH - 1) / kCH);
    bytes = (((size_t)rows * (size_t)L * (size_t)NC * sizeof(float4)) + 255) & ~(size_t)255;
    return true;
}


// Launchers (score.hip, decide.hip): enqueue the kernels for checked parameters.
// With ev_start (and ev_stop) given, the scoring kernel is launched with the two events bound to
// its own start and end.
dllm_status launch_score(const StepParams &P, int32_t dtype, hipStream_t st, hipEvent_t ev_start = nullptr,
                         hipEvent_t ev_stop = nullptr);
// mode: kRuleThreshold / kRuleQuota apply the row's rule; kEmitTriples writes each masked slot's
// merged (max, sum, global index) into P.triples at shard P.shard instead.
constexpr int kRuleThreshold = 0, kRuleQuota = 1, kEmitTriples = 2;
dllm_status launch_decide(const StepParams &P, hipStream_t st, int mode);

}  // namespace dllm
