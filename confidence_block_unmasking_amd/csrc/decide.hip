// Deciding half of the denoise step: each masked slot's partials merged in chunk order into its
// confidence and predicted token, then the row's unmask rule (LowConfidence threshold, or the fixed
// per-step quota), write-back, done flags and accept lengths.
//
// [FDFO] = page "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」" §工程设计一 (LowConfidence)
// and §工程设计二 (accept length 0 or block_size); [DiLaServe] = page "DiLaServe: High SLO
// Attainment Serving for Diffusion Language Models" §三 3.1 (softmax probability as the
// confidence); [BlockServe] = page "BlockServe: 块粒度连续批处理实现高吞吐扩散大语言模型服务"
// §II-E (per-step transfer quota).
#include "step_common.h"

namespace dllm {

constexpr int kDecideThreads = 512;           // one workgroup per row: 8 waves
constexpr int kDecideWaves = kDecideThreads / 64;

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
// Each wave loads the partials and mask bytes of G slots before reducing any of them, so a row of
// up to kDecideWaves*G slots costs about one memory round trip; partials of unmasked slots are
// loaded but never used.  G is the smallest of 4 and 8 that covers the row in one pass (the merges
// a wave runs one after the other are the rest of the kernel's time).
// A row's mask bytes are read before any of its outputs is written, so mask_out may be mask_in.
template <int MODE, int G>
__global__ __launch_bounds__(kDecideThreads) void decide_kernel(StepParams P) {
    constexpr bool QUOTA = MODE == kRuleQuota;
    extern __shared__ float s_conf[];           // [L]
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int L = P.L, NC = P.NC;
    int *s_arg = (int *)(s_conf + L);           // [L]
    uint8_t *s_mask = (uint8_t *)(s_arg + L);   // [L]
    uint8_t *s_u = s_mask + L;                  // [L] quota rule: slot unmasked this step
    fetch_args(P.mask_in, P.partials, P.tau, P.p, P.b, P.ids, P.mask_out, P.conf_out, P.arg_out, P.done, P.accept,
               P.W, P.V, P.check_fit, P.status);
    const uint8_t *mrow = P.mask_in + (int64_t)row * L;
    const float4 *prow = P.partials + (int64_t)row * L * NC;
    // inputs of the rule first (lanes 0, 1, 2: tau, p, b; one vector load), so that their
    // latency overlaps that of the partials
    // (no rule, and no rule inputs, when emitting shard results)
    const int32_t *rin = lane == 1 ? P.p : lane == 2 ? P.b : (const int32_t *)P.tau;
    const int32_t rule_in = MODE == kEmitTriples ? 0 : rin[row];
    for (int g0 = wave; g0 < L; g0 += kDecideWaves * G) {
        // slots g0, g0 + kDecideWaves, ..., g0 + kDecideWaves*(G-1) of this row; addresses are
        // clamped into the row so that every load is unconditional and they all go out together
        float Mr[G], Sr[G];
        int vr[G];
        const int jm = g0 + (lane & (G - 1)) * kDecideWaves;        // lane s loads slot s's mask byte
        const uint32_t mv = mrow[min(jm, L - 1)];
        uint32_t gm = 0;                                            // bit s: slot s is masked
        for (int base = 0; base < NC; base += 64) {
            float4 t[G];
            const bool in = base + lane < NC;
            const int cl = min(base + lane, NC - 1);
#pragma unroll
            for (int s = 0; s < G; ++s) t[s] = prow[(int64_t)min(g0 + s * kDecideWaves, L - 1) * NC + cl];
            if (base == 0) gm = (uint32_t)__ballot(lane < G && jm < L && mv != 0) & ((1u << G) - 1);
#pragma unroll
            for (int s = 0; s < G; ++s) {
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
        if (MODE == kEmitTriples) {
            // one shard's result per masked slot, its index made global
            if (lane == 0) {
#pragma unroll
                for (int s = 0; s < G; ++s) {
                    const int j = g0 + s * kDecideWaves;
                    if (j < L && ((gm >> s) & 1))
                        P.triples[((int64_t)row * L + j) * P.n_shards + P.shard] =
                            make_float4(Mr[s], Sr[s], __int_as_float(vr[s] + P.vocab_offset), 0.0f);
                }
            }
            continue;
        }
        if (lane == 0) {
#pragma unroll
            for (int s = 0; s < G; ++s) {
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
    if (MODE == kEmitTriples) return;
    __syncthreads();
    int nmasked = 0;
    bool u_lane = false;                       // quota rule, L <= 64: wave 0 lane j's slot unmasks
    if (QUOTA) {
        // the masked count and k; then the rank of each masked slot among the row's masked slots
        // by (confidence descending, slot ascending); rank < k unmasks
        if (L <= 64) {
            // one slot per lane of wave 0, the others read from registers
            if (wave != 0) return;
            const bool mj = lane < L && s_mask[lane] != 0;
            const float cj = mj ? s_conf[lane] : 0.0f;
            const uint64_t mb = __ballot(mj);
            nmasked = __popcll(mb);
            const int k = quota_for_remaining(L, P.S, nmasked);
            int rank = 0;
            for (int i = 0; i < L; ++i) {
                const float ci = rlf(cj, i);
                rank += ((mb >> i) & 1) && (ci > cj || (ci == cj && i < lane));
            }
            u_lane = mj && rank < k;
        } else {
            for (int g = 0; g < L; g += 64) nmasked += __popcll(__ballot(g + lane < L && s_mask[g + lane]));
            const int k = quota_for_remaining(L, P.S, nmasked);
            for (int j = tid; j < L; j += kDecideThreads) {
                bool u = false;
                if (s_mask[j]) {
                    const float cj = s_conf[j];
                    int rank = 0;
#pragma unroll 8
                    for (int i = 0; i < L; ++i)
                        rank += s_mask[i] && (s_conf[i] > cj || (s_conf[i] == cj && i < j));
                    u = rank < k;
                }
                s_u[j] = u;
            }
            __syncthreads();
        }
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
        const bool u = masked && (QUOTA ? (L <= 64 ? u_lane : s_u[j] != 0) : any_above ? (s_conf[j] > tau) : (j == best_j));
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
        if (P.unmasked_out) P.unmasked_out[row] = n_unmasked;
        if (P.fallback_out) P.fallback_out[row] = (!QUOTA && nmasked > 0 && !any_above) ? 1 : 0;
    }
}


template <int G>
void launch_decide_g(const StepParams &P, hipStream_t st, int mode, hipEvent_t ev_stop) {
    const size_t lds = (size_t)P.L * 10 + 16;
    const dim3 grid((unsigned)P.rows), block(kDecideThreads);
    // with ev_stop: the same launch, the event taking the kernel's own end time
    auto go = [&](auto kernel) {
        if (ev_stop) hipExtLaunchKernelGGL(kernel, grid, block, lds, st, nullptr, ev_stop, 0, P);
        else hipLaunchKernelGGL(kernel, grid, block, lds, st, P);
    };
    if (mode == kRuleQuota) go(decide_kernel<kRuleQuota, G>);
    else if (mode == kEmitTriples) go(decide_kernel<kEmitTriples, G>);
    else go(decide_kernel<kRuleThreshold, G>);
}

dllm_status launch_decide_ev(const StepParams &P, hipStream_t st, int mode, hipEvent_t ev_stop) {
    if (P.L <= kDecideWaves * 4) launch_decide_g<4>(P, st, mode, ev_stop);
    else launch_decide_g<8>(P, st, mode, ev_stop);
    return check_hip(hipGetLastError(), "dllm_step decide launch");
}

dllm_status launch_decide(const StepParams &P, hipStream_t st, int mode) {
    return launch_decide_ev(P, st, mode, nullptr);
}


}  // namespace dllm
