// dllm_step_features: per-request inputs of a remaining-step predictor, after one denoise step.
//
// [DiLaServe] = page "DiLaServe: High SLO Attainment Serving for Diffusion Language Models",
// §四 4.2 ③ (paper §3.2.3, Step Prediction): progress features (the fraction of tokens already
// unmasked) and confidence features (quantiles of the output tokens' confidences); the scalar
// inputs are the threshold, the output length, the full and block progress, and the min / q25 /
// median / mean / q75 of the confidences.  The page counts 11 and names these 9, which are computed
// here in that order (the predictor itself, a trained model, is not part of this library).
//
// One workgroup per row.  The confidences the step scored (conf >= 0) are ranked in LDS (ascending,
// ties by slot), so thread 0 can interpolate the quantiles linearly between order statistics at
// position q*(n-1) and sum them in order in double precision.  Latency-bound: kilobytes per row,
// so the request lookup (two dependent loads) runs beside the confidence loads, not after them.
#include "common.h"

namespace {

using namespace dllm;

constexpr int kThreads = 256;
constexpr int kFeatures = 9;

// NaN stored as its bit pattern (the library is built without NaN semantics in arithmetic).
__device__ __forceinline__ void store_nan(float *p) { *(uint32_t *)p = 0x7FC00000u; }

__device__ double quantile(const float *sorted, int n, double q) {
    const double pos = q * (n - 1);
    const int lo = (int)floor(pos);
    const int hi = min(lo + 1, n - 1);
    const double a = sorted[lo], b = sorted[hi];
    return a + (b - a) * (pos - lo);
}

__global__ __launch_bounds__(kThreads) void features_kernel(int32_t L, const int32_t *__restrict__ row_req, dllm_reqs R,
                                                            const float *__restrict__ conf,
                                                            const uint8_t *__restrict__ mask_after,
                                                            float *__restrict__ out, int32_t *status) {
    extern __shared__ float s_c[];             // [L] this row's confidences, -1 where not scored
    float *s_sorted = s_c + L;                 // [L] scored confidences in ascending order
    __shared__ int s_n, s_masked;
    fetch_args(L, row_req, R.n_req, R.K, R.b, R.threshold, conf, mask_after, out, status);
    const int row = blockIdx.x, tid = threadIdx.x;
    // Two dependent loads (the row's request, then its fields) on thread 0, while waves 1.. load
    // and count the row's confidences: the two chains overlap.
    int q = -1, Kq = 0, bq = 0;
    float th = 0.0f;
    bool ok = false;
    if (tid == 0) {
        s_n = 0;
        s_masked = 0;
        q = row_req[row];
        ok = q >= 0 && q < R.n_req;
        if (ok) {
            Kq = R.K[q];
            bq = R.b[q];
            th = R.threshold[q];
        }
    }
    int nm = 0, ns = 0;
    if (tid >= 64) {
        for (int j = tid - 64; j < L; j += kThreads - 64) {
            const float c = conf[(int64_t)row * L + j];
            s_c[j] = c;
            ns += c >= 0.0f;
            nm += mask_after[(int64_t)row * L + j] != 0;
        }
        nm = wave_sum_i(nm);
        ns = wave_sum_i(ns);
    }
    __syncthreads();
    if (tid >= 64 && (tid & 63) == 0) {
        atomicAdd(&s_masked, nm);
        atomicAdd(&s_n, ns);
    }
    for (int j = tid; j < L; j += kThreads) {
        const float c = s_c[j];
        if (c >= 0.0f) {
            int rank = 0;
#pragma unroll 8
            for (int i = 0; i < L; ++i) {
                const float ci = s_c[i];
                rank += ci >= 0.0f && (ci < c || (ci == c && i < j));
            }
            s_sorted[rank] = c;
        }
    }
    __syncthreads();
    if (tid != 0) return;
    float *f = out + (int64_t)row * kFeatures;
    if (!ok || Kq < 1) {
        set_status(status, DLLM_ERR_ARG);
        for (int k = 0; k < kFeatures; ++k) store_nan(f + k);
        return;
    }
    const int n = s_n;
    const int unmasked = L - s_masked;
    f[0] = th;
    f[1] = (float)((int64_t)Kq * L);
    f[2] = (float)(((double)bq * L + unmasked) / ((double)Kq * L));
    f[3] = (float)((double)unmasked / L);
    if (n == 0) {
        for (int k = 4; k < kFeatures; ++k) store_nan(f + k);
        return;
    }
    double sum = 0.0;
    for (int i = 0; i < n; ++i) sum += s_sorted[i];
    f[4] = s_sorted[0];
    f[5] = (float)quantile(s_sorted, n, 0.25);
    f[6] = (float)quantile(s_sorted, n, 0.5);
    f[7] = (float)(sum / n);
    f[8] = (float)quantile(s_sorted, n, 0.75);
}

}  // namespace

extern "C" dllm_status dllm_step_features(void *stream, int32_t rows, int32_t L, const int32_t *row_req,
                                          const dllm_reqs *reqs, const float *conf, const uint8_t *mask_out,
                                          float *features, int32_t *status) {
    if (rows < 0) return fail(DLLM_ERR_ARG, "dllm_step_features: rows < 0");
    if (L < 1 || L > DLLM_MAX_L) return fail(DLLM_ERR_SHAPE, "dllm_step_features: L=%d outside [1, %d]", L, DLLM_MAX_L);
    if (rows > DLLM_MAX_ROWS) return fail(DLLM_ERR_SHAPE, "dllm_step_features: rows=%d > %d", rows, DLLM_MAX_ROWS);
    if (rows == 0) return DLLM_OK;
    if (!row_req || !reqs || !conf || !mask_out || !features || !status)
        return fail(DLLM_ERR_ARG, "dllm_step_features: null required pointer");
    if (!reqs->K || !reqs->b || !reqs->threshold || reqs->n_req < 0)
        return fail(DLLM_ERR_ARG, "dllm_step_features: incomplete request table");
    const size_t lds = (size_t)L * 2 * sizeof(float);
    hipLaunchKernelGGL(features_kernel, dim3((unsigned)rows), dim3(kThreads), lds, (hipStream_t)stream, L, row_req,
                       *reqs, conf, mask_out, features, status);
    return check_hip(hipGetLastError(), "dllm_step_features launch");
}
