// Internal helpers shared by the libdllm sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dllm.h"

namespace dllm {

// Host: record the text for dllm_last_error() and return the code.
dllm_status fail(dllm_status code, const char *fmt, ...);
// Host: map a HIP error (if any) to DLLM_ERR_HIP.
dllm_status check_hip(hipError_t e, const char *what);
// Host: compute units of the current device (cached per device).
int cu_count();

// Device: store the first nonzero status code.
__device__ __forceinline__ void set_status(int32_t *status, int32_t code) {
    if (status) atomicCAS(status, 0, code);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// Device: make the listed kernel-argument values available at this point.  Their scalar loads
// then go out together at the start instead of each at its first use, where every wait would be
// one more dependent round trip in a latency-bound kernel.
template <typename T>
__device__ __forceinline__ void fetch_arg(const T &v) {
    asm volatile("" ::"s"(v));
}
template <typename... T>
__device__ __forceinline__ void fetch_args(const T &...v) {
    (fetch_arg(v), ...);
}

// ---- whole-wave operations (every lane active) on DPP: no LDS round trip ----------------------
// Rows of 16 lanes first (quad swaps and mirrors for reductions, right shifts for the scan), then
// the four rows joined by row broadcasts (lane 15 of a row into the next row, lane 31 into rows 2
// and 3); a reduction's result is read from lane 63, so every lane gets it.
namespace wave_dpp {
constexpr int kQuad1 = 0xB1, kQuad2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143;
// lane i reads lane CTRL(i); rows outside ROWS, and (with BC) lanes whose source lies outside the
// row, read `idle`
template <int CTRL, int ROWS = 0xF, bool BC = false>
__device__ __forceinline__ int mov(int idle, int v) {
    return __builtin_amdgcn_update_dpp(idle, v, CTRL, ROWS, 0xF, BC);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float movf(float idle, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(idle), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
}  // namespace wave_dpp

__device__ __forceinline__ float wave_max(float v) {
    using namespace wave_dpp;
    v = fmaxf(v, movf<kQuad1>(v, v));
    v = fmaxf(v, movf<kQuad2>(v, v));
    v = fmaxf(v, movf<kHalfMirror>(v, v));
    v = fmaxf(v, movf<kMirror>(v, v));
    v = fmaxf(v, movf<kBcast15, 0xA>(-INFINITY, v));
    v = fmaxf(v, movf<kBcast31, 0xC>(-INFINITY, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
template <typename Op>
__device__ __forceinline__ int wave_reduce_i(int v, int identity, Op op) {
    using namespace wave_dpp;
    v = op(v, mov<kQuad1>(v, v));
    v = op(v, mov<kQuad2>(v, v));
    v = op(v, mov<kHalfMirror>(v, v));
    v = op(v, mov<kMirror>(v, v));
    v = op(v, mov<kBcast15, 0xA>(identity, v));
    v = op(v, mov<kBcast31, 0xC>(identity, v));
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_min(int v) {
    return wave_reduce_i(v, 0x7FFFFFFF, [](int a, int b) { return min(a, b); });
}
__device__ __forceinline__ int wave_max_i(int v) {
    return wave_reduce_i(v, (int)0x80000000, [](int a, int b) { return max(a, b); });
}
__device__ __forceinline__ int wave_sum_i(int v) {
    return wave_reduce_i(v, 0, [](int a, int b) { return a + b; });
}
// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
    using namespace wave_dpp;
    v += mov<kShr1, 0xF, true>(0, v);
    v += mov<kShr2, 0xF, true>(0, v);
    v += mov<kShr4, 0xF, true>(0, v);
    v += mov<kShr8, 0xF, true>(0, v);
    v += mov<kBcast15, 0xA>(0, v);
    v += mov<kBcast31, 0xC>(0, v);
    return v;
}

}  // namespace dllm
