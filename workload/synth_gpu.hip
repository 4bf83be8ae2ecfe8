// Synthetic logits generator, GPU implementation (gfx950).
//
// Stands in for the mask predictor's forward pass; produces inputs only and holds none of the
// unmasking method's arithmetic.  Written from the same published definition as the CPU
// implementation in synth.c (the two share no code; a GPU test compares them bit for bit):
//
//   sm(k, i) = mix(k + (i+1)*0x9E3779B97F4A7C15)   (SplitMix64, Steele/Lea/Flood 2014; finaliser
//              mix: z^=z>>30; z*=0xBF58476D1CE4E5B9; z^=z>>27; z*=0x94D049BB133111EB; z^=z>>31)
//   k_pos = sm(sm(sm(seed, req), block), j);  t = sm(k_pos, 2^40) mod V
//   k_step = sm(k_pos, 2^41 + m_rem);          off = (sm(k_step, 2^42) >> 44) * umax
//   z(v) = (sum of twelve 16-bit fields of sm(k_step, 3v+r), r = 0..2) - 393210
//   X(v) = 16*sigma*z(v) + [v == t]*off;        fp32 = (float)X * 2^-20;  bf16 = RNE(fp32)
//
// Only masked positions are written (the step never reads the others); with fill_nan the
// others are set to NaN so that a stray read would show up in every result.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t sm(uint64_t k, uint64_t i) { return mix64(k + (i + 1) * kGamma); }

__device__ __forceinline__ uint32_t sum_fields(uint64_t w) {
    uint64_t two = (w & 0x0000FFFF0000FFFFull) + ((w >> 16) & 0x0000FFFF0000FFFFull);
    return (uint32_t)two + (uint32_t)(two >> 32);
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

constexpr int kThreads = 256;
constexpr int kPerThread = 8;
constexpr int kChunk = kThreads * kPerThread;

// grid.x = rows*L*nchunk; one block writes kChunk consecutive vocabulary entries of one position.
__global__ __launch_bounds__(kThreads) void synth_kernel(
    void *__restrict__ logits, int dtype, int64_t pos_stride, int64_t row_stride, int32_t L,
    int32_t V, int32_t nchunk, const int32_t *__restrict__ row_req, const int32_t *__restrict__ blk,
    const uint8_t *__restrict__ mask, uint64_t seed, int32_t sigma, int32_t umax, int fill_nan) {
    const int64_t q = blockIdx.x / nchunk;
    const int32_t chunk = blockIdx.x % nchunk;
    const int32_t r = (int32_t)(q / L), j = (int32_t)(q % L);
    const bool masked = mask[q] != 0;
    const size_t es = dtype == 0 ? 4 : 2;
    char *row = (char *)logits + ((int64_t)r * row_stride + (int64_t)j * pos_stride) * (int64_t)es;
    const int64_t v0 = (int64_t)chunk * kChunk + (int64_t)threadIdx.x * kPerThread;
    if (!masked) {
        if (!fill_nan) return;
        for (int e = 0; e < kPerThread; ++e) {
            int64_t v = v0 + e;
            if (v < V) {
                if (dtype == 0) ((float *)row)[v] = __uint_as_float(0x7FC00000u);
                else ((uint16_t *)row)[v] = 0x7FC0;
            }
        }
        return;
    }
    // masked slots left in this row's block (uniform over the block)
    int m_rem = 0;
    for (int i0 = 0; i0 < L; i0 += kThreads) {
        int i = i0 + (int)threadIdx.x;
        m_rem += __syncthreads_count(i < L && mask[(int64_t)r * L + i] != 0);
    }
    const uint64_t k_pos = sm(sm(sm(seed, (uint64_t)row_req[r]), (uint64_t)blk[r]), (uint64_t)j);
    const uint64_t t = sm(k_pos, 1ull << 40) % (uint64_t)V;
    const uint64_t k_step = sm(k_pos, (1ull << 41) + (uint64_t)m_rem);
    const int32_t off = (int32_t)(sm(k_step, 1ull << 42) >> 44) * umax;

    float f[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
        const uint64_t v = (uint64_t)(v0 + e);
        const uint32_t s = sum_fields(sm(k_step, 3 * v)) + sum_fields(sm(k_step, 3 * v + 1)) +
                           sum_fields(sm(k_step, 3 * v + 2));
        const int32_t z = (int32_t)s - 393210;
        const int32_t X = 16 * sigma * z + (v == t ? off : 0);
        f[e] = (float)X * (1.0f / 1048576.0f);
    }
    const bool full = v0 + kPerThread <= V;
    if (dtype == 1) {
        uint16_t *dst = (uint16_t *)row + v0;
        if (full && (((uintptr_t)dst) & 15) == 0) {
            uint4 pk;
            pk.x = bf16_bits(f[0]) | (bf16_bits(f[1]) << 16);
            pk.y = bf16_bits(f[2]) | (bf16_bits(f[3]) << 16);
            pk.z = bf16_bits(f[4]) | (bf16_bits(f[5]) << 16);
            pk.w = bf16_bits(f[6]) | (bf16_bits(f[7]) << 16);
            *(uint4 *)dst = pk;
        } else {
            for (int e = 0; e < kPerThread; ++e)
                if (v0 + e < V) dst[e] = (uint16_t)bf16_bits(f[e]);
        }
    } else {
        float *dst = (float *)row + v0;
        if (full && (((uintptr_t)dst) & 15) == 0) {
            *(float4 *)dst = make_float4(f[0], f[1], f[2], f[3]);
            *(float4 *)(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
        } else {
            for (int e = 0; e < kPerThread; ++e)
                if (v0 + e < V) dst[e] = f[e];
        }
    }
}

}  // namespace

// Returns 0 on success, 1 on bad arguments, 2 on a HIP launch error.
extern "C" int synth_logits_gpu(void *stream, void *logits, int dtype, int64_t pos_stride,
                                int64_t row_stride, int32_t rows, int32_t L, int32_t V,
                                const int32_t *row_req, const int32_t *blk, const uint8_t *mask,
                                uint64_t seed, int32_t sigma, int32_t umax, int fill_nan) {
    if (!logits || !row_req || !blk || !mask || rows < 0 || L < 1 || V < 1) return 1;
    if ((dtype != 0 && dtype != 1) || pos_stride < V || row_stride < (int64_t)L * pos_stride) return 1;
    if (rows == 0) return 0;
    const int32_t nchunk = (V + kChunk - 1) / kChunk;
    const int64_t nblocks = (int64_t)rows * L * nchunk;
    if (nblocks > 0x7FFFFFFFll) return 1;
    hipLaunchKernelGGL(synth_kernel, dim3((uint32_t)nblocks), dim3(kThreads), 0, (hipStream_t)stream,
                       logits, dtype, pos_stride, row_stride, L, V, nchunk, row_req, blk, mask, seed,
                       sigma, umax, fill_nan);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
