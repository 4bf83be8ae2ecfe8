/* Synthetic logits generator, CPU implementation.
 *
 * Stands in for the mask predictor's forward pass (which needs trained weights and is not
 * built here).  It only produces inputs: it holds none of the unmasking method's arithmetic.
 * A GPU implementation with the same definition lives in synth_gpu.hip; the two share no code,
 * each is written from the definition below, and a GPU test checks them bit for bit.
 *
 * Definition (integer-only up to one int32 -> float32 conversion, so any IEEE machine
 * reproduces every value exactly):
 *
 *   GAMMA = 0x9E3779B97F4A7C15
 *   mix(z)    : z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31
 *   sm(k, i)  = mix(k + (i+1)*GAMMA)        -- the i-th output of SplitMix64 started at state k
 *               (Steele, Lea, Flood, "Fast splittable pseudorandom number generators", 2014;
 *                finaliser constants of Vigna's public-domain splitmix64.c)
 *   k_pos     = sm(sm(sm(seed, req), block), j)            req = request id, block = b, j = slot in block
 *   t         = sm(k_pos, 2^40) mod V                      planted token, fixed per (req, block, j)
 *   k_step    = sm(k_pos, 2^41 + m_rem)                    m_rem = masked slots left in the row's block
 *   off       = (sm(k_step, 2^42) >> 44) * umax            planted offset, ~U[0, umax) in units of 2^-20
 *   z(v)      = sum of the twelve 16-bit fields of sm(k_step, 3v), sm(k_step, 3v+1), sm(k_step, 3v+2)
 *               minus 393210                               Irwin-Hall(12) noise, sd 65536 (= 1.0)
 *   X(v)      = 16*sigma*z(v) + (v == t ? off : 0)         int32, units of 2^-20
 *   fp32(v)   = (float)X(v) * 2^-20                        round-to-nearest-even conversion, exact scale
 *   bf16(v)   = fp32(v) rounded to bfloat16, nearest-even on the bit pattern
 *
 * Keying the step by the count of masked slots left (which strictly falls every step while a
 * block is open) makes the logits a function of the request's state alone, so a request sees
 * the same logits whether it runs alone, in a synchronous batch or under first-done-first-out
 * batching, in any row.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix(uint64_t z) {
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27; z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}
static inline uint64_t sm(uint64_t k, uint64_t i) { return mix(k + (i + 1) * GAMMA); }

/* sum of the four 16-bit fields of w */
static inline uint32_t fields4(uint64_t w) {
    uint64_t pair = (w & 0x0000FFFF0000FFFFULL) + ((w >> 16) & 0x0000FFFF0000FFFFULL);
    return (uint32_t)(pair & 0xFFFFFFFFULL) + (uint32_t)(pair >> 32);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u; memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* One vocabulary row.  out points at element 0 of the row (dtype 0 = fp32, 1 = bf16). */
static void gen_row(void *out, int dtype, int32_t V, uint64_t seed, int64_t req, int64_t block,
                    int64_t j, int64_t m_rem, int32_t sigma, int32_t umax) {
    uint64_t k_pos = sm(sm(sm(seed, (uint64_t)req), (uint64_t)block), (uint64_t)j);
    uint64_t t = sm(k_pos, 1ULL << 40) % (uint64_t)V;
    uint64_t k_step = sm(k_pos, (1ULL << 41) + (uint64_t)m_rem);
    int32_t off = (int32_t)(sm(k_step, 1ULL << 42) >> 44) * umax;
    for (int64_t v = 0; v < V; ++v) {
        uint32_t s = fields4(sm(k_step, 3 * (uint64_t)v)) + fields4(sm(k_step, 3 * (uint64_t)v + 1)) +
                     fields4(sm(k_step, 3 * (uint64_t)v + 2));
        int32_t z = (int32_t)s - 393210;
        int32_t X = 16 * sigma * z + ((uint64_t)v == t ? off : 0);
        float f = (float)X * (1.0f / 1048576.0f);
        if (dtype == 0) ((float *)out)[v] = f;
        else ((uint16_t *)out)[v] = f32_to_bf16_rne(f);
    }
}

/* Fill logits[r, j, 0:V] for every masked (r, j); other positions get NaN (if fill_nan) or are
 * left alone.  Layout: element (r, j, v) at r*row_stride + j*pos_stride + v (in elements).
 * row_req[r] = request id held by row r, blk[r] = its current block index, mask [rows, L] u8. */
void synth_logits_cpu(void *logits, int dtype, int64_t pos_stride, int64_t row_stride,
                      int32_t rows, int32_t L, int32_t V, const int32_t *row_req,
                      const int32_t *blk, const uint8_t *mask, uint64_t seed, int32_t sigma,
                      int32_t umax, int fill_nan) {
    size_t es = dtype == 0 ? 4 : 2;
    int64_t npos = (int64_t)rows * L;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < npos; ++q) {
        int32_t r = (int32_t)(q / L), j = (int32_t)(q % L);
        char *row = (char *)logits + ((int64_t)r * row_stride + (int64_t)j * pos_stride) * es;
        if (mask[q]) {
            int64_t m_rem = 0;
            for (int32_t i = 0; i < L; ++i) m_rem += mask[(int64_t)r * L + i] != 0;
            gen_row(row, dtype, V, seed, row_req[r], blk[r], j, m_rem, sigma, umax);
        } else if (fill_nan) {
            if (dtype == 0) { float nan = NAN; for (int32_t v = 0; v < V; ++v) ((float *)row)[v] = nan; }
            else { for (int32_t v = 0; v < V; ++v) ((uint16_t *)row)[v] = 0x7FC0; }
        }
    }
}

/* Single row, for spot checks of very large workloads. */
void synth_row_cpu(void *out, int dtype, int32_t V, uint64_t seed, int64_t req, int64_t block,
                   int64_t j, int64_t m_rem, int32_t sigma, int32_t umax) {
    gen_row(out, dtype, V, seed, req, block, j, m_rem, sigma, umax);
}

/* The planted token index for (req, block, j): exposed so tests can check the planted law. */
int64_t synth_planted_cpu(int32_t V, uint64_t seed, int64_t req, int64_t block, int64_t j) {
    uint64_t k_pos = sm(sm(sm(seed, (uint64_t)req), (uint64_t)block), (uint64_t)j);
    return (int64_t)(sm(k_pos, 1ULL << 40) % (uint64_t)V);
}
