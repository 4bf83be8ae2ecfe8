/* Float64 scorer for many vocabulary rows at once: the oracle's per-slot definition, in C.
 *
 * TEST INFRASTRUCTURE ONLY.  It is the same definition as score() in step.py, written for
 * replaying whole loops (millions of slots of 126464 or 152064 logits each), where the
 * NumPy version is too slow.  It shares no code with the GPU library; the tests pin it
 * against hand-worked values, closed forms, library routines and step.py's score().
 *
 * Definition ([DiLaServe] "DiLaServe: High SLO Attainment Serving for Diffusion Language
 * Models" §三 3.1: the confidence of a masked slot is the softmax probability of its predicted
 * token; [FDFO] "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」" §工程设计三: the
 * predicted token is the greedy argmax, temperature 0).  For one row x[0..V-1], each element
 * widened exactly to double (a bfloat16 is the upper half of a float32; float32 -> double is
 * exact):
 *   m = max_v x_v
 *   a = the smallest v with x_v = m            (reading: ties go to the lowest index)
 *   S = sum_v exp(x_v - m)
 *   c = 1 / S                                  (= exp(x_a) / sum_v exp(x_v), since x_a = m)
 * Non-finite logits break the step's precondition: such a row is reported, not scored.
 *
 * Arithmetic: float64 throughout; exp is the C library's, in the vector form glibc ships
 * (libmvec, documented maximum error 4 ulp), summed in as many running sums as the vector
 * has lanes.  Both only move S by about V * 1e-16 relative at most.  The maximum is an exact
 * operation whatever the order.  Rows are independent, so they are spread over OpenMP
 * threads; each row is scored by one thread, in the steps above.
 */
#include <float.h>
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#pragma omp declare simd notinbranch
extern double exp(double);

/* One row: the four quantities of the definition, in order.  Returns 0 if a logit is not finite
 * (then nothing is written).  Compiled for the machine's widest vectors (chosen at load time). */
__attribute__((target_clones("avx512f", "avx2", "default")))
int oracle_rows_score_one(const char *row, int dtype, int64_t V, double *buf, int64_t *argmax, double *conf) {
    /* widen every element exactly to double */
    if (dtype == 1) {
        const uint16_t *h = (const uint16_t *)row;
        for (int64_t v = 0; v < V; ++v) {
            uint32_t u = (uint32_t)h[v] << 16;
            float f;
            memcpy(&f, &u, 4);
            buf[v] = (double)f;
        }
    } else {
        const float *f = (const float *)row;
        for (int64_t v = 0; v < V; ++v) buf[v] = (double)f[v];
    }
    int finite = 1;
#pragma omp simd reduction(& : finite)
    for (int64_t v = 0; v < V; ++v) finite &= fabs(buf[v]) <= DBL_MAX;
    if (!finite) return 0;
    /* m = max_v x_v */
    double m = -INFINITY;
#pragma omp simd reduction(max : m)
    for (int64_t v = 0; v < V; ++v) m = buf[v] > m ? buf[v] : m;
    /* a = the smallest v with x_v = m (-0.0 equals +0.0) */
    int64_t a = 0;
    while (buf[a] != m) ++a;
    /* S = sum_v exp(x_v - m); c = 1 / S */
    double S = 0.0;
#pragma omp simd reduction(+ : S)
    for (int64_t v = 0; v < V; ++v) S += exp(buf[v] - m);
    *argmax = a;
    *conf = 1.0 / S;
    return 1;
}

/* Score n rows.  Row i starts at element i*row_stride of x (dtype 0: float32, 1: bfloat16 bit
 * patterns).  Writes argmax[i] and conf[i]; a row with a non-finite element gets argmax -1 and
 * conf NaN.  Returns the number of such rows (0 when every row was scored), or -1 if memory
 * ran out.  nthreads <= 0 lets OpenMP choose. */
int64_t oracle_score_rows(const void *x, int dtype, int64_t n, int64_t V, int64_t row_stride,
                          int64_t *argmax, double *conf, int nthreads) {
    const size_t es = dtype == 1 ? 2 : 4;
    int64_t bad = 0;
    int oom = 0;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(+ : bad) reduction(| : oom)
    {
        double *buf = (double *)malloc((size_t)(V > 0 ? V : 1) * sizeof(double));
        if (!buf) oom = 1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n; ++i) {
            if (!buf) continue;
            const char *row = (const char *)x + (size_t)i * (size_t)row_stride * es;
            if (V < 1 || !oracle_rows_score_one(row, dtype, V, buf, &argmax[i], &conf[i])) {
                argmax[i] = -1;
                conf[i] = NAN;
                bad += 1;
            }
        }
        free(buf);
    }
    return oom ? -1 : bad;
}
