/* dllm_step called from plain C with the HIP runtime API alone (no Python, no PyTorch).
 *
 * Test program: the GPU test tests/test_gpu_c_program.py runs it.  Four rows of a box with L = 8
 * slots, V = 1000 fp32 logits.  Slot (r, j) holds T(r, j) at vocabulary index a(r, j) and 0
 * elsewhere, so its confidence has a closed form:
 *   c = 1 / (1 + (V - 1) exp(-T))      (the softmax probability of the argmax token)
 * and it is unmasked when c > tau ([FDFO] "FDFO: 让 dLLM 推理从「整批等最慢」变成「谁先完成谁先走」"
 * §工程设计一, LowConfidence; [DiLaServe] "DiLaServe: High SLO Attainment Serving for Diffusion
 * Language Models" §三 3.1).  With tau = 0.9 that is T > ln(9 (V - 1)) = 9.10.  Row 3 has every
 * T below that, so its single most confident slot is unmasked instead.  Rows 0-2 unmask j >= 5
 * (T = 5 + j); row 3 unmasks j = 7 (the largest T).  Slot j = 7 of row 2 is not masked on entry
 * and must be left alone.  Prints "ok" and exits 0, or the first mismatch and exits 1. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dllm.h"

enum { ROWS = 4, L = 8, V = 1000, W = 20 };

static int check_hip(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        printf("%s: %s\n", what, hipGetErrorString(e));
        return 1;
    }
    return 0;
}

static double T_of(int r, int j) { return r == 3 ? 1.0 + 0.5 * j : 5.0 + j; }
static int a_of(int r, int j) { return (r * 131 + j * 37 + 11) % V; }

int main(void) {
    static float logits[ROWS][L][V];
    static int32_t ids[ROWS][W];
    uint8_t mask[ROWS][L];
    float tau[ROWS];
    int r, j, v;
    for (r = 0; r < ROWS; ++r) {
        tau[r] = 0.9f;
        for (j = 0; j < W; ++j) ids[r][j] = 7;
        for (j = 0; j < L; ++j) {
            for (v = 0; v < V; ++v) logits[r][j][v] = 0.0f;
            logits[r][j][a_of(r, j)] = (float)T_of(r, j);
            mask[r][j] = !(r == 2 && j == 7);
        }
    }
    const size_t ws_bytes = dllm_step_workspace_bytes(ROWS, L, V, DLLM_FP32);
    void *d_logits, *d_ids, *d_mask_in, *d_mask_out, *d_tau, *d_conf, *d_arg, *d_done, *d_acc, *d_ws, *d_status;
    if (check_hip(hipMalloc(&d_logits, sizeof logits), "hipMalloc") || check_hip(hipMalloc(&d_ids, sizeof ids), "hipMalloc") ||
        check_hip(hipMalloc(&d_mask_in, sizeof mask), "hipMalloc") ||
        check_hip(hipMalloc(&d_mask_out, sizeof mask), "hipMalloc") ||
        check_hip(hipMalloc(&d_tau, sizeof tau), "hipMalloc") ||
        check_hip(hipMalloc(&d_conf, ROWS * L * sizeof(float)), "hipMalloc") ||
        check_hip(hipMalloc(&d_arg, ROWS * L * sizeof(int32_t)), "hipMalloc") ||
        check_hip(hipMalloc(&d_done, ROWS), "hipMalloc") || check_hip(hipMalloc(&d_acc, ROWS * sizeof(int32_t)), "hipMalloc") ||
        check_hip(hipMalloc(&d_ws, ws_bytes), "hipMalloc") || check_hip(hipMalloc(&d_status, sizeof(int32_t)), "hipMalloc"))
        return 1;
    const int32_t zero = 0;
    if (check_hip(hipMemcpy(d_logits, logits, sizeof logits, hipMemcpyHostToDevice), "hipMemcpy") ||
        check_hip(hipMemcpy(d_ids, ids, sizeof ids, hipMemcpyHostToDevice), "hipMemcpy") ||
        check_hip(hipMemcpy(d_mask_in, mask, sizeof mask, hipMemcpyHostToDevice), "hipMemcpy") ||
        check_hip(hipMemcpy(d_tau, tau, sizeof tau, hipMemcpyHostToDevice), "hipMemcpy") ||
        check_hip(hipMemcpy(d_status, &zero, sizeof zero, hipMemcpyHostToDevice), "hipMemcpy"))
        return 1;

    dllm_status rc = dllm_step(NULL, d_logits, DLLM_FP32, V, (int64_t)L * V, ROWS, L, V, (int32_t *)d_ids, W,
                               (const uint8_t *)d_mask_in, (uint8_t *)d_mask_out, (const float *)d_tau, NULL, NULL,
                               (float *)d_conf, (int32_t *)d_arg, (uint8_t *)d_done, (int32_t *)d_acc, d_ws, ws_bytes,
                               (int32_t *)d_status);
    if (rc != DLLM_OK) {
        printf("dllm_step: %d %s\n", (int)rc, dllm_last_error());
        return 1;
    }
    if (check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize")) return 1;

    int32_t ids_out[ROWS][W], arg[ROWS][L], acc[ROWS], status;
    float conf[ROWS][L];
    uint8_t mask_out[ROWS][L], done[ROWS];
    if (check_hip(hipMemcpy(ids_out, d_ids, sizeof ids_out, hipMemcpyDeviceToHost), "hipMemcpy") ||
        check_hip(hipMemcpy(arg, d_arg, sizeof arg, hipMemcpyDeviceToHost), "hipMemcpy") ||
        check_hip(hipMemcpy(conf, d_conf, sizeof conf, hipMemcpyDeviceToHost), "hipMemcpy") ||
        check_hip(hipMemcpy(mask_out, d_mask_out, sizeof mask_out, hipMemcpyDeviceToHost), "hipMemcpy") ||
        check_hip(hipMemcpy(done, d_done, sizeof done, hipMemcpyDeviceToHost), "hipMemcpy") ||
        check_hip(hipMemcpy(acc, d_acc, sizeof acc, hipMemcpyDeviceToHost), "hipMemcpy") ||
        check_hip(hipMemcpy(&status, d_status, sizeof status, hipMemcpyDeviceToHost), "hipMemcpy"))
        return 1;
    if (status != 0) {
        printf("device status %d\n", (int)status);
        return 1;
    }
    for (r = 0; r < ROWS; ++r) {
        int n_left = 0;
        for (j = 0; j < L; ++j) {
            const int masked = mask[r][j];
            const double c = 1.0 / (1.0 + (V - 1) * exp(-T_of(r, j)));
            const int unmask = masked && (r == 3 ? j == 7 : T_of(r, j) > log(9.0 * (V - 1)));
            if (masked) {
                if (arg[r][j] != a_of(r, j) || fabs(conf[r][j] - c) > 1e-5) {
                    printf("row %d slot %d: argmax %d (want %d), conf %.9g (want %.9g)\n", r, j, (int)arg[r][j],
                           a_of(r, j), conf[r][j], c);
                    return 1;
                }
            } else if (arg[r][j] != -1 || conf[r][j] != -1.0f) {
                printf("row %d slot %d: not masked but scored\n", r, j);
                return 1;
            }
            if (mask_out[r][j] != (masked && !unmask)) {
                printf("row %d slot %d: mask_out %d\n", r, j, (int)mask_out[r][j]);
                return 1;
            }
            if (ids_out[r][W - L + j] != (unmask ? a_of(r, j) : 7)) {
                printf("row %d slot %d: id %d\n", r, j, (int)ids_out[r][W - L + j]);
                return 1;
            }
            n_left += masked && !unmask;
        }
        for (j = 0; j < W - L; ++j)
            if (ids_out[r][j] != 7) {
                printf("row %d column %d outside the block was written\n", r, j);
                return 1;
            }
        if (done[r] != (n_left == 0) || acc[r] != (n_left == 0 ? L : 0)) {
            printf("row %d: done %d accept %d\n", r, (int)done[r], (int)acc[r]);
            return 1;
        }
    }
    printf("ok: %d rows, L=%d, V=%d fp32 through the C ABI\n", ROWS, L, V);
    return 0;
}
