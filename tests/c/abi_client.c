/* A plain C client of liblr.so: the C ABI (include/lr.h) used with device
 * memory from the HIP runtime and no Python or torch.  It runs a row softmax,
 * an RMSNorm and a cross-entropy on small inputs, checks them against
 * properties that hold exactly or nearly (rows of the softmax sum to one; the
 * RMSNorm of a constant row c is gamma * sign(c) at eps = 0; the
 * cross-entropy of a uniform row is log(cols)), runs a fused residual
 * LayerNorm whose rows are split across workgroups through lr_run_f32 and a
 * workspace, and checks that an invalid call returns its status before
 * touching the device.  Prints "abi_client
 * ok" and exits 0 on success. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "lr.h"

#define CHECK_HIP(e)                                                       \
    do {                                                                   \
        hipError_t e_ = (e);                                               \
        if (e_ != hipSuccess) {                                            \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

#define CHECK_LR(s)                                                              \
    do {                                                                         \
        lr_status s_ = (s);                                                      \
        if (s_ != LR_OK) {                                                       \
            fprintf(stderr, "%s at line %d\n", lr_status_string(s_), __LINE__); \
            return 1;                                                            \
        }                                                                        \
    } while (0)

int main(void) {
    enum { ROWS = 5, COLS = 1000 };
    const size_t n = (size_t)ROWS * COLS;
    float* hx = (float*)malloc(n * sizeof(float));
    float* hy = (float*)malloc(n * sizeof(float));
    float hg[COLS];
    int64_t hl[ROWS];
    float hloss[ROWS];
    if (!hx || !hy) return 1;
    for (size_t i = 0; i < n; ++i) hx[i] = (float)((int)(i * 2654435761u % 2001u) - 1000) / 250.0f;
    for (int j = 0; j < COLS; ++j) hg[j] = 0.5f + (float)j / COLS;

    float *dx, *dy, *dg, *dloss;
    int64_t* dl;
    CHECK_HIP(hipMalloc((void**)&dx, n * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&dy, n * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&dg, COLS * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&dl, ROWS * sizeof(int64_t)));
    CHECK_HIP(hipMalloc((void**)&dloss, ROWS * sizeof(float)));
    CHECK_HIP(hipMemcpy(dx, hx, n * sizeof(float), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dg, hg, COLS * sizeof(float), hipMemcpyHostToDevice));

    /* softmax: every row sums to 1 */
    for (int pol = LR_UNORDERED_TREE; pol <= LR_FOLD_RIGHT; ++pol) {
        CHECK_LR(lr_softmax_f32(dx, dy, ROWS, COLS, (lr_reduction_policy)pol, NULL));
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(hy, dy, n * sizeof(float), hipMemcpyDeviceToHost));
        for (int r = 0; r < ROWS; ++r) {
            double s = 0.0;
            for (int j = 0; j < COLS; ++j) s += hy[(size_t)r * COLS + j];
            if (fabs(s - 1.0) > 1e-5) {
                fprintf(stderr, "softmax row %d sums to %.9g (policy %d)\n", r, s, pol);
                return 1;
            }
        }
    }

    /* RMSNorm of a constant row c at eps = 0 is gamma * sign(c) */
    for (size_t i = 0; i < n; ++i) hx[i] = (i / COLS) % 2 ? 3.0f : -0.25f;
    CHECK_HIP(hipMemcpy(dx, hx, n * sizeof(float), hipMemcpyHostToDevice));
    CHECK_LR(lr_rmsnorm_f32(dx, dg, dy, ROWS, COLS, 0.0f, LR_ORDERED_FOLD, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hy, dy, n * sizeof(float), hipMemcpyDeviceToHost));
    for (int r = 0; r < ROWS; ++r)
        for (int j = 0; j < COLS; ++j) {
            const float want = (r % 2 ? 1.0f : -1.0f) * hg[j];
            if (fabsf(hy[(size_t)r * COLS + j] - want) > 1e-6f * fabsf(want)) {
                fprintf(stderr, "rmsnorm (%d,%d) = %.9g, want %.9g\n", r, j, hy[(size_t)r * COLS + j], want);
                return 1;
            }
        }

    /* cross-entropy of a uniform row is log(cols), wherever the label points */
    for (size_t i = 0; i < n; ++i) hx[i] = 1.5f;
    for (int r = 0; r < ROWS; ++r) hl[r] = r == 3 ? -1 : (int64_t)r * 199;
    CHECK_HIP(hipMemcpy(dx, hx, n * sizeof(float), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dl, hl, sizeof(hl), hipMemcpyHostToDevice));
    CHECK_LR(lr_cross_entropy_f32(dx, dl, dloss, ROWS, COLS, LR_UNORDERED_TREE, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hloss, dloss, sizeof(hloss), hipMemcpyDeviceToHost));
    for (int r = 0; r < ROWS; ++r) {
        /* label -1 is out of range: the guard selects 0, so the loss is the log-sum-exp */
        const double want = log((double)COLS) + (r == 3 ? 1.5 : 0.0);
        if (fabs(hloss[r] - want) > 1e-5 * want) {
            fprintf(stderr, "cross-entropy row %d = %.9g, want %.9g\n", r, hloss[r], want);
            return 1;
        }
    }

    /* The fused residual LayerNorm through lr_run_f32 with a workspace: 8
     * rows of 4096 are too few to fill the device, so the automatic plan
     * splits each row over several workgroups.  x alternates +2, -2 and the
     * residual is 0: every segment's mean is 0 and its sum of squared
     * deviations is exact, so y = +-1 (eps = 0). */
    {
        enum { LR_ROWS = 8, LR_COLS = 4096 };
        const size_t m = (size_t)LR_ROWS * LR_COLS;
        float* hz = (float*)malloc(m * sizeof(float));
        float *dz, *dr, *dw;
        uint64_t ws = 0;
        lr_plan plan;
        lr_device_facts facts;
        if (!hz) return 1;
        for (size_t i = 0; i < m; ++i) hz[i] = (i % 2) ? -2.0f : 2.0f;
        CHECK_LR(lr_device_facts_query(&facts));
        CHECK_LR(lr_plan_for_device_ws(&facts, LR_OP_ADD_LAYERNORM, LR_ROWS, LR_COLS, LR_UNORDERED_TREE, 1, &plan));
        if (plan.family != LR_FAMILY_SPLIT || plan.splits < 2) {
            fprintf(stderr, "expected a split plan, got family %d\n", plan.family);
            return 1;
        }
        CHECK_LR(lr_workspace_query(LR_OP_ADD_LAYERNORM, LR_ROWS, LR_COLS, LR_UNORDERED_TREE, &ws));
        if (ws < lr_plan_workspace_bytes(&plan, LR_ROWS) || ws == 0) return 1;
        CHECK_HIP(hipMalloc((void**)&dz, m * sizeof(float)));
        CHECK_HIP(hipMalloc((void**)&dw, ws));
        CHECK_HIP(hipMalloc((void**)&dr, m * sizeof(float)));
        CHECK_HIP(hipMemcpy(dz, hz, m * sizeof(float), hipMemcpyHostToDevice));
        CHECK_HIP(hipMemset(dr, 0, m * sizeof(float)));
        lr_tensors t = {0};
        t.x = dz;
        t.residual = dr;
        t.y = dz; /* in place */
        CHECK_LR(lr_run_f32(LR_OP_ADD_LAYERNORM, &t, LR_ROWS, LR_COLS, 0.0f, LR_UNORDERED_TREE, NULL, dw, ws, NULL));
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(hz, dz, m * sizeof(float), hipMemcpyDeviceToHost));
        for (size_t i = 0; i < m; ++i) {
            const float want = (i % 2) ? -1.0f : 1.0f;
            if (fabsf(hz[i] - want) > 1e-6f) {
                fprintf(stderr, "split add_layernorm [%zu] = %.9g, want %.9g\n", i, hz[i], want);
                return 1;
            }
        }
        /* a member the operation does not use is an error */
        t.sums = dy;
        if (lr_run_f32(LR_OP_ADD_LAYERNORM, &t, LR_ROWS, LR_COLS, 0.0f, LR_UNORDERED_TREE, NULL, dw, ws, NULL) !=
            LR_ERR_INVALID_ARGUMENT)
            return 1;
        CHECK_HIP(hipFree(dz));
        CHECK_HIP(hipFree(dr));
        CHECK_HIP(hipFree(dw));
        free(hz);
    }

    /* an invalid call is rejected before any device work */
    if (lr_softmax_f32(NULL, dy, ROWS, COLS, LR_UNORDERED_TREE, NULL) != LR_ERR_NULL_POINTER) return 1;
    if (lr_softmax_f32(dx, dx + 4, ROWS, COLS, LR_UNORDERED_TREE, NULL) != LR_ERR_ALIASING) return 1;

    CHECK_HIP(hipFree(dx));
    CHECK_HIP(hipFree(dy));
    CHECK_HIP(hipFree(dg));
    CHECK_HIP(hipFree(dl));
    CHECK_HIP(hipFree(dloss));
    free(hx);
    free(hy);
    printf("abi_client ok (%s)\n", lr_version());
    return 0;
}
