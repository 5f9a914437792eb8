/*
 * CPU oracle for FP32 row reductions -- TEST INFRASTRUCTURE ONLY.
 * Definitions and citations are in oracle.h.  Build with
 *   gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared oracle.c -o liboracle.so -lm
 * (no fast-math: the FP32 replay needs every operation rounded on its own).
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>

/* Row softmax: the source program of section 1 of "TIRx Metal reduction
 * lowering" takes exp of the row minus its maximum, then divides by the sum
 * of those exponentials.  Computed here in double. */
void oracle_softmax_f64(const float* x, double* y, int64_t rows, int64_t cols) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        double* yr = y + r * cols;
        double m = -INFINITY;
        for (int64_t j = 0; j < cols; ++j) {
            if ((double)xr[j] > m) m = (double)xr[j];
        }
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            double e = exp((double)xr[j] - m);
            yr[j] = e;
            s += e;
        }
        for (int64_t j = 0; j < cols; ++j) yr[j] = yr[j] / s;
    }
}

/* RMSNorm: not written out on the pages (only timed).  Reading used: the
 * mean of squares over the row, eps added inside the square root (as the
 * LayerNorm source of section 5.1 adds its eps), gamma applied last. */
void oracle_rmsnorm_f64(const float* x, const float* gamma, double* y,
                        int64_t rows, int64_t cols, double eps) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        double* yr = y + r * cols;
        double ss = 0.0;
        for (int64_t j = 0; j < cols; ++j) ss += (double)xr[j] * (double)xr[j];
        double ms = ss / (double)cols;
        double d = sqrt(ms + eps);
        for (int64_t j = 0; j < cols; ++j) {
            double g = gamma ? (double)gamma[j] : 1.0;
            yr[j] = g * ((double)xr[j] / d);
        }
    }
}

void oracle_layernorm_stats_f64(const float* x, double* mean, double* var,
                                int64_t rows, int64_t cols) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) s += (double)xr[j];
        double mu = s / (double)cols;
        double q = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            double c = (double)xr[j] - mu;
            q += c * c;
        }
        mean[r] = mu;
        var[r] = q / (double)cols;
    }
}

/* LayerNorm: section 5.1 of "TIRx Metal reduction lowering" -- mean = sum/width,
 * centred = x - mean, variance = sum(centred^2)/width, output centred /
 * sqrt(variance + eps); the section 8 test applies a per-column affine
 * (gamma, beta) to those outputs. */
void oracle_layernorm_f64(const float* x, const float* gamma, const float* beta,
                          double* y, int64_t rows, int64_t cols, double eps) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        double* yr = y + r * cols;
        double mu, var;
        oracle_layernorm_stats_f64(xr, &mu, &var, 1, cols);
        double d = sqrt(var + eps);
        for (int64_t j = 0; j < cols; ++j) {
            double g = gamma ? (double)gamma[j] : 1.0;
            double b = beta ? (double)beta[j] : 0.0;
            yr[j] = ((double)xr[j] - mu) / d * g + b;
        }
    }
}

/* Fused residual LayerNorm: section 5.1 of "TIRx Metal reduction lowering"
 * forms combined = X + residual elementwise in the tile's FP32 arithmetic and
 * takes the two-pass LayerNorm of combined (mean, centred values, variance,
 * centred / sqrt(variance + eps)).  The affine step and the optional copy of
 * combined are this library's additions; with gamma = beta = NULL the result
 * is the pages' program.  The FP32 sum is formed here with one float
 * addition per element (C float arithmetic, no contraction), the rest in
 * double as oracle_layernorm_f64. */
int oracle_add_layernorm_f64(const float* x, const float* res, const float* gamma,
                             const float* beta, double* y, float* sum_out,
                             int64_t rows, int64_t cols, double eps) {
    float* c = (float*)malloc((size_t)cols * sizeof(float));
    if (c == NULL) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        const float* rr = res + r * cols;
        for (int64_t j = 0; j < cols; ++j) {
            const float sum = xr[j] + rr[j];
            c[j] = sum;
        }
        oracle_layernorm_f64(c, gamma, beta, y + r * cols, 1, cols, eps);
        if (sum_out != NULL) {
            for (int64_t j = 0; j < cols; ++j) sum_out[r * cols + j] = c[j];
        }
    }
    free(c);
    return 0;
}

/* Cross-entropy: section 1 composes peak = max(row), total = sum exp(row -
 * peak), selected = gather(row, label) and stores log(total) + peak -
 * selected; section 5.2 makes the gather a guarded read of the logits tensor
 * with fill 0 when the label is outside [0, cols). */
void oracle_cross_entropy_f64(const float* logits, const int64_t* labels,
                              double* losses, int64_t rows, int64_t cols) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = logits + r * cols;
        double m = -INFINITY;
        for (int64_t j = 0; j < cols; ++j) {
            if ((double)xr[j] > m) m = (double)xr[j];
        }
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) s += exp((double)xr[j] - m);
        int64_t l = labels[r];
        double sel = (l >= 0 && l < cols) ? (double)xr[l] : 0.0;
        losses[r] = log(s) + m - sel;
    }
}

/* Row sum (the plain add reduction; section 8 of "TIRx Metal reduction
 * lowering" checks row sums at widths 127, 257, 1024 and 4096):
 * out[r] = sum_j x[r][j], accumulated in double. */
void oracle_row_sum_f64(const float* x, double* out, int64_t rows, int64_t cols) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j) s += (double)xr[j];
        out[r] = s;
    }
}

/* Row minimum and maximum together (section 8: minimum and maximum of each
 * row in one pass, 7 x 1024).  Exact: both are input values. */
void oracle_row_minmax_f32(const float* x, float* mins, float* maxs, int64_t rows, int64_t cols) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        float lo = xr[0], hi = xr[0];
        for (int64_t j = 1; j < cols; ++j) {
            if (xr[j] < lo) lo = xr[j];
            if (xr[j] > hi) hi = xr[j];
        }
        if (mins != NULL) mins[r] = lo;
        if (maxs != NULL) maxs[r] = hi;
    }
}

/* ---------------------------------------------------------------------------
 * ordered_fold replay in FP32.  The pages' fold_left restriction (section 1
 * of "TIRx Metal reduction lowering") keeps a reduction as one ordered chain
 * and requires precise math; here each chain starts from the add identity
 * +0.0f and takes elements j = 0, 1, ..., n-1.
 * ------------------------------------------------------------------------- */
float oracle_fold_left_f32(const float* x, int64_t n, int kind) {
    float acc = 0.0f;
    for (int64_t j = 0; j < n; ++j) {
        float c = (kind == 1) ? x[j] * x[j] : x[j];
        acc = acc + c;
    }
    return acc;
}

/* fold_right: the same chain taken from the right end, acc = c_j + acc for
 * j = n-1, n-2, ..., 0, starting from +0.0f. */
float oracle_fold_right_f32(const float* x, int64_t n, int kind) {
    float acc = 0.0f;
    for (int64_t j = n - 1; j >= 0; --j) {
        float c = (kind == 1) ? x[j] * x[j] : x[j];
        acc = c + acc;
    }
    return acc;
}

/* ordered_tree (reading used: the pairwise tree in index order).  The row's
 * contributions c_0 .. c_{n-1} are padded with the add identity to the next
 * power of two; each level adds adjacent pairs, node 2i + node 2i+1, until
 * one value is left.  Every addition is one FP32 rounding.  The identity is
 * -0.0f, IEEE 754's exact one: x + (-0) = x for every x, whereas -0 + (+0)
 * rounds to +0, so with -0 padding a tree padded further (to any larger
 * power of two) gives the same bits, and a sum of negative zeros stays -0. */
float oracle_tree_f32(const float* x, int64_t n, int kind) {
    int64_t p = 1;
    while (p < n) p *= 2;
    float* t = (float*)malloc((size_t)p * sizeof(float));
    if (t == NULL) return NAN;
    for (int64_t j = 0; j < p; ++j) {
        float c = -0.0f;
        if (j < n) c = (kind == 1) ? x[j] * x[j] : x[j];
        t[j] = c;
    }
    for (int64_t w = p; w > 1; w /= 2) {
        for (int64_t i = 0; i < w / 2; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    }
    float out = t[0];
    free(t);
    return out;
}

/* The FP32 sum of one row's contributions in the order of `policy`:
 * 1 fold_left, 2 ordered_tree, 3 fold_right (kind as above). */
float oracle_ordered_sum_f32(const float* x, int64_t n, int kind, int policy) {
    if (policy == 2) return oracle_tree_f32(x, n, kind);
    if (policy == 3) return oracle_fold_right_f32(x, n, kind);
    return oracle_fold_left_f32(x, n, kind);
}

/* RMSNorm and LayerNorm replays under any ordered policy: the same FP32
 * operation sequence as the fold_left replays below, with each add
 * reduction taken in the policy's order. */
void oracle_rmsnorm_ordered_f32(const float* x, const float* gamma, float* y, int64_t rows,
                                int64_t cols, float eps, int policy) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        float* yr = y + r * cols;
        float acc = oracle_ordered_sum_f32(xr, cols, 1, policy);
        float ms = acc / (float)cols;
        float rr = 1.0f / sqrtf(ms + eps);
        for (int64_t j = 0; j < cols; ++j) {
            float t = xr[j] * rr;
            yr[j] = gamma ? t * gamma[j] : t;
        }
    }
}

int oracle_layernorm_ordered_f32(const float* x, const float* gamma, const float* beta, float* y,
                                 int64_t rows, int64_t cols, float eps, int policy) {
    float* d = (float*)malloc((size_t)cols * sizeof(float));
    if (d == NULL) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        float* yr = y + r * cols;
        float mu = oracle_ordered_sum_f32(xr, cols, 0, policy) / (float)cols;
        for (int64_t j = 0; j < cols; ++j) d[j] = xr[j] - mu;
        float var = oracle_ordered_sum_f32(d, cols, 1, policy) / (float)cols;
        float rr = 1.0f / sqrtf(var + eps);
        for (int64_t j = 0; j < cols; ++j) {
            float t = d[j] * rr;
            if (gamma) t = t * gamma[j];
            if (beta) t = t + beta[j];
            yr[j] = t;
        }
    }
    free(d);
    return 0;
}

void oracle_rmsnorm_fold_f32(const float* x, const float* gamma, float* y,
                             int64_t rows, int64_t cols, float eps) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        float* yr = y + r * cols;
        float acc = oracle_fold_left_f32(xr, cols, 1);
        float ms = acc / (float)cols;
        float rr = 1.0f / sqrtf(ms + eps);
        for (int64_t j = 0; j < cols; ++j) {
            float t = xr[j] * rr;
            yr[j] = gamma ? t * gamma[j] : t;
        }
    }
}

void oracle_layernorm_fold_f32(const float* x, const float* gamma,
                               const float* beta, float* y, int64_t rows,
                               int64_t cols, float eps) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        float* yr = y + r * cols;
        float mu = oracle_fold_left_f32(xr, cols, 0) / (float)cols;
        float acc = 0.0f;
        for (int64_t j = 0; j < cols; ++j) {
            float c = xr[j] - mu;
            acc = acc + c * c;
        }
        float var = acc / (float)cols;
        float rr = 1.0f / sqrtf(var + eps);
        for (int64_t j = 0; j < cols; ++j) {
            float t = (xr[j] - mu) * rr;
            if (gamma) t = t * gamma[j];
            if (beta) t = t + beta[j];
            yr[j] = t;
        }
    }
}
