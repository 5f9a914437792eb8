/*
 * CPU oracle for FP32 row reductions -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may link or call this code.  The GPU library never does, and this code
 * shares nothing with it (no headers, helpers or tables).
 *
 * Every function works on a row-major rows x cols FP32 tensor (row stride =
 * cols).  The "_f64" functions promote each input to double, accumulate with
 * a plain left-to-right loop in double and return double results: they are
 * the plain definitions of the operations on the page "TIRx Metal reduction
 * lowering" (LuisaCompute), section 1 (row softmax and cross-entropy sources),
 * section 5.1 (two-pass LayerNorm statistics) and section 5.2 (guarded label
 * gather).  RMSNorm has no formula on the pages; its reading is stated below.
 *
 * The "_fold_f32" functions replay the ordered_fold policy (the pages'
 * fold_left restriction, section 1) in FP32: one left-to-right chain per
 * row, each multiply and add rounded separately (this file is compiled with
 * -ffp-contract=off), IEEE division and square root.  Their results are the
 * one FP32 answer that ordered_fold admits for RMSNorm and LayerNorm.
 *
 * Pins: tests/test_oracle_pins.py checks every function against closed forms,
 * invariants, brute force on tiny rows and golden values (tests/golden/).
 */
#ifndef LR_ORACLE_H
#define LR_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* y[r][j] = exp(x[r][j] - max_r) / sum_k exp(x[r][k] - max_r)   (double) */
void oracle_softmax_f64(const float* x, double* y, int64_t rows, int64_t cols);

/* y[r][j] = gamma[j] * x[r][j] / sqrt(mean_k x[r][k]^2 + eps)    (double)
 * gamma == NULL means gamma = 1. */
void oracle_rmsnorm_f64(const float* x, const float* gamma, double* y,
                        int64_t rows, int64_t cols, double eps);

/* mu = mean_k x, var = mean_k (x - mu)^2 (biased, centred two-pass),
 * y = (x - mu) / sqrt(var + eps) * gamma + beta                  (double)
 * gamma == NULL means 1, beta == NULL means 0. */
void oracle_layernorm_f64(const float* x, const float* gamma, const float* beta,
                          double* y, int64_t rows, int64_t cols, double eps);

/* Fused residual LayerNorm: combined = fl32(x + res) elementwise (one FP32
 * addition), then y = layernorm(combined) as above (double).  sum_out, when
 * not NULL, receives combined (rows*cols floats).  Returns 0, or -1 when the
 * row scratch cannot be allocated. */
int oracle_add_layernorm_f64(const float* x, const float* res, const float* gamma,
                             const float* beta, double* y, float* sum_out,
                             int64_t rows, int64_t cols, double eps);

/* Row statistics of LayerNorm (mean and biased variance), for invariant tests. */
void oracle_layernorm_stats_f64(const float* x, double* mean, double* var,
                                int64_t rows, int64_t cols);

/* loss[r] = log(sum_k exp(x[r][k] - m)) + m - sel,  m = max_k x[r][k],
 * sel = x[r][label[r]] if 0 <= label[r] < cols (int64 compare), else 0. */
void oracle_cross_entropy_f64(const float* logits, const int64_t* labels,
                              double* losses, int64_t rows, int64_t cols);

/* out[r] = sum_j x[r][j]   (double) */
void oracle_row_sum_f64(const float* x, double* out, int64_t rows, int64_t cols);

/* mins[r] = min_j x[r][j], maxs[r] = max_j x[r][j] (exact; either may be NULL). */
void oracle_row_minmax_f32(const float* x, float* mins, float* maxs, int64_t rows, int64_t cols);

/* ordered_fold replay in FP32 (see above). */
void oracle_rmsnorm_fold_f32(const float* x, const float* gamma, float* y,
                             int64_t rows, int64_t cols, float eps);
void oracle_layernorm_fold_f32(const float* x, const float* gamma,
                               const float* beta, float* y, int64_t rows,
                               int64_t cols, float eps);
/* The FP32 left fold of one row: sum_{j in order} c_j with c_j = x_j (kind 0),
 * x_j*x_j (kind 1).  Exposed so tests can pin the fold order directly. */
float oracle_fold_left_f32(const float* x, int64_t n, int kind);

/* The other ordered policies of section 1 ("fold_right", "ordered_tree"):
 * fold_right takes the chain from the right end (acc = c_j + acc,
 * j = n-1 .. 0, from +0.0f).  ordered_tree (reading: the pairwise tree in
 * index order) pads the contributions with -0.0f (the exact add identity) to the next power of two
 * and adds adjacent pairs level by level.  Both round every operation. */
float oracle_fold_right_f32(const float* x, int64_t n, int kind);
float oracle_tree_f32(const float* x, int64_t n, int kind);
/* policy: 1 fold_left, 2 ordered_tree, 3 fold_right. */
float oracle_ordered_sum_f32(const float* x, int64_t n, int kind, int policy);
void oracle_rmsnorm_ordered_f32(const float* x, const float* gamma, float* y, int64_t rows,
                                int64_t cols, float eps, int policy);
/* Returns 0, or -1 when the row scratch cannot be allocated. */
int oracle_layernorm_ordered_f32(const float* x, const float* gamma, const float* beta, float* y,
                                 int64_t rows, int64_t cols, float eps, int policy);

#ifdef __cplusplus
}
#endif

#endif
