// Kernel entry.  The kernel-argument fields a kernel needs before its first
// row load travel as its nine leading arguments, ahead of the whole KArgs.
// The build preloads the first nine kernel arguments into scalar registers
// at wave launch (gfx950 kernel-argument preloading, hipcc
// -mllvm -amdgpu-kernarg-preload-count=9), so a wave computes its row's
// address and issues the row loads without first waiting for a read of the
// kernel-argument segment; the rest of KArgs is read while those loads are
// in flight.  (The code object also carries a prologue that reads the
// preloaded arguments from memory, for firmware without preloading.)
// Measured on MI355X at 768 x 6144, cold launches, against the same kernels
// reading every field from KArgs: softmax 6.68 -> 6.48 us, RMSNorm 6.84 ->
// 6.68 us, LayerNorm 6.93 -> 6.78 us.
#pragma once

#include <hip/hip_runtime.h>

#include "lr_internal.hpp"

// Parameter list of a kernel entry: the nine preloaded fields, then KArgs.
#define LR_ENTRY_PARAMS                                                                                   \
    const float *e_x, int64_t e_rows, int32_t e_cols, int32_t e_S, int32_t e_Q, int32_t e_magic,          \
        const float *e_gamma, const float *e_beta, const float *e_residual, const lr::KArgs e_a

// Inside an entry: its KArgs, the leading fields taken from the preloaded
// arguments (the copies in e_a are then never read).
#define LR_ENTRY_KARGS \
    lr::entry_kargs(e_a, e_x, e_rows, e_cols, e_S, e_Q, e_magic, e_gamma, e_beta, e_residual)

// Argument list of a launch of an entry with KArgs `a`.
#define LR_ENTRY_ARGS(a) \
    (a).x, (a).rows, (a).cols, (a).S, (a).Q, (a).team_magic, (a).gamma, (a).beta, (a).residual, (a)

namespace lr {

__device__ __forceinline__ KArgs entry_kargs(KArgs a, const float* x, int64_t rows, int32_t cols, int32_t S,
                                             int32_t Q, int32_t magic, const float* gamma, const float* beta,
                                             const float* residual) {
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.S = S;
    a.Q = Q;
    a.team_magic = magic;
    a.gamma = gamma;
    a.beta = beta;
    a.residual = residual;
    return a;
}

}  // namespace lr
