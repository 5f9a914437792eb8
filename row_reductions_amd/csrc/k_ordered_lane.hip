// ORDERED family, one lane per row, for narrow rows (lanes_per_row = 1): the
// ordered reduction policies of "TIRx Metal reduction lowering", section 1,
// exactly as in k_ordered.hip -- fold_left and fold_right from +0.0f, the
// pairwise tree in index order over the contributions padded with the add
// identity -0.0f -- but with each lane owning one whole row.  Lane l of a
// workgroup of Q lanes takes row blockIdx.x * Q + l and keeps it in
// registers (N4 16-byte chunks, cols <= 4 N4, the row 16-byte aligned), so
// every ordered sum is that lane's own chain or tree over its registers and
// the elementwise passes read registers: 64 rows progress per wave, with no
// LDS and no cross-lane operation.  A row wider than a few chunks is better
// served by a wave (k_ordered.hip).  Same operation sequence as k_ordered.hip
// (each multiply and add rounded on its own, IEEE division and square root,
// precise expf / logf), so the results are the same bits.
#pragma clang fp contract(off)

#include "lr_device.hpp"
#include "lr_internal.hpp"

namespace lr {
namespace {

// The FP32 sum of c[0 .. cols) in the order of policy POL (N: a power of two
// >= cols; slots past cols are not read by the folds and are the tree's
// padding).
template <int POL, int N>
__device__ __forceinline__ float lane_sum(const float (&c)[N], int cols) {
    if constexpr (POL == kPolFoldLeft) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j)
            if (j < cols) acc = acc + c[j];
        return acc;
    } else if constexpr (POL == kPolFoldRight) {
        float acc = 0.0f;
#pragma unroll
        for (int j = N - 1; j >= 0; --j)
            if (j < cols) acc = c[j] + acc;
        return acc;
    } else {
        float t[N];
#pragma unroll
        for (int j = 0; j < N; ++j) t[j] = j < cols ? c[j] : -0.0f;
#pragma unroll
        for (int w = N / 2; w >= 1; w /= 2) {
#pragma unroll
            for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
        }
        return t[0];
    }
}

// Row r's chunk c (16 bytes) read as four floats: one 128-bit access when
// the pointer's rows are 16-byte aligned (AL), else four.
template <bool AL>
__device__ __forceinline__ float4 chunk_ld(const float* p, int c, bool cached) {
    if constexpr (AL) {
        return cached ? ld4_cached(reinterpret_cast<const float4*>(p) + c) : ld4(reinterpret_cast<const float4*>(p) + c);
    } else {
        return make_float4(p[4 * c], p[4 * c + 1], p[4 * c + 2], p[4 * c + 3]);
    }
}

template <bool AL>
__device__ __forceinline__ void chunk_st(float* p, int c, float4 v) {
    if constexpr (AL) {
        st4(reinterpret_cast<float4*>(p) + c, v);
    } else {
        p[4 * c] = v.x;
        p[4 * c + 1] = v.y;
        p[4 * c + 2] = v.z;
        p[4 * c + 3] = v.w;
    }
}

// AL: y, gamma, beta, the residual and the combined output are 16-byte
// aligned too (x always is: the plan requires it).
template <int OP, int POL, int N4, bool AL>
__global__ void __launch_bounds__(256) k_ordered_lane(const KArgs a) {
    constexpr int N = 4 * N4;
    const int64_t row = (int64_t)blockIdx.x * a.Q + threadIdx.x;
    if (row >= a.rows) return;  // no barrier and no cross-lane operation in this kernel
    const int cols = a.cols;
    const int nv = cols / kVec;  // whole chunks: cols % 4 == 0
    const float n = (float)cols;
    const int64_t roff = row * (int64_t)cols;
    const float* xr = a.x + roff;

    // the row (x + residual for the fused residual LayerNorm), in registers
    float x[N];
#pragma unroll
    for (int c = 0; c < N4; ++c) {
        float4 q = splat4(0.0f);
        if (c < nv) {
            q = chunk_ld<true>(xr, c, false);
            if constexpr (OP == kAddLayerNorm) {
                const float4 r = chunk_ld<AL>(a.residual + roff, c, false);
                q = make_float4(q.x + r.x, q.y + r.y, q.z + r.z, q.w + r.w);
                if (a.sum_out != nullptr) chunk_st<AL>(a.sum_out + roff, c, q);
            }
        }
        x[4 * c] = q.x;
        x[4 * c + 1] = q.y;
        x[4 * c + 2] = q.z;
        x[4 * c + 3] = q.w;
    }

    if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < N; ++j)
            if (j < cols) m = fmaxf(m, x[j]);
        float e[N];
#pragma unroll
        for (int j = 0; j < N; ++j) e[j] = j < cols ? expf(x[j] - m) : 0.0f;
        const float s = lane_sum<POL>(e, cols);
        if constexpr (OP == kCrossEntropy) {
            const int64_t lab = a.labels[row];
            const float sel = (lab >= 0 && lab < (int64_t)cols) ? xr[lab] : 0.0f;
            a.losses[row] = logf(s) + (m - sel);
        } else {
#pragma unroll
            for (int c = 0; c < N4; ++c)
                if (c < nv)
                    chunk_st<AL>(a.y + roff, c,
                                 make_float4(e[4 * c] / s, e[4 * c + 1] / s, e[4 * c + 2] / s, e[4 * c + 3] / s));
        }
    } else if constexpr (OP == kRowSum) {
        a.sums[row] = lane_sum<POL>(x, cols);
    } else if constexpr (OP == kRowMinMax) {
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if (j < cols) {
                lo = fmin2(lo, x[j]);
                hi = fmax2(hi, x[j]);
            }
        }
        if (a.mins) a.mins[row] = lo;
        if (a.maxs) a.maxs[row] = hi;
    } else if constexpr (OP == kRmsNorm) {
        float q[N];
#pragma unroll
        for (int j = 0; j < N; ++j) q[j] = x[j] * x[j];
        const float ms = lane_sum<POL>(q, cols) / n;
        const float r = 1.0f / sqrtf(ms + a.eps);
#pragma unroll
        for (int c = 0; c < N4; ++c) {
            if (c < nv) {
                float4 t = make_float4(x[4 * c] * r, x[4 * c + 1] * r, x[4 * c + 2] * r, x[4 * c + 3] * r);
                if (a.gamma) {
                    const float4 g = chunk_ld<AL>(a.gamma, c, true);
                    t = make_float4(t.x * g.x, t.y * g.y, t.z * g.z, t.w * g.w);
                }
                chunk_st<AL>(a.y + roff, c, t);
            }
        }
    } else {  // LayerNorm, fused residual LayerNorm
        const float mu = lane_sum<POL>(x, cols) / n;
        float q[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const float d = x[j] - mu;
            q[j] = d * d;
        }
        const float var = lane_sum<POL>(q, cols) / n;
        const float r = 1.0f / sqrtf(var + a.eps);
#pragma unroll
        for (int c = 0; c < N4; ++c) {
            if (c < nv) {
                float4 t = make_float4((x[4 * c] - mu) * r, (x[4 * c + 1] - mu) * r, (x[4 * c + 2] - mu) * r,
                                       (x[4 * c + 3] - mu) * r);
                if (a.gamma) {
                    const float4 g = chunk_ld<AL>(a.gamma, c, true);
                    t = make_float4(t.x * g.x, t.y * g.y, t.z * g.z, t.w * g.w);
                }
                if (a.beta) {
                    const float4 b = chunk_ld<AL>(a.beta, c, true);
                    t = make_float4(t.x + b.x, t.y + b.y, t.z + b.z, t.w + b.w);
                }
                chunk_st<AL>(a.y + roff, c, t);
            }
        }
    }
}

template <int OP, int POL, bool AL>
hipError_t launch_lane_n4(const KArgs& a, const lr_plan& p, hipStream_t s) {
    const dim3 grid((unsigned)p.blocks), block(p.threads_per_block);
    switch (p.chunks_per_lane) {
        case 1: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 1, AL>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 2, AL>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 4, AL>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 8, AL>), grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 16, AL>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int POL, bool AL>
hipError_t launch_lane_op(int op, const KArgs& a, const lr_plan& p, hipStream_t s) {
    switch (op) {
        case kSoftmax: return launch_lane_n4<kSoftmax, POL, AL>(a, p, s);
        case kRmsNorm: return launch_lane_n4<kRmsNorm, POL, AL>(a, p, s);
        case kLayerNorm: return launch_lane_n4<kLayerNorm, POL, AL>(a, p, s);
        case kCrossEntropy: return launch_lane_n4<kCrossEntropy, POL, AL>(a, p, s);
        case kAddLayerNorm: return launch_lane_n4<kAddLayerNorm, POL, AL>(a, p, s);
        case kRowSum: return launch_lane_n4<kRowSum, POL, AL>(a, p, s);
        case kRowMinMax: return launch_lane_n4<kRowMinMax, POL, AL>(a, p, s);
        default: return hipErrorInvalidValue;
    }
}

template <int POL>
hipError_t launch_lane_pol(int op, const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    return aligned ? launch_lane_op<POL, true>(op, a, p, s) : launch_lane_op<POL, false>(op, a, p, s);
}

}  // namespace

hipError_t launch_ordered_lane(int op, int policy, const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    switch (policy) {
        case kPolFoldLeft: return launch_lane_pol<kPolFoldLeft>(op, a, p, aligned, s);
        case kPolTree: return launch_lane_pol<kPolTree>(op, a, p, aligned, s);
        case kPolFoldRight: return launch_lane_pol<kPolFoldRight>(op, a, p, aligned, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lr
