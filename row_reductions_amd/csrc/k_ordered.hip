// ORDERED family: the ordered_fold policy (the pages' fold_left restriction,
// "TIRx Metal reduction lowering", section 1): every add fold of a row is one
// FP32 chain taken left to right, j = 0 .. cols-1, from the identity +0.0f,
// with each multiply and add rounded on its own; division and square root
// are IEEE (built with -ffp-contract=off and correctly rounded divide/sqrt);
// max folds are exact and use the wave tree.  The result does not depend on
// the plan, and RMSNorm / LayerNorm results are the unique FP32 values of the
// stated operation sequence.
//
// One wavefront owns a row.  Per 256-element slab, each lane loads four
// elements (coalesced 32-bit loads at 64*i + lane), computes their
// contributions elementwise in parallel and writes them to the wave's LDS
// slab; then every lane folds the slab in order from LDS (broadcast reads),
// so the serial chain costs one dependent add per element.
#pragma clang fp contract(off)

#include "lr_device.hpp"
#include "lr_internal.hpp"

namespace lr {

// Wave-local ordering point for the LDS slab: no instruction of this wave
// moves across it, and its LDS accesses complete in program order.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

enum Contrib : int { kValue = 0, kSquare = 1, kCentredSquare = 2, kExpShift = 3 };

template <int C>
__device__ __forceinline__ float contrib(float x, float ref) {
    if constexpr (C == kValue) return x;
    if constexpr (C == kSquare) return x * x;
    if constexpr (C == kCentredSquare) {
        const float d = x - ref;
        return d * d;
    }
    return expf(x - ref);  // kExpShift: ref is the row maximum
}

// Element j of the row: x_j, or the FP32 sum x_j + residual_j when the row
// is the fused residual LayerNorm's combined input (rr not null).
__device__ __forceinline__ float row_elem(const float* xr, const float* rr, int e) {
    return rr ? xr[e] + rr[e] : xr[e];
}

// acc_{j+1} = acc_j + c(x_j), j = 0 .. cols-1, in FP32, identical in all lanes.
template <int C>
__device__ float ordered_fold(const float* xr, const float* rr, int cols, float ref, float* slab, int lane) {
    float acc = 0.0f;
    for (int base = 0; base < cols; base += kSlab) {
        const int slab_id = base / kSlab;
#pragma unroll
        for (int i = 0; i < kSlab / kWave; ++i) {
            const int e = ordered_elem(slab_id, i, lane);
            if (e < cols) slab[kWave * i + lane] = contrib<C>(row_elem(xr, rr, e), ref);
        }
        wave_sync();
        const int n = min(kSlab, cols - base);
        int j = 0;
        for (; j + 4 <= n; j += 4) {
            const float4 c = *reinterpret_cast<const float4*>(slab + j);
            acc = acc + c.x;
            acc = acc + c.y;
            acc = acc + c.z;
            acc = acc + c.w;
        }
        for (; j < n; ++j) acc = acc + slab[j];
        wave_sync();
    }
    return acc;
}

template <int OP>
__global__ void __launch_bounds__(1024) k_ordered(const KArgs a) {
    __shared__ __attribute__((aligned(16))) float slabs[kMaxWaves][kSlab];
    const int lane = (int)threadIdx.x % kWave;
    const int wave = (int)threadIdx.x / kWave;
    const int64_t row = row_of(blockIdx.x, a.Q, wave);
    if (row >= a.rows) return;  // no workgroup barrier in this kernel
    const int cols = a.cols;
    const float* xr = a.x + row * (int64_t)cols;
    float* slab = slabs[wave];
    const float n = (float)cols;

    if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        float m = -INFINITY;
        for (int e = lane; e < cols; e += kWave) m = fmaxf(m, xr[e]);
        m = wave_allreduce<MaxOp>(m);
        const float s = ordered_fold<kExpShift>(xr, nullptr, cols, m, slab, lane);
        if constexpr (OP == kCrossEntropy) {
            if (lane == 0) {
                const int64_t lab = a.labels[row];
                const float sel = (lab >= 0 && lab < (int64_t)cols) ? xr[lab] : 0.0f;
                a.losses[row] = (logf(s) + m) - sel;
            }
        } else {
            float* yr = a.y + row * (int64_t)cols;
            for (int e = lane; e < cols; e += kWave) yr[e] = expf(xr[e] - m) / s;
        }
    } else if constexpr (OP == kRowSum) {
        const float sum = ordered_fold<kValue>(xr, nullptr, cols, 0.0f, slab, lane);
        if (lane == 0) a.sums[row] = sum;
    } else if constexpr (OP == kRowMinMax) {
        // exact in any order: the wave tree, as the max fold above
        float lo = INFINITY, hi = -INFINITY;
        for (int e = lane; e < cols; e += kWave) {
            lo = fmin2(lo, xr[e]);
            hi = fmax2(hi, xr[e]);
        }
        lo = wave_allreduce<MinOp>(lo);
        hi = wave_allreduce<MaxOp>(hi);
        if (lane == 0) {
            if (a.mins) a.mins[row] = lo;
            if (a.maxs) a.maxs[row] = hi;
        }
    } else if constexpr (OP == kRmsNorm) {
        const float ss = ordered_fold<kSquare>(xr, nullptr, cols, 0.0f, slab, lane);
        const float ms = ss / n;
        const float r = 1.0f / sqrtf(ms + a.eps);
        float* yr = a.y + row * (int64_t)cols;
        for (int e = lane; e < cols; e += kWave) {
            const float t = xr[e] * r;
            yr[e] = a.gamma ? t * a.gamma[e] : t;
        }
    } else {  // LayerNorm; fused residual LayerNorm folds over x + residual
        const float* rr = OP == kAddLayerNorm ? a.residual + row * (int64_t)cols : nullptr;
        const float mu = ordered_fold<kValue>(xr, rr, cols, 0.0f, slab, lane) / n;
        const float var = ordered_fold<kCentredSquare>(xr, rr, cols, mu, slab, lane) / n;
        const float r = 1.0f / sqrtf(var + a.eps);
        float* yr = a.y + row * (int64_t)cols;
        float* sr = (OP == kAddLayerNorm && a.sum_out) ? a.sum_out + row * (int64_t)cols : nullptr;
        for (int e = lane; e < cols; e += kWave) {
            // every read of element e precedes its writes (y or the sum may be
            // x or the residual itself)
            const float c = row_elem(xr, rr, e);
            float t = (c - mu) * r;
            if (a.gamma) t = t * a.gamma[e];
            if (a.beta) t = t + a.beta[e];
            yr[e] = t;
            if (sr) sr[e] = c;
        }
    }
}

hipError_t launch_ordered(int op, const KArgs& a, const lr_plan& p, hipStream_t s) {
    const dim3 grid((unsigned)p.blocks), block(p.threads_per_block);
    switch (op) {
        case kSoftmax: hipLaunchKernelGGL(k_ordered<kSoftmax>, grid, block, 0, s, a); break;
        case kRmsNorm: hipLaunchKernelGGL(k_ordered<kRmsNorm>, grid, block, 0, s, a); break;
        case kLayerNorm: hipLaunchKernelGGL(k_ordered<kLayerNorm>, grid, block, 0, s, a); break;
        case kCrossEntropy: hipLaunchKernelGGL(k_ordered<kCrossEntropy>, grid, block, 0, s, a); break;
        case kAddLayerNorm: hipLaunchKernelGGL(k_ordered<kAddLayerNorm>, grid, block, 0, s, a); break;
        case kRowSum: hipLaunchKernelGGL(k_ordered<kRowSum>, grid, block, 0, s, a); break;
        case kRowMinMax: hipLaunchKernelGGL(k_ordered<kRowMinMax>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lr
