// TREE family: the ordered_tree policy ("TIRx Metal reduction lowering",
// section 1) on the CACHE family's register layout, for rows whose start is
// 16-byte aligned (cols % 4 == 0 and an aligned x).
//
// ordered_tree is read as the pairwise tree in index order over a row's
// contributions padded with +0.0f to the next power of two.  In the cache
// layout worker w = 64 s + l of a W = 64 S team holds chunk k = w + W c,
// elements 4k .. 4k+3, so the 64 lanes of wave s at stripe slot c hold the
// aligned 256-element slab j = S c + s.  The tree is computed in exactly
// that structure:
//   levels 1-2  inside a lane: (c0 + c1) + (c2 + c3);
//   levels 3-8  the wave64 all-reduce, whose steps add aligned adjacent lane
//               blocks (pairs, quads, octets, rows, row pairs): the slab sum;
//   above       slab sums go to LDS and one more wave tree (a pair per lane
//               first when there are more than 64 slabs) combines them;
//               slabs past the row are the padding's exact +0.
// Every wave of the team computes the same bits, so the result does not
// depend on S or the chunk count.  Max and min folds are exact and use the
// usual team reduction.  The translation units that instantiate this file
// are built without contraction and with IEEE division and square root;
// exp and log are the precise library functions, as for the other ordered
// policies.
#pragma once

#include "lr_kernels.hpp"

namespace lr {

constexpr int kTreeMaxSlabs = 128;  // 32768 floats per row

// Tree over the row's slab sums `slots[0 .. nslab)`; identical in all lanes.
__device__ __forceinline__ float slab_tree(const float* slots, int nslab, int lane) {
    float u;
    if (nslab <= kWave) {
        u = lane < nslab ? slots[lane] : 0.0f;
    } else {
        const float l = 2 * lane < nslab ? slots[2 * lane] : 0.0f;
        const float r = 2 * lane + 1 < nslab ? slots[2 * lane + 1] : 0.0f;
        u = l + r;
    }
    return wave_allreduce<AddOp>(u);
}

template <int OP, int NCH, bool AL, int PM>
__global__ void __launch_bounds__(cache_max_threads(NCH))
k_tree(const KArgs a) {
    __shared__ float red[2][kMaxWaves];
    __shared__ float tsl[2][kMaxWaves][kTreeMaxSlabs];
    constexpr bool RES = OP == kAddLayerNorm;
    const int S = a.S;
    const int W = kWave * S;
    const Team t = team_of_wave(wave_id(), (int)threadIdx.x & (kWave - 1), S, a.team_magic);
    const int64_t row = row_of(blockIdx.x, a.Q, t.q);
    const bool active = row < a.rows;
    const int cols = a.cols;
    const int64_t roff = (active ? row : 0) * (int64_t)cols;
    const float* xr = a.x + roff;
    const int nv = active ? cols / kVec : 0;  // the x row starts on a 16-byte boundary
    const int nslab = (nv + kWave - 1) / kWave;
    const float n = (float)cols;
    const BufRes rx = make_res(xr, nv * 16);
    const BufRes rr = make_res(RES ? a.residual + roff : nullptr, RES && active ? (AL ? nv * 16 : cols * 4) : 0);
    const BufRes rg = make_res(a.gamma, num_params<OP>() >= 1 && a.gamma ? cols * 4 : 0);
    const BufRes rb = make_res(a.beta, num_params<OP>() == 2 && a.beta ? cols * 4 : 0);
    auto chunk = [&](int c) { return chunk_index(t.w, W, c); };

    // the row (x + residual for the fused residual LayerNorm); zeros past it
    float4 v[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int k = chunk(c);
        float4 raw = res_ld4<LR_NT_LOADS ? kAuxNt : kAuxDefault>(rx, k * 16);
        if constexpr (RES) {
            const float4 q = AL ? res_ld4<LR_NT_LOADS ? kAuxNt : kAuxDefault>(rr, k * 16) : elem_chunk(rr, k, 0, cols);
            raw = make_float4(raw.x + q.x, raw.y + q.y, raw.z + q.z, raw.w + q.w);
            if (k >= nv) raw = splat4(0.0f);
        }
        v[c] = raw;
    }

    // one ordered-tree add reduction of the contributions f (zero past the row)
    auto tree_sum = [&](const float4 (&f)[NCH], int round) {
        float* slots = tsl[round][t.q];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const float p = wave_allreduce<AddOp>((f[c].x + f[c].y) + (f[c].z + f[c].w));
            const int j = S * c + t.s;
            if (t.lane == 0 && j < nslab) slots[j] = p;
        }
        __syncthreads();
        return slab_tree(slots, nslab, t.lane);
    };

    float* yr = a.y + roff;
    if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        float m = -INFINITY;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (chunk(c) < nv) m = fmax2(fmax2(m, fmax2(v[c].x, v[c].y)), fmax2(v[c].z, v[c].w));
        }
        m = team_reduce<MaxOp>(m, red[0], S, t);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            v[c] = chunk(c) < nv ? make_float4(expf(v[c].x - m), expf(v[c].y - m), expf(v[c].z - m), expf(v[c].w - m))
                                 : splat4(0.0f);
        }
        const float s = tree_sum(v, 0);
        if constexpr (OP == kCrossEntropy) {
            if (active && t.w == 0) {
                const float sel = gather_label(a, xr, row);
                a.losses[row] = logf(s) + (m - sel);
            }
        } else {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int k = chunk(c);
                if (k < nv) {
                    const float4 o = make_float4(v[c].x / s, v[c].y / s, v[c].z / s, v[c].w / s);
                    store_chunk<AL>(yr, a.y_same_phase, k, 0, cols, o);
                }
            }
        }
    } else if constexpr (OP == kRowSum) {
        const float sum = tree_sum(v, 0);
        if (active && t.w == 0) a.sums[row] = sum;
    } else if constexpr (OP == kRowMinMax) {
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (chunk(c) < nv) {
                lo = fmin2(fmin2(lo, fmin2(v[c].x, v[c].y)), fmin2(v[c].z, v[c].w));
                hi = fmax2(fmax2(hi, fmax2(v[c].x, v[c].y)), fmax2(v[c].z, v[c].w));
            }
        }
        lo = team_reduce<MinOp>(lo, red[0], S, t);
        hi = team_reduce<MaxOp>(hi, red[1], S, t);
        if (active && t.w == 0) {
            if (a.mins) a.mins[row] = lo;
            if (a.maxs) a.maxs[row] = hi;
        }
    } else if constexpr (OP == kRmsNorm) {
        float4 f[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) f[c] = make_float4(v[c].x * v[c].x, v[c].y * v[c].y, v[c].z * v[c].z, v[c].w * v[c].w);
        const float ms = tree_sum(f, 0) / n;
        const float r = 1.0f / sqrtf(ms + a.eps);
        const bool has_g = a.gamma != nullptr;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int k = chunk(c);
            if (k < nv) {
                float4 o = make_float4(v[c].x * r, v[c].y * r, v[c].z * r, v[c].w * r);
                if (PM != kParNone && has_g) {
                    const float4 g = param_load<AL, PM>(rg, true, k, 0, cols, 1.0f);
                    o = make_float4(o.x * g.x, o.y * g.y, o.z * g.z, o.w * g.w);
                }
                store_chunk<AL>(yr, a.y_same_phase, k, 0, cols, o);
            }
        }
    } else {  // LayerNorm, fused residual LayerNorm
        if constexpr (RES) {
            if (a.sum_out != nullptr) {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const int k = chunk(c);
                    if (k < nv) store_chunk<AL>(a.sum_out + roff, a.s_same_phase, k, 0, cols, v[c]);
                }
            }
        }
        const float mu = tree_sum(v, 0) / n;
        float4 f[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            v[c] = chunk(c) < nv ? make_float4(v[c].x - mu, v[c].y - mu, v[c].z - mu, v[c].w - mu) : splat4(0.0f);
            f[c] = make_float4(v[c].x * v[c].x, v[c].y * v[c].y, v[c].z * v[c].z, v[c].w * v[c].w);
        }
        const float var = tree_sum(f, 1) / n;
        const float r = 1.0f / sqrtf(var + a.eps);
        const bool has_g = a.gamma != nullptr, has_b = a.beta != nullptr;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int k = chunk(c);
            if (k < nv) {
                float4 o = make_float4(v[c].x * r, v[c].y * r, v[c].z * r, v[c].w * r);
                if (PM != kParNone && has_g) {
                    const float4 g = param_load<AL, PM>(rg, true, k, 0, cols, 1.0f);
                    o = make_float4(o.x * g.x, o.y * g.y, o.z * g.z, o.w * g.w);
                }
                if (PM != kParNone && has_b) {
                    const float4 b = param_load<AL, PM>(rb, true, k, 0, cols, 0.0f);
                    o = make_float4(o.x + b.x, o.y + b.y, o.z + b.z, o.w + b.w);
                }
                store_chunk<AL>(yr, a.y_same_phase, k, 0, cols, o);
            }
        }
    }
}

template <int OP, int NCH, bool AL, int PM>
hipError_t launch_tree_inst(const KArgs& a, const lr_plan& p, hipStream_t s) {
    hipLaunchKernelGGL((k_tree<OP, NCH, AL, PM>), dim3((unsigned)p.blocks), dim3(p.threads_per_block), 0, s, a);
    return hipGetLastError();
}

template <int OP, bool AL, int PM>
hipError_t launch_tree_nch(const KArgs& a, const lr_plan& p, hipStream_t s) {
    switch (p.chunks_per_lane) {
        case 1: return launch_tree_inst<OP, 1, AL, PM>(a, p, s);
        case 2: return launch_tree_inst<OP, 2, AL, PM>(a, p, s);
        case 3: return launch_tree_inst<OP, 3, AL, PM>(a, p, s);
        case 4: return launch_tree_inst<OP, 4, AL, PM>(a, p, s);
        case 6: return launch_tree_inst<OP, 6, AL, PM>(a, p, s);
        case 8: return launch_tree_inst<OP, 8, AL, PM>(a, p, s);
        case 12: return launch_tree_inst<OP, 12, AL, PM>(a, p, s);
        case 16: return launch_tree_inst<OP, 16, AL, PM>(a, p, s);
        case 24: return launch_tree_inst<OP, 24, AL, PM>(a, p, s);
        case 32: return launch_tree_inst<OP, 32, AL, PM>(a, p, s);
        default: return hipErrorInvalidValue;
    }
}

// Launch of the tree family for one op.  `aligned`: every pointer is 16-byte
// aligned (else outputs, parameters and the residual take per-float paths;
// the x row itself is always aligned here).
template <int OP>
hipError_t launch_tree_op(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    if constexpr (num_params<OP>() == 0) {
        return aligned ? launch_tree_nch<OP, true, kParNone>(a, p, s) : launch_tree_nch<OP, false, kParNone>(a, p, s);
    } else {
        const bool any = a.gamma != nullptr || (num_params<OP>() == 2 && a.beta != nullptr);
        if (!any)
            return aligned ? launch_tree_nch<OP, true, kParNone>(a, p, s) : launch_tree_nch<OP, false, kParNone>(a, p, s);
        return aligned ? launch_tree_nch<OP, true, kParRuntime>(a, p, s)
                       : launch_tree_nch<OP, false, kParRuntime>(a, p, s);
    }
}

}  // namespace lr
