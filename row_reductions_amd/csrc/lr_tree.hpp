// TREE family: the ordered_tree policy ("TIRx Metal reduction lowering",
// section 1) on the CACHE family's register layout, for rows whose start is
// 16-byte aligned (cols % 4 == 0 and an aligned x).
//
// ordered_tree is read as the pairwise tree in index order over a row's
// contributions padded with the add identity -0.0f to the next power of two;
// since x + -0 is x for every x, padding further (to whole slabs and whole
// waves, as below) changes no bit.  In the cache
// layout worker w = 64 s + l of a W = 64 S team holds chunk k = w + W c,
// elements 4k .. 4k+3, so the 64 lanes of wave s at stripe slot c hold the
// aligned 256-element slab j = S c + s.  The tree is computed in exactly
// that structure:
//   levels 1-2  inside a lane: (c0 + c1) + (c2 + c3);
//   levels 3-8  the wave64 all-reduce, whose steps add aligned adjacent lane
//               blocks (pairs, quads, octets, rows, row pairs): the slab sum;
//   above       slab sums go to LDS and one more wave tree (a pair per lane
//               first when there are more than 64 slabs) combines them;
//               slabs past the row are padding (-0, an exact identity).
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
        u = lane < nslab ? slots[lane] : -0.0f;
    } else {
        const float l = 2 * lane < nslab ? slots[2 * lane] : -0.0f;
        const float r = 2 * lane + 1 < nslab ? slots[2 * lane + 1] : -0.0f;
        u = l + r;
    }
    return wave_allreduce<AddOp>(u);
}

// The body of both TREE kernels.  LW = 64: a row team of S waves (k_tree).
// LW = 4, 8, 16 or 32 with one chunk per lane: sub-wave teams (k_tree_narrow),
// 64 / LW rows per wave; the row's 4 LW leaves (padding -0) are then the
// whole tree, two levels inside each lane and log2(LW) DPP levels across the
// team, with no LDS.  The wave's rows are read through one resource (rows
// are 16-byte aligned: lane row at byte xo).
template <int OP, int NCH, bool AL, int PM, int LW>
__device__ __forceinline__ void tree_body(const KArgs& a, float (&red)[2][kMaxWaves],
                                          float (&tsl)[2][kMaxWaves][kTreeMaxSlabs]) {
    constexpr bool NARROW = LW < kWave;
    static_assert(!NARROW || NCH == 1, "sub-wave tree teams hold one chunk per lane");
    constexpr bool RES = OP == kAddLayerNorm;
    const int S = NARROW ? 1 : a.S;
    const int W = NARROW ? LW : kWave * S;
    const int lane = (int)threadIdx.x & (kWave - 1);
    const Team t = NARROW ? team_of_group(wave_id(), lane, LW) : team_of_wave(wave_id(), lane, S, a.team_magic);
    const int64_t row = row_of(blockIdx.x, a.Q, t.q);
    const bool active = row < a.rows;
    const int cols = a.cols;
    const int64_t roff = (active ? row : 0) * (int64_t)cols;
    const float* xr = a.x + roff;
    const int nv = active ? cols / kVec : 0;  // the x row starts on a 16-byte boundary
    const int nslab = (nv + kWave - 1) / kWave;
    const float n = (float)cols;
    BufRes rx, rr;
    int xo = 0;  // byte offset of this lane's row in rx and rr
    if constexpr (!NARROW) {
        rx = make_res(xr, nv * 16);
        rr = make_res(RES ? a.residual + roff : nullptr, RES && active ? (AL ? nv * 16 : cols * 4) : 0);
    } else {
        const int64_t r0 = row_of(blockIdx.x, a.Q, wave_id() * (kWave / LW));  // the wave's first row
        const int64_t left = a.rows - r0;
        const int nr = left <= 0 ? 0 : (left < kWave / LW ? (int)left : kWave / LW);
        const int64_t off0 = (nr > 0 ? r0 : 0) * (int64_t)cols;
        rx = make_res(a.x + off0, nr * cols * 4);
        rr = make_res(RES ? a.residual + off0 : nullptr, RES ? nr * cols * 4 : 0);
        xo = active ? (int)((row - r0) * cols * 4) : 0;
    }
    const ParamRes rg = param_res<AL>(a.gamma, cols, num_params<OP>() >= 1 && a.gamma);
    const ParamRes rb = param_res<AL>(a.beta, cols, num_params<OP>() == 2 && a.beta);
    auto chunk = [&](int c) { return chunk_index(t.w, W, c); };

    // the row (x + residual for the fused residual LayerNorm); zeros past it
    float4 v[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int k = chunk(c);
        float4 raw = res_ld4<LR_NT_LOADS ? kAuxNt : kAuxDefault>(rx, xo + k * 16);
        if constexpr (RES) {
            const float4 q = AL ? res_ld4<LR_NT_LOADS ? kAuxNt : kAuxDefault>(rr, xo + k * 16)
                                : elem_chunk(rr, k, 0, cols, xo);
            raw = make_float4(raw.x + q.x, raw.y + q.y, raw.z + q.z, raw.w + q.w);
        }
        // past the row: zeros (a sub-wave team's resource holds the next row there)
        v[c] = (RES || NARROW) && k >= nv ? splat4(0.0f) : raw;
    }

    // one ordered-tree add reduction of the contributions f; chunks past the
    // row are padding, -0
    auto tree_sum = [&](const float4 (&f)[NCH], int round) {
        if constexpr (NARROW) {
            const float4 g = chunk(0) < nv ? f[0] : splat4(-0.0f);
            return group_allreduce<AddOp, LW>((g.x + g.y) + (g.z + g.w));
        } else {
            float* slots = tsl[round][t.q];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const float4 g = chunk(c) < nv ? f[c] : splat4(-0.0f);
                const float p = wave_allreduce<AddOp>((g.x + g.y) + (g.z + g.w));
                const int j = S * c + t.s;
                if (t.lane == 0 && j < nslab) slots[j] = p;
            }
            __syncthreads();
            return slab_tree(slots, nslab, t.lane);
        }
    };

    float* yr = a.y + roff;
    if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        float m = -INFINITY;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if (chunk(c) < nv) m = fmax2(fmax2(m, fmax2(v[c].x, v[c].y)), fmax2(v[c].z, v[c].w));
        }
        m = row_reduce<MaxOp, LW>(m, red[0], S, t);
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
            // e / s rounded once: div_rowsum unless some e of this wave lies
            // in (0, 2^-96), then the division (a choice per wave)
            unsigned lo = ~0u;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                lo = min(min(min(lo, rowsum_guard(v[c].x)), rowsum_guard(v[c].y)),
                         min(rowsum_guard(v[c].z), rowsum_guard(v[c].w)));
            if (__builtin_amdgcn_ballot_w64(lo < kRowsumTiny) == 0) {
                const float y = 1.0f / s;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const int k = chunk(c);
                    if (k < nv) {
                        const float4 o = make_float4(div_rowsum(v[c].x, s, y), div_rowsum(v[c].y, s, y),
                                                     div_rowsum(v[c].z, s, y), div_rowsum(v[c].w, s, y));
                        store_chunk<AL>(yr, a.y_same_phase, k, 0, cols, o);
                    }
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
        lo = row_reduce<MinOp, LW>(lo, red[0], S, t);
        hi = row_reduce<MaxOp, LW>(hi, red[1], S, t);
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
__global__ void __launch_bounds__(cache_max_threads(NCH))
k_tree(LR_ENTRY_PARAMS) {
    __shared__ float red[2][kMaxWaves];
    __shared__ float tsl[2][kMaxWaves][kTreeMaxSlabs];
    tree_body<OP, NCH, AL, PM, kWave>(LR_ENTRY_KARGS, red, tsl);
}

// Sub-wave teams: LW lanes per row, one chunk per lane, 64 / LW rows per wave.
template <int OP, bool AL, int PM, int LW>
__global__ void __launch_bounds__(1024)
k_tree_narrow(LR_ENTRY_PARAMS) {
    __shared__ float red[2][kMaxWaves];               // untouched: no cross-wave exchange
    __shared__ float tsl[2][kMaxWaves][kTreeMaxSlabs];  // untouched
    tree_body<OP, 1, AL, PM, LW>(LR_ENTRY_KARGS, red, tsl);
}

template <int OP, int NCH, bool AL, int PM>
hipError_t launch_tree_inst(const KArgs& a, const lr_plan& p, hipStream_t s) {
    hipLaunchKernelGGL((k_tree<OP, NCH, AL, PM>), dim3((unsigned)p.blocks), dim3(p.threads_per_block), 0, s,
                       LR_ENTRY_ARGS(a));
    return hipGetLastError();
}

template <int OP, bool AL, int PM, int LW>
hipError_t launch_tree_narrow(const KArgs& a, const lr_plan& p, hipStream_t s) {
    if (p.chunks_per_lane != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_tree_narrow<OP, AL, PM, LW>), dim3((unsigned)p.blocks), dim3(p.threads_per_block), 0, s,
                       LR_ENTRY_ARGS(a));
    return hipGetLastError();
}

template <int OP, bool AL, int PM>
hipError_t launch_tree_nch(const KArgs& a, const lr_plan& p, hipStream_t s) {
    switch (p.lanes_per_row) {
        case 4: return launch_tree_narrow<OP, AL, PM, 4>(a, p, s);
        case 8: return launch_tree_narrow<OP, AL, PM, 8>(a, p, s);
        case 16: return launch_tree_narrow<OP, AL, PM, 16>(a, p, s);
        case 32: return launch_tree_narrow<OP, AL, PM, 32>(a, p, s);
        default: break;  // whole-wave teams
    }
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
