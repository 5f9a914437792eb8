// SPLIT family (unordered policy): rows too few to fill the device are cut
// into G segments of whole 16-byte chunks, one workgroup per segment, so
// that every CU streams part of a row (64 rows on 256 CUs: G = 4).  The
// rows' statistics then combine across workgroups, through a workspace the
// caller provides, in a second kernel:
//
//   k_split_stats  each workgroup folds its segment (loaded into registers as
//                  in the CACHE family) into partial statistics, written to
//                  the workspace: softmax / cross-entropy (max m_g and
//                  sum_g exp(x - m_g)), RMSNorm (sum of squares), LayerNorm
//                  (segment mean and M2, the sum of squared deviations from
//                  it, two passes over the registers), row sum, row minimum
//                  and maximum;
//   k_split_apply  softmax and the norms: each workgroup merges its row's G
//                  partials, re-reads its segment (block b of both kernels
//                  runs on the same XCD, whose L2 still holds it) and writes
//                  the normalised segment;
//   k_split_merge  per-row outputs (loss, sum, minimum and maximum): one
//                  wave per row merges the partials and writes the result.
//
// Merges (lane g of a wave holds partial g, the wave tree combines them, so
// every wave of a row gets the same bits):
//   max / sum of exp (the merge of Milakov and Gimelshein, "Online
//   normalizer calculation for softmax", 2018): M = max_g m_g,
//   s = sum_g s_g exp(m_g - M);
//   LayerNorm (section 5.1 statistics, merged as Chan, Golub and LeVeque's
//   pairwise update): mean = sum_g n_g mean_g / cols,
//   M2 = sum_g (M2_g + n_g (mean_g - mean)^2), var = M2 / cols.
#pragma once

#include "lr_kernels.hpp"

namespace lr {

struct SplitCtx {
    int64_t row;
    int g;   // segment of the row
    int h;   // 16-byte phase of the row
    int nv;  // chunks of the row's grid
    SegmentBounds sb;
};

template <bool AL>
__device__ __forceinline__ SplitCtx split_ctx(const KArgs& a) {
    SplitCtx c;
    const int64_t b = blockIdx.x;
    c.row = b / a.splits;
    c.g = (int)(b - c.row * a.splits);
    const float* xr = a.x + c.row * (int64_t)a.cols;
    c.h = AL ? 0 : phase_of(reinterpret_cast<uintptr_t>(xr));
    c.nv = AL ? a.cols / kVec : chunks_of(c.h, a.cols);
    c.sb = segment_bounds(c.nv, a.splits, c.g);
    return c;
}

// Row elements inside chunks [k0, k1) of a grid at phase h.
__device__ __forceinline__ int segment_elems(SegmentBounds sb, int h, int cols) {
    const int lo = min(max(kVec * sb.k0 - h, 0), cols);
    const int hi = min(max(kVec * sb.k1 - h, 0), cols);
    return hi - lo;
}

// The segment's chunks in registers (x, plus the residual for the fused
// residual LayerNorm); slots outside the segment or the row take the op's
// identity.  The buffer resources cover the segment alone, so a stripe slot
// past its end reads zeros without touching memory.
template <int OP, int NCH, bool AL, int AUX>
__device__ __forceinline__ void load_segment(const KArgs& a, const SplitCtx& c, int w, int W, float4 (&v)[NCH]) {
    constexpr float ID = op_identity<OP>();
    const int cols = a.cols;
    const int64_t roff = c.row * (int64_t)cols;
    const int seg_bytes = (c.sb.k1 - c.sb.k0) * 16;
    const BufRes rx = make_res(a.x + roff - c.h + kVec * c.sb.k0, seg_bytes);
    constexpr bool RES = OP == kAddLayerNorm;
    // misaligned rows read the residual one float at a time at row indexes
    const BufRes rr = make_res(RES ? a.residual + roff + (AL ? kVec * c.sb.k0 : 0) : nullptr,
                               RES ? (AL ? seg_bytes : cols * 4) : 0);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int kk = w + W * i;  // chunk within the segment
        const int k = c.sb.k0 + kk;
        float4 raw = res_ld4<AUX>(rx, kk * 16);
        if constexpr (RES) {
            const float4 q = AL ? res_ld4<AUX>(rr, kk * 16) : elem_chunk(rr, k, c.h, cols);
            raw = make_float4(raw.x + q.x, raw.y + q.y, raw.z + q.z, raw.w + q.w);
        }
        if constexpr (AL && ID == 0.0f) {
            v[i] = raw;  // past the segment: zeros, the add identity
        } else {
            v[i] = k < c.sb.k1 ? raw : splat4(ID);
            if (!AL) mask_chunk(v[i], k, c.h, cols, ID);
        }
    }
}

template <int OP, int NCH, bool AL>
__global__ void __launch_bounds__(1024) k_split_stats(LR_ENTRY_PARAMS) {
    const KArgs a = LR_ENTRY_KARGS;
    __shared__ float red[2][kMaxWaves];
    constexpr float ID = op_identity<OP>();
    const int S = a.S;
    const int W = kWave * S;
    const Team t = team_of_wave(wave_id(), (int)threadIdx.x & (kWave - 1), S, a.team_magic);
    const SplitCtx c = split_ctx<AL>(a);
    float4 v[NCH];
    // kept in L2 for the second kernel's re-read
    load_segment<OP, NCH, AL, kAuxDefault>(a, c, t.w, W, v);
    float p0 = 0.0f, p1 = 0.0f;
    if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        float m = ID;
#pragma unroll
        for (int i = 0; i < NCH; ++i) m = fmax2(fmax2(m, fmax2(v[i].x, v[i].y)), fmax2(v[i].z, v[i].w));
        m = team_reduce<MaxOp>(m, red[0], S, t);
        float s = 0.0f;
        if (m != -INFINITY) {  // an empty segment keeps (-inf, 0)
#pragma unroll
            for (int i = 0; i < NCH; ++i)
                s += (fast_exp(v[i].x - m) + fast_exp(v[i].y - m)) + (fast_exp(v[i].z - m) + fast_exp(v[i].w - m));
        }
        p0 = m;
        p1 = team_reduce<AddOp>(s, red[1], S, t);
    } else if constexpr (OP == kRmsNorm) {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            ss += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
        p0 = team_reduce<AddOp>(ss, red[0], S, t);
    } else if constexpr (OP == kRowSum) {
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
        p0 = team_reduce<AddOp>(sum, red[0], S, t);
    } else if constexpr (OP == kRowMinMax) {
        float lo = ID, hi = ID;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            lo = fminnum(fminnum(lo, fminnum(v[i].x, v[i].y)), fminnum(v[i].z, v[i].w));
            hi = fmaxnum(fmaxnum(hi, fmaxnum(v[i].x, v[i].y)), fmaxnum(v[i].z, v[i].w));
        }
        lo = __builtin_isnan(lo) ? INFINITY : lo;
        hi = __builtin_isnan(hi) ? -INFINITY : hi;
        p0 = team_reduce<MinOp>(lo, red[0], S, t);
        p1 = team_reduce<MaxOp>(hi, red[1], S, t);
    } else {  // LayerNorm, fused residual LayerNorm: segment mean and M2
        const int n = segment_elems(c.sb, c.h, a.cols);
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
        sum = team_reduce<AddOp>(sum, red[0], S, t);
        const float mg = n > 0 ? sum / (float)n : 0.0f;
        float q = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int k = c.sb.k0 + t.w + W * i;
            float4 d = make_float4(v[i].x - mg, v[i].y - mg, v[i].z - mg, v[i].w - mg);
            if (k >= c.sb.k1) d = splat4(0.0f);
            if (!AL) mask_chunk(d, k, c.h, a.cols, 0.0f);
            q += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
        }
        p0 = mg;
        p1 = team_reduce<AddOp>(q, red[1], S, t);
    }
    if (threadIdx.x == 0) {
        float* o = a.ws + 2 * (int64_t)blockIdx.x;
        o[0] = p0;
        o[1] = p1;
    }
}

// Partial g of `row` in lane g (lanes >= G read partial 0 and ignore it).
struct Partial {
    float p0, p1;
    bool mine;
};

__device__ __forceinline__ Partial fetch_partial(const KArgs& a, int64_t row, int lane) {
    Partial q;
    q.mine = lane < a.splits;
    const float* pr = a.ws + 2 * (row * a.splits + (q.mine ? lane : 0));
    q.p0 = pr[0];
    q.p1 = pr[1];
    return q;
}

// The row's statistics from its partials, the same in every lane.
struct RowStats {
    float a, b;  // softmax/CE: (max, sum of exp); RMSNorm, row sum: (sum, -);
                 // LayerNorm: (mean, M2); row min/max: (min, max)
};

template <int OP>
__device__ __forceinline__ RowStats merge_partials(const KArgs& a, Partial q, int lane, int nv, int h) {
    RowStats r;
    if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        const float m = q.mine ? q.p0 : -INFINITY;
        const float M = wave_allreduce<MaxOp>(m);
        const float s = (q.mine && m != -INFINITY) ? q.p1 * fast_exp(m - M) : 0.0f;
        r.a = M;
        r.b = wave_allreduce<AddOp>(s);
    } else if constexpr (OP == kRmsNorm || OP == kRowSum) {
        r.a = wave_allreduce<AddOp>(q.mine ? q.p0 : 0.0f);
        r.b = 0.0f;
    } else if constexpr (OP == kRowMinMax) {
        r.a = wave_allreduce<MinOp>(q.mine ? q.p0 : INFINITY);
        r.b = wave_allreduce<MaxOp>(q.mine ? q.p1 : -INFINITY);
    } else {  // LayerNorm
        const float ng = q.mine ? (float)segment_elems(segment_bounds(nv, a.splits, lane), h, a.cols) : 0.0f;
        const float mg = q.mine ? q.p0 : 0.0f;
        const float mean = wave_allreduce<AddOp>(ng * mg) * a.inv_cols;
        const float dm = mg - mean;
        r.a = mean;
        r.b = wave_allreduce<AddOp>(q.mine ? q.p1 + ng * dm * dm : 0.0f);
    }
    return r;
}

template <int OP, int NCH, bool AL, int PM>
__global__ void __launch_bounds__(1024) k_split_apply(LR_ENTRY_PARAMS) {
    const KArgs a = LR_ENTRY_KARGS;
    constexpr int NP = num_params<OP>();
    const int S = a.S;
    const int W = kWave * S;
    const Team t = team_of_wave(wave_id(), (int)threadIdx.x & (kWave - 1), S, a.team_magic);
    const SplitCtx c = split_ctx<AL>(a);
    const int cols = a.cols;
    const Partial q = fetch_partial(a, c.row, t.lane);  // issued before the segment's loads
    float4 v[NCH];
    load_segment<OP, NCH, AL, LR_NT_LOADS ? kAuxNt : kAuxDefault>(a, c, t.w, W, v);
    // the parameters do not depend on the statistics: their loads are in
    // flight while the partials merge
    const ParamRes rg = param_res<AL>(a.gamma, cols, NP >= 1 && a.gamma);
    const ParamRes rb = param_res<AL>(a.beta, cols, NP == 2 && a.beta);
    float4 gv[NP >= 1 ? NCH : 1], bv[NP == 2 ? NCH : 1];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int k = c.sb.k0 + t.w + W * i;
        if constexpr (!AL && NCH >= 2) {
            // does this wave (chunks k0 .. k0 + 63) hold the row's first or last chunk?
            const int k0 = c.sb.k0 + t.s * kWave + W * i;
            const bool edge = k0 == 0 || (k0 < c.nv && c.nv <= k0 + kWave);
            if constexpr (NP >= 1) gv[i] = param_load_wide<PM>(rg, a.gamma != nullptr, k, c.h, 1.0f, edge);
            if constexpr (NP == 2) bv[i] = param_load_wide<PM>(rb, a.beta != nullptr, k, c.h, 0.0f, edge);
        } else {
            if constexpr (NP >= 1) gv[i] = param_load<AL, PM>(rg, a.gamma != nullptr, k, c.h, cols, 1.0f);
            if constexpr (NP == 2) bv[i] = param_load<AL, PM>(rb, a.beta != nullptr, k, c.h, cols, 0.0f);
        }
    }
    const RowStats st = merge_partials<OP>(a, q, t.lane, c.nv, c.h);
    float* yr = a.y + c.row * (int64_t)cols;
    float r = 0.0f;
    if constexpr (OP == kSoftmax) r = fast_rcp(st.b);
    if constexpr (OP == kRmsNorm) r = fast_rsqrt(st.a * a.inv_cols + a.eps);
    if constexpr (is_layernorm(OP)) r = fast_rsqrt(st.b * a.inv_cols + a.eps);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int k = c.sb.k0 + t.w + W * i;
        if (k < c.sb.k1) {
            float4 o;
            if constexpr (OP == kSoftmax) {
                o = make_float4(fast_exp(v[i].x - st.a) * r, fast_exp(v[i].y - st.a) * r,
                                fast_exp(v[i].z - st.a) * r, fast_exp(v[i].w - st.a) * r);
            } else if constexpr (OP == kRmsNorm) {
                const float4 g = gv[i];
                o = make_float4(v[i].x * r * g.x, v[i].y * r * g.y, v[i].z * r * g.z, v[i].w * r * g.w);
            } else {
                const float mu = st.a;
                const float4 g = gv[i];
                const float4 b = bv[i];
                o = make_float4((v[i].x - mu) * r * g.x + b.x, (v[i].y - mu) * r * g.y + b.y,
                                (v[i].z - mu) * r * g.z + b.z, (v[i].w - mu) * r * g.w + b.w);
                // the combined input; the segment was read above, so an
                // output that is x or the residual itself is safe
                if (OP == kAddLayerNorm && a.sum_out != nullptr)
                    store_chunk<AL>(a.sum_out + c.row * (int64_t)cols, a.s_same_phase, k, c.h, cols, v[i]);
            }
            store_chunk<AL>(yr, a.y_same_phase, k, c.h, cols, o);
        }
    }
}

// Per-row outputs: one wave per row merges the row's partials.
constexpr int kMergeWaves = 4;

template <int OP>
__global__ void __launch_bounds__(kMergeWaves * kWave) k_split_merge(LR_ENTRY_PARAMS) {
    const KArgs a = LR_ENTRY_KARGS;
    const int lane = (int)threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kMergeWaves + wave_id();
    if (row >= a.rows) return;  // whole waves leave; this kernel has no barrier
    const float* xr = a.x + row * (int64_t)a.cols;
    const Partial q = fetch_partial(a, row, lane);
    const RowStats st = merge_partials<OP>(a, q, lane, 0, 0);
    if (lane == 0) {
        if constexpr (OP == kCrossEntropy) {
            a.losses[row] = fast_log(st.b) + (st.a - gather_label(a, xr, row));
        } else if constexpr (OP == kRowSum) {
            a.sums[row] = st.a;
        } else {
            if (a.mins) a.mins[row] = st.a;
            if (a.maxs) a.maxs[row] = st.b;
        }
    }
}

// ---------------------------------------------------------------------------
// Launch: the statistics kernel, then (same stream) the apply or merge kernel.
// ---------------------------------------------------------------------------
template <int OP, int NCH, bool AL, int PM>
hipError_t launch_split_inst(const KArgs& a, const lr_plan& p, hipStream_t s) {
    const dim3 grid((unsigned)p.blocks), block(p.threads_per_block);
    hipLaunchKernelGGL((k_split_stats<OP, NCH, AL>), grid, block, 0, s, LR_ENTRY_ARGS(a));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (OP == kCrossEntropy || OP == kRowSum || OP == kRowMinMax) {
        const unsigned mb = (unsigned)((a.rows + kMergeWaves - 1) / kMergeWaves);
        hipLaunchKernelGGL((k_split_merge<OP>), dim3(mb), dim3(kMergeWaves * kWave), 0, s, LR_ENTRY_ARGS(a));
    } else {
        hipLaunchKernelGGL((k_split_apply<OP, NCH, AL, PM>), grid, block, 0, s, LR_ENTRY_ARGS(a));
    }
    return hipGetLastError();
}

template <int OP, bool AL, int PM>
hipError_t launch_split_nch(const KArgs& a, const lr_plan& p, hipStream_t s) {
    switch (p.chunks_per_lane) {
        case 1: return launch_split_inst<OP, 1, AL, PM>(a, p, s);
        case 2: return launch_split_inst<OP, 2, AL, PM>(a, p, s);
        case 3: return launch_split_inst<OP, 3, AL, PM>(a, p, s);
        case 4: return launch_split_inst<OP, 4, AL, PM>(a, p, s);
        case 6: return launch_split_inst<OP, 6, AL, PM>(a, p, s);
        case 8: return launch_split_inst<OP, 8, AL, PM>(a, p, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP, bool AL>
hipError_t launch_split_pm(const KArgs& a, const lr_plan& p, hipStream_t s) {
    if constexpr (num_params<OP>() == 0) {
        return launch_split_nch<OP, AL, kParNone>(a, p, s);
    } else {
        const bool all = a.gamma != nullptr && (OP == kRmsNorm || a.beta != nullptr);
        const bool none = a.gamma == nullptr && (OP == kRmsNorm || a.beta == nullptr);
        if (all) return launch_split_nch<OP, AL, kParAll>(a, p, s);
        if (none) return launch_split_nch<OP, AL, kParNone>(a, p, s);
        return launch_split_nch<OP, AL, kParRuntime>(a, p, s);
    }
}

// Unordered-policy dispatch of one operation: CACHE, STREAM or SPLIT.
template <int OP>
hipError_t launch_unordered(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    if (p.family == LR_FAMILY_SPLIT) {
        if (a.ws == nullptr || a.splits < 2 || a.splits > kMaxSplits) return hipErrorInvalidValue;
        return aligned ? launch_split_pm<OP, true>(a, p, s) : launch_split_pm<OP, false>(a, p, s);
    }
    return launch_op<OP>(a, p, aligned, s);
}

}  // namespace lr
