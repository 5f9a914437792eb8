// ORDERED family, one lane per row, for narrow rows (lanes_per_row = 1): the
// ordered reduction policies of "TIRx Metal reduction lowering", section 1,
// exactly as in k_ordered.hip -- fold_left and fold_right from +0.0f, the
// pairwise tree in index order over the contributions padded with the add
// identity -0.0f -- but with each lane owning one whole row.  A workgroup is
// one wavefront; lane l takes row 64 blockIdx.x + l and keeps it in registers
// (cols <= 4 N4 <= 64), so every ordered sum is that lane's own chain or tree
// over its registers and the elementwise passes read registers: 64 rows
// progress per wave, with no cross-lane arithmetic.  The rows come in and go
// out through an LDS tile with coalesced accesses (below).  Same operation
// sequence as k_ordered.hip (each multiply and add rounded on its own, IEEE
// division and square root, precise expf / logf), so the results are the
// same bits.
#pragma clang fp contract(off)

#include "lr_device.hpp"
#include "lr_entry.hpp"
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

// Wave-local ordering point for the LDS tile: this wave's LDS accesses
// before it complete before any after it.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Each wavefront owns 64 consecutive rows, which sit in memory as one block
// of 64 * cols floats.  The block is copied through an LDS tile with
// coalesced 32-bit accesses (flat element f = lane + 64 i goes to tile row
// f / cols, column f % cols); the tile's row pitch is odd, so that the 64
// lanes reading one element of their own rows hit distinct banks.  Any row
// alignment works, and the rows past the tensor's end are read as zeros and
// never written (the buffer resources cover the existing rows only).  The
// copies and the element loops have no branches: a load past its resource
// returns 0, a store past it is dropped, and an LDS write for a slot past
// the row goes to a spare slot (the copies) or the row's pad column.  So every global load of a copy,
// and of gamma / beta, is in flight before the first is used; loads left
// inside `i < cols` branches were each waited for before the next one went
// out, one memory round trip per element.
// FULL: cols == N, a compile-time constant, so that no element loop keeps
// a `j < cols` test.
template <int N>
constexpr int lane_tile_floats() {
    return kWave * (N + 1) + kWave;  // 64 rows of pitch <= N + 1, the spare slots
}

template <int OP, int POL, int N4, bool FULL>
__device__ __forceinline__ void lane_body(const KArgs& a, float* tile) {
    constexpr int N = 4 * N4;       // cols <= N
    constexpr int PMAX = N + 1;     // largest pitch (cols <= N, N even)
    constexpr int SPARE = kWave * PMAX;  // one spare slot per lane past the rows
    const int lane = (int)threadIdx.x;
    const int cols = FULL ? N : a.cols;
    // odd row pitch with at least one pad column (column `cols`)
    const int pitch = (cols + 1) | 1;
    const int64_t r0 = (int64_t)blockIdx.x * kWave;  // the wave's first row
    const int64_t left = a.rows - r0;
    const int nr = left < kWave ? (int)left : kWave;  // its rows that exist (>= 1)
    const int64_t off0 = r0 * (int64_t)cols;
    const int nflat = nr * cols;
    const float n = (float)cols;
    const int64_t row = r0 + lane;
    const bool active = lane < nr;

    // Tile slots of this lane's flat elements f = lane + 64 i, i = 0, 1, ...:
    // row f / cols, column f % cols, stepped 64 elements at a time (q rows and
    // rem columns further on, one more row when the column passes cols) with
    // full-rate adds only.  Past the wave's 64 rows (i >= cols) the slot is at
    // least SPARE and clamps into the spare slots, which nothing reads back.
    const int q = kWave / cols, rem = kWave - q * cols;
    const int step = q * pitch + rem, wrap = pitch - cols;
    struct Walk {
        unsigned c, idx;
    };
    auto walk0 = [&]() {
        const int r = lane / cols;
        return Walk{(unsigned)(lane - r * cols), (unsigned)(r * pitch + (lane - r * cols))};
    };
    auto next = [&](Walk& w) {
        const unsigned c = w.c + rem;
        const unsigned t = c - (unsigned)cols;    // wraps around (huge) when c < cols
        w.c = min(c, t);
        w.idx += (unsigned)step + (t < c ? (unsigned)wrap : 0u);
    };
    auto slot = [&](const Walk& w) { return (int)min(w.idx, (unsigned)(SPARE + lane)); };
    // gamma, beta (read only where present): entry j alike in every lane;
    // past cols, or when absent, the resources read 0
    constexpr int NP = OP == kRmsNorm ? 1 : (OP == kLayerNorm || OP == kAddLayerNorm ? 2 : 0);
    float g[NP >= 1 ? N : 1], b[NP == 2 ? N : 1];
    if constexpr (NP >= 1) {
        const BufRes rg = make_res(a.gamma, a.gamma ? cols * 4 : 0);
#pragma unroll
        for (int j = 0; j < N; ++j) g[j] = res_ld1(rg, j * 4);
    }
    if constexpr (NP == 2) {
        const BufRes rb = make_res(a.beta, a.beta ? cols * 4 : 0);
#pragma unroll
        for (int j = 0; j < N; ++j) b[j] = res_ld1(rb, j * 4);
    }
    // cross-entropy: the row's label, read with the parameters, ahead of the
    // rows (-1 for the lanes past the tensor's last row)
    int64_t lab = -1;
    if constexpr (OP == kCrossEntropy) {
        if (active) lab = a.labels[row];
    }
    // the rows (x + residual for the fused residual LayerNorm, in FP32)
    {
        const BufRes rs = make_res(a.x + off0, nflat * 4);
        float v[N];
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = res_ld1(rs, (lane + kWave * i) * 4);
        if constexpr (OP == kAddLayerNorm) {
            const BufRes ra = make_res(a.residual + off0, nflat * 4);
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = v[i] + res_ld1(ra, (lane + kWave * i) * 4);
        }
        Walk w = walk0();
#pragma unroll
        for (int i = 0; i < N; ++i) {
            tile[slot(w)] = v[i];
            next(w);
        }
    }
    // the tile to `dst`: every read first (slots past the rows read entry 0),
    // then the stores (those past the block are dropped)
    auto copy_out = [&](float* dst) {
        const BufRes rd = make_res(dst + off0, nflat * 4);
        float o[N];
        Walk w = walk0();
#pragma unroll
        for (int i = 0; i < N; ++i) {
            o[i] = tile[slot(w)];
            next(w);
        }
#pragma unroll
        for (int i = 0; i < N; ++i) res_st1(rd, (lane + kWave * i) * 4, o[i]);
    };
    wave_sync();
    if constexpr (OP == kAddLayerNorm) {
        if (a.sum_out != nullptr) copy_out(a.sum_out);
    }
    float x[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const float t = tile[lane * pitch + j];  // inside the tile for every j < N
        x[j] = j < cols ? t : 0.0f;
    }
    // cross-entropy: the labelled logit, from the lane's row in the tile (0
    // for a label outside [0, cols))
    float sel = 0.0f;
    if constexpr (OP == kCrossEntropy) {
        const bool in = lab >= 0 && lab < (int64_t)cols;
        const float t = tile[lane * pitch + (in ? (int)lab : 0)];
        sel = in ? t : 0.0f;
    }
    wave_sync();  // every lane has its row before any lane writes the tile

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
            if (active) {
                a.losses[row] = logf(s) + (m - sel);
            }
        } else {
            // e / s rounded once: div_rowsum unless some e of the wave's rows
            // lies in (0, 2^-96), then the division (a choice per wave)
            const float y = 1.0f / s;
            unsigned lo = ~0u;
#pragma unroll
            for (int j = 0; j < N; ++j) lo = min(lo, rowsum_guard(e[j]));
            if (__builtin_amdgcn_ballot_w64(lo < kRowsumTiny) == 0) {
#pragma unroll
                for (int j = 0; j < N; ++j) tile[lane * pitch + min(j, cols)] = div_rowsum(e[j], s, y);
            } else {
#pragma unroll
                for (int j = 0; j < N; ++j) tile[lane * pitch + min(j, cols)] = e[j] / s;
            }
            wave_sync();
            copy_out(a.y);
        }
    } else if constexpr (OP == kRowSum) {
        const float sum = lane_sum<POL>(x, cols);
        if (active) a.sums[row] = sum;
    } else if constexpr (OP == kRowMinMax) {
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            if (j < cols) {
                lo = fmin2(lo, x[j]);
                hi = fmax2(hi, x[j]);
            }
        }
        if (active) {
            if (a.mins) a.mins[row] = lo;
            if (a.maxs) a.maxs[row] = hi;
        }
    } else if constexpr (OP == kRmsNorm) {
        float q[N];
#pragma unroll
        for (int j = 0; j < N; ++j) q[j] = x[j] * x[j];
        const float ms = lane_sum<POL>(q, cols) / n;
        const float r = 1.0f / sqrtf(ms + a.eps);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const float t = x[j] * r;
            tile[lane * pitch + min(j, cols)] = a.gamma ? t * g[j] : t;
        }
        wave_sync();
        copy_out(a.y);
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
        for (int j = 0; j < N; ++j) {
            float t = (x[j] - mu) * r;
            if (a.gamma) t = t * g[j];
            if (a.beta) t = t + b[j];
            tile[lane * pitch + min(j, cols)] = t;
        }
        wave_sync();
        copy_out(a.y);
    }
}

template <int OP, int POL, int N4>
__global__ void __launch_bounds__(64) k_ordered_lane(LR_ENTRY_PARAMS) {
    const KArgs a = LR_ENTRY_KARGS;
    __shared__ float tile[lane_tile_floats<4 * N4>()];
    if (a.cols == 4 * N4) {
        lane_body<OP, POL, N4, true>(a, tile);
    } else {
        lane_body<OP, POL, N4, false>(a, tile);
    }
}

template <int OP, int POL>
hipError_t launch_lane_n4(const KArgs& a, const lr_plan& p, hipStream_t s) {
    const dim3 grid((unsigned)p.blocks), block(p.threads_per_block);
    switch (p.chunks_per_lane) {
        case 1: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 1>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case 2: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 2>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case 4: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 4>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case 8: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 8>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case 16: hipLaunchKernelGGL((k_ordered_lane<OP, POL, 16>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int POL>
hipError_t launch_lane_pol(int op, const KArgs& a, const lr_plan& p, hipStream_t s) {
    switch (op) {
        case kSoftmax: return launch_lane_n4<kSoftmax, POL>(a, p, s);
        case kRmsNorm: return launch_lane_n4<kRmsNorm, POL>(a, p, s);
        case kLayerNorm: return launch_lane_n4<kLayerNorm, POL>(a, p, s);
        case kCrossEntropy: return launch_lane_n4<kCrossEntropy, POL>(a, p, s);
        case kAddLayerNorm: return launch_lane_n4<kAddLayerNorm, POL>(a, p, s);
        case kRowSum: return launch_lane_n4<kRowSum, POL>(a, p, s);
        case kRowMinMax: return launch_lane_n4<kRowMinMax, POL>(a, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_ordered_lane(int op, int policy, const KArgs& a, const lr_plan& p, hipStream_t s) {
    switch (policy) {
        case kPolFoldLeft: return launch_lane_pol<kPolFoldLeft>(op, a, p, s);
        case kPolTree: return launch_lane_pol<kPolTree>(op, a, p, s);
        case kPolFoldRight: return launch_lane_pol<kPolFoldRight>(op, a, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lr
