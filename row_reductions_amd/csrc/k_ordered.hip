// ORDERED family: the ordered reduction policies of "TIRx Metal reduction
// lowering", section 1, for any row:
//   fold_left (LR_ORDERED_FOLD): every add fold of a row is one FP32 chain
//       taken left to right, j = 0 .. cols-1, from the identity +0.0f;
//   fold_right: the same chain taken from the right end, acc = c_j + acc,
//       j = cols-1 .. 0;
//   ordered_tree: the pairwise tree in index order over the contributions
//       padded with the add identity -0.0f to the next power of two (x + -0
//       is x for every x, so padding further, as the 256-leaf slabs do,
//       changes no bit).
// Each multiply and add is rounded on its own; division and square root are
// IEEE (built with -ffp-contract=off and correctly rounded divide/sqrt); max
// and min folds are exact and use the wave tree.  The result does not depend
// on the plan, and RMSNorm / LayerNorm / row-sum results are the unique FP32
// values of the stated operation sequence.
//
// One wavefront owns a row.  Per 256-element slab, each lane loads four
// elements (coalesced 32-bit loads at 64*i + lane), computes their
// contributions elementwise in parallel and writes them to the wave's LDS
// slab.  Folds: every lane folds the slab in order from LDS (broadcast
// reads), one dependent add per element.  Tree: lane l reads slab entries
// 4l .. 4l+3 and adds them pairwise, and the wave64 all-reduce -- whose steps
// combine aligned adjacent lane blocks -- completes the slab's 256-leaf tree;
// slab sums are then merged like a binary counter on a small LDS stack (two
// adjacent complete subtrees of equal size merge at once), and the partial
// subtrees left at the end are added from the smallest up, which is the tree
// over the padded row.
#pragma clang fp contract(off)

#include "lr_device.hpp"
#include "lr_entry.hpp"
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

// Elementwise passes (the row's maximum, minimum, and the output) walk the
// row in trips of kPass elements per lane, element base + 64*u + lane at slot
// u, through buffer resources: every load of a trip is issued before the
// first is used, and a load past the row returns 0 (a store past it is
// dropped).  An element loop that used each load at once would wait for one
// memory round trip per element.
constexpr int kPass = 16;

__device__ __forceinline__ int pass_elem(int base, int u, int lane) { return base + kWave * u + lane; }

// The row's maximum, exact in any order (the wave tree combines the lanes).
__device__ __forceinline__ float row_max(BufRes rx, int cols, int lane) {
    float m = -INFINITY;
    for (int base = 0; base < cols; base += kWave * kPass) {
        float v[kPass];
#pragma unroll
        for (int u = 0; u < kPass; ++u) v[u] = res_ld1(rx, pass_elem(base, u, lane) * 4);
#pragma unroll
        for (int u = 0; u < kPass; ++u)
            if (pass_elem(base, u, lane) < cols) m = fmaxf(m, v[u]);
    }
    return wave_allreduce<MaxOp>(m);
}

// Folds one full 256-entry slab into acc, left to right (FOLD_RIGHT: right to
// left), one dependent add per entry.  The slab is read in 16-float groups
// through a three-group rolling register buffer: group g+2's four reads are
// issued before group g's sixteen adds, and scheduling barriers on both sides
// of the adds keep them there.  Without the barriers the scheduler moved each
// group's reads down next to their adds (reusing one register quad), and the
// chain waited out the LDS latency once per group.  A wave issues one
// instruction per slot, so the adds, reads and waits share the issue rate:
// on MI355X a chain fed this way takes 6.7 cycles per add, against 8.3 with
// the reads next to their adds and 4.3 for adds alone.
// Ordering point of the fold: no LDS read crosses it (the empty asm
// statement clobbers memory) and neither does the chain (the statement takes
// and returns `acc`, so the adds before it come first and those after it
// consume its result); the scheduling barrier keeps the machine scheduler
// from moving anything else across.  It emits no instruction.
__device__ __forceinline__ void fold_fence(float& acc) {
    asm volatile("" : "+v"(acc)::"memory");
    __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt operands that wait for the LDS counter alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14 and expcnt bits 6:4 at their maxima, lgkmcnt in
// bits 11:8).
constexpr int kWaitLgkm8 = 0xC07F | (8 << 8);
constexpr int kWaitLgkm4 = 0xC07F | (4 << 8);
constexpr int kWaitLgkm0 = 0xC07F;

template <int POL>
__device__ __forceinline__ float fold_full_slab(const float* slab, float acc) {
    const float4* s4 = reinterpret_cast<const float4*>(slab);
    constexpr int G = kSlab / 16;  // groups of four float4
    auto grp = [&](int g, float4 (&q)[4]) {
        const int base = POL == kPolFoldRight ? 4 * (G - 1 - g) : 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = s4[base + i];
    };
    float4 q[3][4];
    grp(0, q[0]);
    grp(1, q[1]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (g + 2 < G) grp(g + 2, q[(g + 2) % 3]);
        fold_fence(acc);
        // one wait for the whole group: LDS reads complete in order, so
        // leaving the later groups' reads (4 each) outstanding suffices
        switch (min(2, G - 1 - g)) {
            case 2: __builtin_amdgcn_s_waitcnt(kWaitLgkm8); break;
            case 1: __builtin_amdgcn_s_waitcnt(kWaitLgkm4); break;
            default: __builtin_amdgcn_s_waitcnt(kWaitLgkm0); break;
        }
        __builtin_amdgcn_sched_barrier(0);
        float4 (&cur)[4] = q[g % 3];
        if constexpr (POL == kPolFoldRight) {
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                acc = cur[i].w + acc;
                acc = cur[i].z + acc;
                acc = cur[i].y + acc;
                acc = cur[i].x + acc;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = acc + cur[i].x;
                acc = acc + cur[i].y;
                acc = acc + cur[i].z;
                acc = acc + cur[i].w;
            }
        }
        fold_fence(acc);
    }
    return acc;
}

// The FP32 sum of c(x_j), j = 0 .. cols-1, in the order of policy POL,
// identical in all lanes.  `stk`: this wave's tree stack (kTreeStack floats).
// The row is read through buffer resources (reads past the row return 0, so
// the loads are unconditional), two slabs ahead of the fold.  Inlined into
// the kernel, so that `slab` stays an LDS address (an out-of-line copy reads
// it through flat loads, which slowed the dependent chain of adds by half).
template <int C, int POL>
__device__ __forceinline__ float ordered_sum(const float* xr, const float* rr, int cols, float ref, float* slab,
                                             float* stk, int lane) {
    const int nslab = (cols + kSlab - 1) / kSlab;
    const BufRes rx = make_res(xr, cols * 4);
    const BufRes rres = make_res(rr, rr ? cols * 4 : 0);
    auto slab_of = [&](int t) { return POL == kPolFoldRight ? nslab - 1 - t : t; };
    auto fetch = [&](int slab_id, float (&f)[kSlab / kWave]) {
#pragma unroll
        for (int i = 0; i < kSlab / kWave; ++i) {
            const int e = ordered_elem(slab_id, i, lane);
            f[i] = res_ld1(rx, e * 4);
            if (rr) f[i] = f[i] + res_ld1(rres, e * 4);
        }
    };
    float acc = 0.0f;
    int depth = 0;           // tree: subtrees on the stack
    unsigned done = 0;       // tree: slabs merged so far
    // one slab: contributions to LDS, then (`buf` free again) the loads of
    // slab `refill` into `buf`, then the fold / tree step
    auto step = [&](int t, float (&buf)[kSlab / kWave], int refill) {
        const int slab_id = slab_of(t);
        const int base = slab_id * kSlab;
#pragma unroll
        for (int i = 0; i < kSlab / kWave; ++i) {
            const int e = ordered_elem(slab_id, i, lane);
            // past the row: the add identity -0 (the tree's padding; never read by the folds)
            slab[kWave * i + lane] = e < cols ? contrib<C>(buf[i], ref) : -0.0f;
        }
        wave_sync();
        fetch(refill < nslab ? slab_of(refill) : nslab, buf);  // past the last slab: zeros, no traffic
        const int n = min(kSlab, cols - base);
        if constexpr (POL == kPolFoldLeft) {
            if (n == kSlab) {
                acc = fold_full_slab<POL>(slab, acc);
            } else {
                for (int j = 0; j < n; ++j) acc = acc + slab[j];
            }
        } else if constexpr (POL == kPolFoldRight) {
            if (n == kSlab) {
                acc = fold_full_slab<POL>(slab, acc);
            } else {
                for (int j = n - 1; j >= 0; --j) acc = slab[j] + acc;
            }
        } else {  // kPolTree
            const float4 q = *reinterpret_cast<const float4*>(slab + kVec * lane);
            float s = wave_allreduce<AddOp>((q.x + q.y) + (q.z + q.w));
            for (unsigned c = done; c & 1u; c >>= 1) s = stk[--depth] + s;  // left sibling + right
            wave_sync();
            if (lane == 0) stk[depth] = s;
            ++depth;
            ++done;
        }
        wave_sync();
    };
    // two register buffers, slabs t and t+1: the loads of slab t+2 go out as
    // soon as slab t's values are in LDS, so each slab's loads have two slab
    // folds to arrive
    float bufa[kSlab / kWave], bufb[kSlab / kWave];
    fetch(slab_of(0), bufa);
    // slab 0's loads stay ahead of slab 1's, as in the loop, so that the
    // first use of each buffer waits for its own loads only
    __builtin_amdgcn_sched_barrier(0);
    fetch(1 < nslab ? slab_of(1) : nslab, bufb);
    // both steps of a trip unconditional (an odd last slab is peeled), so
    // every path into a step has the same loads outstanding and each step
    // waits for its own buffer's loads only
    int t = 0;
    for (; t + 1 < nslab; t += 2) {
        step(t, bufa, t + 2);
        step(t + 1, bufb, t + 3);
    }
    if (t < nslab) step(t, bufa, t + 2);
    if constexpr (POL == kPolTree) {
        // partial subtrees, largest first: add from the smallest up (each one's
        // missing right sibling is all padding, -0, whose addition is exact)
        acc = stk[depth - 1];
        for (int k = depth - 2; k >= 0; --k) acc = stk[k] + acc;
    }
    return acc;
}

template <int OP, int POL>
__global__ void __launch_bounds__(1024) k_ordered(LR_ENTRY_PARAMS) {
    const KArgs a = LR_ENTRY_KARGS;
    __shared__ __attribute__((aligned(16))) float slabs[kMaxWaves][kSlab];
    __shared__ float stacks[kMaxWaves][kTreeStack];
    const int lane = (int)threadIdx.x % kWave;
    const int wave = (int)threadIdx.x / kWave;
    const int64_t row = row_of(blockIdx.x, a.Q, wave);
    if (row >= a.rows) return;  // no workgroup barrier in this kernel
    const int cols = a.cols;
    const float* xr = a.x + row * (int64_t)cols;
    float* slab = slabs[wave];
    float* stk = stacks[wave];
    const float n = (float)cols;

    const BufRes rx = make_res(xr, cols * 4);
    if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        const float m = row_max(rx, cols, lane);
        const float s = ordered_sum<kExpShift, POL>(xr, nullptr, cols, m, slab, stk, lane);
        if constexpr (OP == kCrossEntropy) {
            if (lane == 0) {
                const int64_t lab = a.labels[row];
                const float sel = (lab >= 0 && lab < (int64_t)cols) ? xr[lab] : 0.0f;
                a.losses[row] = logf(s) + (m - sel);
            }
        } else {
            const BufRes ry = make_res(a.y + row * (int64_t)cols, cols * 4);
            const float y = 1.0f / s;
            for (int base = 0; base < cols; base += kWave * kPass) {
                float v[kPass];
#pragma unroll
                for (int u = 0; u < kPass; ++u) v[u] = res_ld1(rx, pass_elem(base, u, lane) * 4);
                // e / s rounded once: div_rowsum unless some e of the trip
                // lies in (0, 2^-96), then the division (a choice per wave)
                unsigned lo = ~0u;
#pragma unroll
                for (int u = 0; u < kPass; ++u) {
                    v[u] = expf(v[u] - m);
                    lo = min(lo, rowsum_guard(v[u]));
                }
                if (__builtin_amdgcn_ballot_w64(lo < kRowsumTiny) == 0) {
#pragma unroll
                    for (int u = 0; u < kPass; ++u) res_st1(ry, pass_elem(base, u, lane) * 4, div_rowsum(v[u], s, y));
                } else {
#pragma unroll
                    for (int u = 0; u < kPass; ++u) res_st1(ry, pass_elem(base, u, lane) * 4, v[u] / s);
                }
            }
        }
    } else if constexpr (OP == kRowSum) {
        const float sum = ordered_sum<kValue, POL>(xr, nullptr, cols, 0.0f, slab, stk, lane);
        if (lane == 0) a.sums[row] = sum;
    } else if constexpr (OP == kRowMinMax) {
        // exact in any order: the wave tree, as the max fold above
        float lo = INFINITY, hi = -INFINITY;
        for (int base = 0; base < cols; base += kWave * kPass) {
            float v[kPass];
#pragma unroll
            for (int u = 0; u < kPass; ++u) v[u] = res_ld1(rx, pass_elem(base, u, lane) * 4);
#pragma unroll
            for (int u = 0; u < kPass; ++u) {
                if (pass_elem(base, u, lane) < cols) {
                    lo = fmin2(lo, v[u]);
                    hi = fmax2(hi, v[u]);
                }
            }
        }
        lo = wave_allreduce<MinOp>(lo);
        hi = wave_allreduce<MaxOp>(hi);
        if (lane == 0) {
            if (a.mins) a.mins[row] = lo;
            if (a.maxs) a.maxs[row] = hi;
        }
    } else if constexpr (OP == kRmsNorm) {
        const float ss = ordered_sum<kSquare, POL>(xr, nullptr, cols, 0.0f, slab, stk, lane);
        const float ms = ss / n;
        const float r = 1.0f / sqrtf(ms + a.eps);
        const BufRes ry = make_res(a.y + row * (int64_t)cols, cols * 4);
        const BufRes rg = make_res(a.gamma, a.gamma ? cols * 4 : 0);
        for (int base = 0; base < cols; base += kWave * kPass) {
            float v[kPass], g[kPass];
#pragma unroll
            for (int u = 0; u < kPass; ++u) {
                v[u] = res_ld1(rx, pass_elem(base, u, lane) * 4);
                g[u] = res_ld1(rg, pass_elem(base, u, lane) * 4);
            }
#pragma unroll
            for (int u = 0; u < kPass; ++u) {
                const float t = v[u] * r;
                res_st1(ry, pass_elem(base, u, lane) * 4, a.gamma ? t * g[u] : t);
            }
        }
    } else {  // LayerNorm; fused residual LayerNorm folds over x + residual
        const float* rr = OP == kAddLayerNorm ? a.residual + row * (int64_t)cols : nullptr;
        const float mu = ordered_sum<kValue, POL>(xr, rr, cols, 0.0f, slab, stk, lane) / n;
        const float var = ordered_sum<kCentredSquare, POL>(xr, rr, cols, mu, slab, stk, lane) / n;
        const float r = 1.0f / sqrtf(var + a.eps);
        const BufRes ry = make_res(a.y + row * (int64_t)cols, cols * 4);
        const bool with_sum = OP == kAddLayerNorm && a.sum_out != nullptr;
        const BufRes rs = make_res(with_sum ? a.sum_out + row * (int64_t)cols : nullptr, with_sum ? cols * 4 : 0);
        const BufRes rres = make_res(rr, rr ? cols * 4 : 0);
        const BufRes rg = make_res(a.gamma, a.gamma ? cols * 4 : 0);
        const BufRes rb = make_res(a.beta, a.beta ? cols * 4 : 0);
        for (int base = 0; base < cols; base += kWave * kPass) {
            // every read of a trip's elements precedes their writes (y or the
            // sum may be x or the residual itself)
            float c[kPass], g[kPass], b[kPass];
#pragma unroll
            for (int u = 0; u < kPass; ++u) {
                const int off = pass_elem(base, u, lane) * 4;
                c[u] = res_ld1(rx, off);
                if (rr) c[u] = c[u] + res_ld1(rres, off);
                g[u] = res_ld1(rg, off);
                b[u] = res_ld1(rb, off);
            }
#pragma unroll
            for (int u = 0; u < kPass; ++u) {
                const int off = pass_elem(base, u, lane) * 4;
                float t = (c[u] - mu) * r;
                if (a.gamma) t = t * g[u];
                if (a.beta) t = t + b[u];
                res_st1(ry, off, t);
                if (with_sum) res_st1(rs, off, c[u]);
            }
        }
    }
}

template <int POL>
hipError_t launch_ordered_pol(int op, const KArgs& a, const lr_plan& p, hipStream_t s) {
    const dim3 grid((unsigned)p.blocks), block(p.threads_per_block);
    switch (op) {
        case kSoftmax: hipLaunchKernelGGL((k_ordered<kSoftmax, POL>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case kRmsNorm: hipLaunchKernelGGL((k_ordered<kRmsNorm, POL>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case kLayerNorm: hipLaunchKernelGGL((k_ordered<kLayerNorm, POL>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case kCrossEntropy: hipLaunchKernelGGL((k_ordered<kCrossEntropy, POL>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case kAddLayerNorm: hipLaunchKernelGGL((k_ordered<kAddLayerNorm, POL>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case kRowSum: hipLaunchKernelGGL((k_ordered<kRowSum, POL>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        case kRowMinMax: hipLaunchKernelGGL((k_ordered<kRowMinMax, POL>), grid, block, 0, s, LR_ENTRY_ARGS(a)); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_ordered(int op, int policy, const KArgs& a, const lr_plan& p, hipStream_t s) {
    switch (policy) {
        case kPolFoldLeft: return launch_ordered_pol<kPolFoldLeft>(op, a, p, s);
        case kPolTree: return launch_ordered_pol<kPolTree>(op, a, p, s);
        case kPolFoldRight: return launch_ordered_pol<kPolFoldRight>(op, a, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lr
