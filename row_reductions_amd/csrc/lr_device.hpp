// Device helpers for gfx950: wave64 cross-lane reductions, the cross-wave
// combine through LDS and 128-bit global accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "lr_map.hpp"

namespace lr {

enum Op : int {
    kSoftmax = 0,
    kRmsNorm = 1,
    kLayerNorm = 2,
    kCrossEntropy = 3,
    kAddLayerNorm = 4,
    kRowSum = 5,
    kRowMinMax = 6
};

// LayerNorm statistics (mean, then centred variance) with a per-column affine.
constexpr bool is_layernorm(int op) { return op == kLayerNorm || op == kAddLayerNorm; }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Wave64 all-reduce.  Within each 16-lane DPP row: xor-1 and xor-2 quad
// permutes, then the half-row mirror and the row mirror, after which all 16
// lanes of a row hold the row's total.  Rows are then paired with gfx950's
// v_permlane16_swap (rows 0<->1, 2<->3) and halves with v_permlane32_swap:
// adding the two swapped copies gives every lane the pair total.  Each step
// combines the same two partials in every lane (only operand order differs,
// and add/max commute), so all 64 lanes finish with the same bits.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

struct AddOp {
    static __device__ __forceinline__ float apply(float a, float b) { return a + b; }
    static constexpr float identity() { return 0.0f; }
};
// Max of two floats: IEEE 754-2019 maximum (v_maximum*_f32 on gfx950; NaN
// propagates), which needs no input canonicalisation and folds three
// operands per instruction.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float fmin2(float a, float b) { return __builtin_elementwise_minimum(a, b); }

struct MaxOp {
    static __device__ __forceinline__ float apply(float a, float b) { return fmax2(a, b); }
    static constexpr float identity() { return -INFINITY; }
};
struct MinOp {
    static __device__ __forceinline__ float apply(float a, float b) { return fmin2(a, b); }
    static constexpr float identity() { return INFINITY; }
};

template <class R>
__device__ __forceinline__ float wave_allreduce(float v) {
    v = R::apply(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
    v = R::apply(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
    v = R::apply(v, dpp_mov<0x141>(v));  // row_half_mirror
    v = R::apply(v, dpp_mov<0x140>(v));  // row_mirror
    const unsigned b = __builtin_bit_cast(unsigned, v);
    auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    v = R::apply(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
    const unsigned c = __builtin_bit_cast(unsigned, v);
    auto q = __builtin_amdgcn_permlane32_swap(c, c, false, false);
    v = R::apply(__builtin_bit_cast(float, (unsigned)q[0]), __builtin_bit_cast(float, (unsigned)q[1]));
    // every lane holds the same value: keep it in a scalar register
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// Two independent wave64 all-reduces taken step by step side by side, so
// that each step's cross-lane moves of the two values overlap instead of
// running one whole chain after the other.  Same bits as two calls.
template <class R>
__device__ __forceinline__ void wave_allreduce2(float& a, float& b) {
    a = R::apply(a, dpp_mov<0xB1>(a));
    b = R::apply(b, dpp_mov<0xB1>(b));
    a = R::apply(a, dpp_mov<0x4E>(a));
    b = R::apply(b, dpp_mov<0x4E>(b));
    a = R::apply(a, dpp_mov<0x141>(a));
    b = R::apply(b, dpp_mov<0x141>(b));
    a = R::apply(a, dpp_mov<0x140>(a));
    b = R::apply(b, dpp_mov<0x140>(b));
    const unsigned ua = __builtin_bit_cast(unsigned, a), ub = __builtin_bit_cast(unsigned, b);
    auto pa = __builtin_amdgcn_permlane16_swap(ua, ua, false, false);
    auto pb = __builtin_amdgcn_permlane16_swap(ub, ub, false, false);
    a = R::apply(__builtin_bit_cast(float, (unsigned)pa[0]), __builtin_bit_cast(float, (unsigned)pa[1]));
    b = R::apply(__builtin_bit_cast(float, (unsigned)pb[0]), __builtin_bit_cast(float, (unsigned)pb[1]));
    const unsigned va = __builtin_bit_cast(unsigned, a), vb = __builtin_bit_cast(unsigned, b);
    auto qa = __builtin_amdgcn_permlane32_swap(va, va, false, false);
    auto qb = __builtin_amdgcn_permlane32_swap(vb, vb, false, false);
    a = R::apply(__builtin_bit_cast(float, (unsigned)qa[0]), __builtin_bit_cast(float, (unsigned)qa[1]));
    b = R::apply(__builtin_bit_cast(float, (unsigned)qb[0]), __builtin_bit_cast(float, (unsigned)qb[1]));
    a = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a)));
    b = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, b)));
}

// All-reduce over aligned groups of L lanes (L = 4, 8, 16, 32 or 64): the
// first log2(L) steps of the wave64 all-reduce above, after which every lane
// of a group holds the group's total (with the same bits in every lane of
// the group).  The result may differ between groups, so it stays per lane.
template <class R, int L>
__device__ __forceinline__ float group_allreduce(float v) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32 || L == 64, "group of 4 .. 64 lanes");
    if constexpr (L == kWave) {
        return wave_allreduce<R>(v);
    } else {
        v = R::apply(v, dpp_mov<0xB1>(v));                        // quad_perm [1,0,3,2]
        v = R::apply(v, dpp_mov<0x4E>(v));                        // quad_perm [2,3,0,1]
        if constexpr (L >= 8) v = R::apply(v, dpp_mov<0x141>(v));  // row_half_mirror
        if constexpr (L >= 16) v = R::apply(v, dpp_mov<0x140>(v)); // row_mirror
        if constexpr (L >= 32) {
            const unsigned b = __builtin_bit_cast(unsigned, v);
            auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
            v = R::apply(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
        }
        return v;
    }
}

// Merge of the S <= 16 per-wave values of a row team, held by lanes 0 .. S-1
// (the identity elsewhere): the four in-row steps of the all-reduce, then
// lane 0's value to every lane.  Two cross-row steps shorter than a wave64
// all-reduce; on MI355X (HIP-graph replays) LayerNorm 64 x 12289 5.37 ->
// 5.28 us and RMSNorm 256 x 3072 2.64 -> 2.55 us.
template <class R>
__device__ __forceinline__ float team_merge(float v) {
    v = R::apply(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
    v = R::apply(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
    v = R::apply(v, dpp_mov<0x141>(v));  // row_half_mirror
    v = R::apply(v, dpp_mov<0x140>(v));  // row_mirror
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// Reduction over a row team of S wavefronts ("TIRx Metal reduction
// lowering", section 4.2 protocol): wave collective in every wave, lane 0
// publishes its wave's partial to LDS, one workgroup barrier, then every wave
// re-reduces the S partials (identity in the other lanes), so all workers hold
// the row result with no broadcast barrier.  `slots` is this round's LDS
// array of Q*S floats; separate rounds use separate arrays, so no second
// barrier is needed.  S is uniform over the workgroup, so the barrier is
// reached by every thread or by none.
template <class R>
__device__ __forceinline__ float team_reduce(float v, float* slots, int S, const Team& t) {
    v = wave_allreduce<R>(v);
    if (S > 1) {
        if (t.lane == 0) slots[t.q * S + t.s] = v;
        __syncthreads();
        const float u = (t.lane < S) ? slots[t.q * S + t.lane] : R::identity();
        v = team_merge<R>(u);
    }
    return v;
}

// ---------------------------------------------------------------------------
// Memory access.  Rows are read through their 16-byte aligned grid: a chunk
// that holds at least one row element lies inside one page of the tensor's
// allocation, so reading the whole chunk cannot fault even where its other
// floats belong to a neighbouring row; those floats are replaced by the
// identity before use and are never written.
// ---------------------------------------------------------------------------
// Cache policy.  Every row element is read once and written once, so the
// row stream carries the nontemporal (streaming) hint on loads and stores;
// the per-column parameters (gamma, beta) are re-read by every workgroup and
// use ordinary cached loads.
#ifndef LR_NT_LOADS
#define LR_NT_LOADS 1
#endif
#ifndef LR_NT_STORES
#define LR_NT_STORES 1
#endif

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// Row-stream load.
__device__ __forceinline__ float4 ld4(const float4* p) {
    if constexpr (LR_NT_LOADS) {
        const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    } else {
        return *p;
    }
}

// Cached load (parameters reused across workgroups).
__device__ __forceinline__ float4 ld4_cached(const float4* p) { return *p; }

// Row-stream store.
__device__ __forceinline__ void st4(float4* p, float4 v) {
    if constexpr (LR_NT_STORES) {
        v4f w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<v4f*>(p));
    } else {
        *p = v;
    }
}

// ---------------------------------------------------------------------------
// Buffer resources.  A resource covers `bytes` bytes from a wave-uniform base;
// a load past the end returns 0 and a store past the end is dropped, so
// straight-line code needs no per-lane bounds test to stay inside the range.
// Offsets passed here are never negative.  A null base with 0 bytes is a valid
// empty resource (every load returns 0).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t BufRes;

constexpr int kAuxNt = 2;  // cache policy: nontemporal (streamed once)
constexpr int kAuxDefault = 0;

__device__ __forceinline__ uint64_t wave_uniform(uint64_t u) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Word 3 of the resource: 32-bit data format, raw (unswizzled) addressing.
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ BufRes make_res(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(wave_uniform(reinterpret_cast<uint64_t>(base))),
                                             (short)0, __builtin_amdgcn_readfirstlane(bytes), kBufWord3);
}

template <int AUX>
__device__ __forceinline__ float4 res_ld4(BufRes r, int byte_off) {
    const v4f v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, AUX);
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float res_ld1(BufRes r, int byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kAuxDefault));
}

__device__ __forceinline__ void res_st1(BufRes r, int byte_off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, byte_off, 0,
                                          LR_NT_STORES ? kAuxNt : kAuxDefault);
}

__device__ __forceinline__ void res_st4(BufRes r, int byte_off, float4 v) {
    const v4f w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, byte_off, 0, LR_NT_STORES ? kAuxNt : kAuxDefault);
}

__device__ __forceinline__ float get(const float4& v, int j) {
    return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

__device__ __forceinline__ void set(float4& v, int j, float f) {
    if (j == 0) v.x = f; else if (j == 1) v.y = f; else if (j == 2) v.z = f; else v.w = f;
}

__device__ __forceinline__ float4 splat4(float f) { return make_float4(f, f, f, f); }

// Replace the floats of chunk k that are not row elements by `id`.
__device__ __forceinline__ void mask_chunk(float4& v, int k, int phase, int cols, float id) {
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        if (!elem_valid(elem_index(k, j, phase), cols)) set(v, j, id);
    }
}

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float fast_log(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// a / s rounded once (the IEEE quotient) in three instructions, for s >= 1
// and y = 1 / s rounded once: q = a y, r = a - s q (exact, by the fused
// multiply-add), then q + r y rounded once (P. Markstein's correction of a
// quotient from a correctly rounded reciprocal, IBM J. Res. Dev. 34(1),
// 1990).  The argument needs q and r clear of the subnormal range; a == 0
// or a >= 2^-96 keeps them there (q >= 2^-120).  Below that the result can
// be one unit off (a near 2^-121 and smaller), so callers check their
// numerators with rowsum_guard first.  The translation units that call this
// must not contract a * y into the fma.
__device__ __forceinline__ float div_rowsum(float a, float s, float y) {
    const float q = a * y;
    return __builtin_fmaf(__builtin_fmaf(-q, s, a), y, q);
}

// The unsigned minimum of rowsum_guard(a) over a set of non-negative
// numerators is below kRowsumTiny exactly when one of them lies in
// (0, 2^-96), where div_rowsum may differ from the division: the bit pattern
// minus one, so that zeros wrap to the top.
constexpr unsigned kRowsumTiny = 0x0F7FFFFFu;  // bits(2^-96) - 1
__device__ __forceinline__ unsigned rowsum_guard(float a) { return __float_as_uint(a) - 1u; }

// 1/sqrt(x) to about one ulp with the hardware reciprocal square root, which
// takes a subnormal argument as zero and returns +inf.  An argument below
// 2^-126 (eps = 0 and a row whose mean square or variance is subnormal) is
// scaled by 2^24 into the normal range first and the result by 2^12; both
// scalings are exact.
__device__ __forceinline__ float fast_rsqrt(float x) {
    const bool sub = x < 0x1p-126f;
    const float r = __builtin_amdgcn_rsqf(sub ? x * 0x1p24f : x);
    return sub ? r * 0x1p12f : r;
}

// Softmax state over a row team with one exchange: every wave brings its
// own (max m_w, sum of exp(x - m_w)) pair, lane 0 publishes it, one workgroup
// barrier, then every wave merges the S pairs with the (max, sum of
// exponentials) merge of Milakov and Gimelshein's online normaliser
// ("Online normalizer calculation for softmax", 2018; the pages compose max,
// sum of exp and the division, section 1, but give no merge):
// M = max_w m_w, s = sum_w s_w exp(m_w - M).  A wave with no element of the row brings
// (-inf, 0).  `sm`, `ss`: this round's LDS arrays of Q*S floats.
struct MaxSum {
    float m, s;
};

__device__ __forceinline__ MaxSum team_maxsum(float m, float s, float* sm, float* ss, int S, const Team& t) {
    if (S > 1) {
        if (t.lane == 0) {
            sm[t.q * S + t.s] = m;
            ss[t.q * S + t.s] = s;
        }
        __syncthreads();
        const bool in = t.lane < S;
        const float mi = in ? sm[t.q * S + t.lane] : -INFINITY;
        const float si = in ? ss[t.q * S + t.lane] : 0.0f;
        const float M = team_merge<MaxOp>(mi);
        const float sc = (mi == -INFINITY) ? 0.0f : si * fast_exp(mi - M);
        return MaxSum{M, team_merge<AddOp>(sc)};
    }
    return MaxSum{m, s};
}

}  // namespace lr
