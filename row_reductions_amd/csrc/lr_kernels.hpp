// Unordered-policy kernels: the CACHE family (row stripe kept in VGPRs) and
// the STREAM family (passes reload the row).  Instantiated once per op by
// the k_<op>.hip translation units.
//
// Roles of the steps ("TIRx Metal reduction lowering"):
//   section 1   softmax: exp(x - max) / sum;  cross-entropy: log(sum) + (max - selected),
//               the difference first: it is exact whenever selected >= max / 2
//               (Sterbenz), so a confident prediction's small loss is not lost
//               in the rounding of max + log(sum)
//   section 4   S waves cooperate on a row, Q rows share a workgroup
//   section 4.4 blocked-cyclic ownership, V = 4 (one 128-bit access per chunk)
//   section 5   the row's chunks are kept per worker (here: in VGPRs) so every
//               pass after the first reads registers, not memory
//   section 5.1 LayerNorm mean, then variance of the centred values
//   section 5.2 cross-entropy reads logits[row, label] from the global tensor
//               under a 0 <= label < cols guard (fill 0)
#pragma once

#include "lr_device.hpp"
#include "lr_entry.hpp"
#include "lr_internal.hpp"

namespace lr {

template <int OP>
constexpr float op_identity() {
    // row minimum and maximum share one stripe: missing elements hold NaN,
    // which the minimum/maximum-number folds skip
    return (OP == kSoftmax || OP == kCrossEntropy) ? -INFINITY : (OP == kRowMinMax ? __builtin_nanf("") : 0.0f);
}

// IEEE minNum / maxNum: a NaN operand yields the other one.
__device__ __forceinline__ float fminnum(float a, float b) { return __builtin_fminf(a, b); }
__device__ __forceinline__ float fmaxnum(float a, float b) { return __builtin_fmaxf(a, b); }

// Writes the row's minimum and maximum after the stripe folds: a lane that
// held no element of the row still has NaN and takes the identities.
// A row's team reduction: S cooperating waves (LW = 64), or a sub-wave team
// of LW lanes (one DPP group, no LDS).
template <class R, int LW>
__device__ __forceinline__ float row_reduce(float v, float* slots, int S, const Team& t) {
    if constexpr (LW < kWave) {
        return group_allreduce<R, LW>(v);
    } else {
        return team_reduce<R>(v, slots, S, t);
    }
}

template <int LW = kWave>
__device__ __forceinline__ void finish_minmax(const KArgs& a, float lo, float hi, float* red_lo, float* red_hi,
                                              int S, const Team& t, bool active, int64_t row) {
    lo = __builtin_isnan(lo) ? INFINITY : lo;
    hi = __builtin_isnan(hi) ? -INFINITY : hi;
    lo = row_reduce<MinOp, LW>(lo, red_lo, S, t);
    hi = row_reduce<MaxOp, LW>(hi, red_hi, S, t);
    if (active && t.w == 0) {
        if (a.mins) a.mins[row] = lo;
        if (a.maxs) a.maxs[row] = hi;
    }
}

// Reads label[row] and the guarded logit once per row (worker 0 of the team).
__device__ __forceinline__ float gather_label(const KArgs& a, const float* xr, int64_t row) {
    const int64_t lab = a.labels[row];
    return (lab >= 0 && lab < (int64_t)a.cols) ? xr[lab] : 0.0f;
}

// Stores out, the values of chunk k of the x row's grid (phase h), into the
// destination row dr.  `same_phase`: dr starts at the x row's 16-byte phase,
// so whole chunks can be stored as one 128-bit access.
template <bool AL>
__device__ __forceinline__ void store_chunk(float* dr, bool same_phase, int k, int h, int cols, float4 out) {
    if (AL) {
        st4(reinterpret_cast<float4*>(dr) + k, out);
    } else if (same_phase && chunk_full(k, h, cols)) {
        st4(reinterpret_cast<float4*>(dr - h) + k, out);
    } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int e = elem_index(k, j, h);
            if (elem_valid(e, cols)) dr[e] = get(out, j);
        }
    }
}

// Keeps the values of o[] computed here, ahead of the stores that follow.
// Without it the compiler moves each chunk's arithmetic, and the wait for
// its parameter load, into that chunk's store branch, behind the stores of
// the chunks before it; on gfx9 a store counts in the same vmcnt as the
// loads, so that wait then includes the earlier stores' completion.
template <int N>
__device__ __forceinline__ void pin_chunks(float4 (&o)[N]) {
#pragma unroll
    for (int c = 0; c < N; ++c) {
        float x = o[c].x, y = o[c].y, z = o[c].z, w = o[c].w;
        asm volatile("" : "+v"(x), "+v"(y), "+v"(z), "+v"(w)::"memory");
        o[c] = make_float4(x, y, z, w);
    }
}

// Chunk k of a row that sits at its own (unknown) phase, read one float at a
// time at clamped, in-range indexes of the x row's grid (phase h); grid slots
// outside [0, cols) hold some element of the row and must not be used.
// `base`: byte offset of the row within the resource.
__device__ __forceinline__ float4 elem_chunk(BufRes r, int k, int h, int cols, int base = 0) {
    float4 g;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        const int e = min(max(elem_index(k, j, h), 0), cols - 1);
        set(g, j, res_ld1(r, base + e * 4));
    }
    return g;
}

// Per-column parameter (gamma or beta) for chunk k; `fill` where absent.
// Used by the STREAM family.
template <bool AL>
__device__ __forceinline__ float4 param_chunk(const float* p, int k, int h, int cols, float fill) {
    if (p == nullptr) return splat4(fill);
    if (AL) return ld4_cached(reinterpret_cast<const float4*>(p) + k);
    float4 g;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        const int e = elem_index(k, j, h);
        set(g, j, elem_valid(e, cols) ? p[e] : fill);
    }
    return g;
}

// How a kernel instance reads the per-column parameters (gamma, beta).
//   kParNone:    no parameter present; nothing is loaded.
//   kParAll:     every parameter the op uses is present.
//   kParRuntime: some present, some not; absent ones read an empty resource
//                (zeros) and take their fill value.
enum ParamMode : int { kParNone = 0, kParAll = 1, kParRuntime = 2 };

// A per-column parameter vector p (gamma or beta, cols floats) as a buffer
// resource.  Aligned rows (p 16-byte aligned too) read it as 16-byte blocks
// from p.  Misaligned rows read whole 16-byte blocks of p's own grid (phase
// hp): the resource starts at the block holding p[0] and ends with the
// block holding p[cols - 1], so no read leaves a block that holds p's data.
// Absent: an empty resource (every read returns 0).
struct ParamRes {
    BufRes r;
    int hp;
};

template <bool AL>
__device__ __forceinline__ ParamRes param_res(const float* p, int cols, bool present) {
    if (AL || !present) return ParamRes{make_res(p, present ? cols * 4 : 0), 0};
    const int hp = phase_of(reinterpret_cast<uintptr_t>(p));
    return ParamRes{make_res(p - hp, (cols + hp + kVec - 1) / kVec * 16), hp};
}

// Chunk k of a parameter vector, in the row's 16-byte grid of phase h: slot
// j holds p[4k + j - h].  Straight-line.  Aligned rows: one 16-byte read (a
// chunk past the end reads zeros).  Misaligned rows: element 4k + j - h sits
// at position 4k + j + d of p's grid (d = hp - h, -3..3), so the chunk is
// the two blocks from k + floor(d / 4) shifted by d mod 4 -- two 16-byte
// reads and selects in place of four 4-byte reads (those cost misaligned
// LayerNorm 262144 x 50 on MI355X 12.6 us for gamma and 4.6 more for beta).
// Grid slots outside the row hold other elements or 0 and are never used.
template <bool AL, int PM>
__device__ __forceinline__ float4 param_load(const ParamRes& pr, bool present, int k, int h, int cols, float fill) {
    if constexpr (PM == kParNone) {
        return splat4(fill);
    } else {
        float4 g;
        if constexpr (AL) {
            g = res_ld4<kAuxDefault>(pr.r, k * 16);
        } else {
            const int d = pr.hp - h;
            const int kb = k + (d >> 2);  // arithmetic shift: floor(d / 4)
            const int sh = d & 3;
            // block -1 (k = 0, d < 0) holds no element of p: an offset past
            // the resource, which reads 0
            const float4 A = res_ld4<kAuxDefault>(pr.r, kb >= 0 ? kb * 16 : 0x7ffffff0);
            const float4 B = res_ld4<kAuxDefault>(pr.r, kb * 16 + 16);
            g.x = sh == 0 ? A.x : sh == 1 ? A.y : sh == 2 ? A.z : A.w;
            g.y = sh == 0 ? A.y : sh == 1 ? A.z : sh == 2 ? A.w : B.x;
            g.z = sh == 0 ? A.z : sh == 1 ? A.w : sh == 2 ? B.x : B.y;
            g.w = sh == 0 ? A.w : sh == 1 ? B.x : sh == 2 ? B.y : B.z;
        }
        if constexpr (PM == kParRuntime) {
            if (!present) g = splat4(fill);
        }
        return g;
    }
}

// The same chunk, on a misaligned row, read by a whole-wave team whose lanes
// hold several chunks each.  For every chunk of a row but its first and its
// last, p[4k - h] .. p[4k + 3 - h] lie inside p's blocks (they sit at grid
// positions q .. q + 3, q = 4k + hp - h: q >= 4 - 3 > 0 for k >= 1, and
// q + 4 <= cols + hp for every k below the last), so one 16-byte read at the
// 4-byte aligned offset 4q returns the chunk.  `edge` (wave-uniform) says
// this wave may hold the row's first or last chunk at this k: then the
// two-block read above.  Being uniform, the test leaves the other waves'
// reads straight-line.  On MI355X, against two reads for every chunk
// (HIP-graph replays): LayerNorm 64 x 12289 5.88 -> 5.64 us, the fused
// residual LayerNorm 64 x 12289 7.15 -> 6.61, RMSNorm 256 x 12289 6.55 ->
// 6.26, RMSNorm 4096 x 1030 7.45 -> 7.03, LayerNorm 256 x 12289 7.56 -> 7.63.
// (A per-lane test instead sent waves holding several rows down both paths:
// LayerNorm 262144 x 50 24.8 -> 38.6 us.)  A chunk past the row reads zeros
// or other elements of p, which are never used.  The two-block read is
// written out here rather than shared with param_load: that is the form
// measured above (the compiler schedules these kernels' store loops
// differently otherwise).
template <int PM>
__device__ __forceinline__ float4 param_load_wide(const ParamRes& pr, bool present, int k, int h, float fill,
                                                  bool edge) {
    if constexpr (PM == kParNone) {
        return splat4(fill);
    } else {
        float4 g;
        if (!edge) {
            g = res_ld4<kAuxDefault>(pr.r, (kVec * k + pr.hp - h) * 4);
        } else {
            const int d = pr.hp - h;
            const int kb = k + (d >> 2);
            const int sh = d & 3;
            const float4 A = res_ld4<kAuxDefault>(pr.r, kb >= 0 ? kb * 16 : 0x7ffffff0);
            const float4 B = res_ld4<kAuxDefault>(pr.r, kb * 16 + 16);
            g.x = sh == 0 ? A.x : sh == 1 ? A.y : sh == 2 ? A.z : A.w;
            g.y = sh == 0 ? A.y : sh == 1 ? A.z : sh == 2 ? A.w : B.x;
            g.z = sh == 0 ? A.z : sh == 1 ? A.w : sh == 2 ? B.x : B.y;
            g.w = sh == 0 ? A.w : sh == 1 ? B.x : sh == 2 ? B.y : B.z;
        }
        if constexpr (PM == kParRuntime) {
            if (!present) g = splat4(fill);
        }
        return g;
    }
}

// Parameters of a norm (gamma; gamma and beta for LayerNorm).
template <int OP>
constexpr int num_params() {
    return is_layernorm(OP) ? 2 : (OP == kRmsNorm ? 1 : 0);
}

// Wave index within the workgroup, as a scalar (uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// ===========================================================================
// CACHE family: worker w keeps chunks k = w + W*c, c < NCH, in registers.
//
// Row, team and base addresses are wave-uniform and live in scalar
// registers.  The row is read through a buffer resource covering its chunks,
// so every load is issued unconditionally (a slot past the row's last chunk
// reads zeros and then takes the identity) and each wait covers only the
// loads it needs.
//
// The per-column parameters are read chunk by chunk in the store loop.  Every
// workgroup reads the same few kilobytes of gamma/beta, so the alternatives
// measured on MI355X (768 x 6144) concentrate requests on the same L2 lines:
// issuing them with the row loads, or as one burst per wave before the last
// reduction, was 0.3-2 us slower; rotating each workgroup's chunk order to
// spread those requests cost more in the row stream than it saved.
// ===========================================================================
// The body of both CACHE kernels.  LW = 64: a row team of S waves (k_cache).
// LW = 4, 8, 16 or 32: sub-wave teams for narrow rows (k_cache_narrow), 64 /
// LW rows per wave.  Row, phase and chunk count are then per lane, and the
// row is read through one resource per wave covering all its rows: a lane's
// chunk k sits at byte xo + 16 k, xo being its row's 16-byte grid base
// relative to the wave's first row's.  Past a row's chunks that resource
// holds the next row, so every slot past the row takes the identity.
template <int OP, int NCH, bool AL, int PM, int LW>
__device__ __forceinline__ void cache_body(const KArgs& a, float (&red)[4][kMaxWaves]) {
    constexpr bool NARROW = LW < kWave;
    constexpr float ID = op_identity<OP>();
    constexpr int NP = num_params<OP>();
    const int S = NARROW ? 1 : a.S;
    const int W = NARROW ? LW : kWave * S;
    const int lane = (int)threadIdx.x & (kWave - 1);
    const Team t = NARROW ? team_of_group(wave_id(), lane, LW) : team_of_wave(wave_id(), lane, S, a.team_magic);
    const int64_t row = row_of(blockIdx.x, a.Q, t.q);
    const bool active = row < a.rows;
    const int cols = a.cols;
    const float* xr = a.x + (active ? row : 0) * (int64_t)cols;
    const int h = AL ? 0 : phase_of(reinterpret_cast<uintptr_t>(xr));
    const int nv = active ? (AL ? cols / kVec : chunks_of(h, cols)) : 0;
    const ParamRes rg = param_res<AL>(a.gamma, cols, NP >= 1 && a.gamma);
    const ParamRes rb = param_res<AL>(a.beta, cols, NP == 2 && a.beta);
    // fused residual: read on the x grid where its rows sit at x's phases
    // (below), else one float at a time
    constexpr bool RES = OP == kAddLayerNorm;
    const int64_t roff = (active ? row : 0) * (int64_t)cols;
    BufRes rx, rr;
    int xo = 0, ro = 0;  // byte offsets of this lane's row in rx and rr
    const float* rx_base;  // rx covers rx_bytes from rx_base
    int rx_bytes;
    if constexpr (!NARROW) {
        rx_base = xr - h;
        rx_bytes = nv * 16;
        rx = make_res(rx_base, rx_bytes);
        rr = make_res(RES ? a.residual + roff : nullptr, RES && active ? (AL ? nv * 16 : cols * 4) : 0);
    } else {
        const int64_t r0 = row_of(blockIdx.x, a.Q, wave_id() * (kWave / LW));  // the wave's first row
        const int64_t left = a.rows - r0;
        const int nr = left <= 0 ? 0 : (left < kWave / LW ? (int)left : kWave / LW);  // its rows that exist
        const int64_t off0 = (nr > 0 ? r0 : 0) * (int64_t)cols;
        const int h0 = AL ? 0 : phase_of(reinterpret_cast<uintptr_t>(a.x + off0));
        const int xbytes = (nr * cols + h0 + kVec - 1) / kVec * 16;
        rx_base = a.x + off0 - h0;
        rx_bytes = xbytes;
        rx = make_res(rx_base, xbytes);
        xo = active ? (int)(((row - r0) * cols - h + h0) * 4) : 0;
        rr = make_res(RES ? a.residual + off0 : nullptr, RES ? (AL ? xbytes : nr * cols * 4) : 0);
        ro = active ? (int)((row - r0) * cols * 4) : 0;
    }
    auto chunk = [&](int c) { return chunk_index(t.w, W, c); };

    // cross-entropy on narrow teams: the label is read before the rows, so
    // that the gather of its logit waits for the label alone (loads complete
    // in order) and overlaps the rows' loads.  Both loads are unconditional
    // (through resources: a lane past the last row reads 0), so that every
    // path has the same loads outstanding.  Against a gather after the rows:
    // cross-entropy 262144 x 32 11.8 -> 10.0 us on MI355X.  Whole-wave teams
    // keep the gather by the team's first wave after the row's loads: done
    // this way there, every wave of the team waited for its whole row first
    // (4096 x 32000 at 8 waves per row: 76.9 -> 80.7 us).
    int64_t lab = 0;
    if constexpr (OP == kCrossEntropy && NARROW) {
        const int64_t r0 = row_of(blockIdx.x, a.Q, wave_id() * (kWave / LW));
        const int64_t left = a.rows - r0;
        const int nr = left <= 0 ? 0 : (left < kWave / LW ? (int)left : kWave / LW);
        const BufRes rl = make_res(a.labels + (nr > 0 ? r0 : 0), nr * 8);
        const v2i w = __builtin_amdgcn_raw_buffer_load_b64(rl, active ? (int)(row - r0) * 8 : 0, 0, kAuxDefault);
        __builtin_amdgcn_sched_barrier(0);  // keeps the label load ahead of the rows'
        lab = (int64_t)(((uint64_t)(uint32_t)w[1] << 32) | (uint32_t)w[0]);
    }

    // narrow teams: gamma / beta (one or two chunks per lane, the same for
    // every row) are read before the rows, so that the store loop does not
    // wait for them after the reductions.  Whole-wave teams read them chunk
    // by chunk in the store loop (see above).
    float4 gpre[NARROW && NP >= 1 ? NCH : 1], bpre[NARROW && NP == 2 ? NCH : 1];
    if constexpr (NARROW && NP >= 1) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            gpre[c] = param_load<AL, PM>(rg, a.gamma != nullptr, chunk(c), h, cols, 1.0f);
            if constexpr (NP == 2) bpre[c] = param_load<AL, PM>(rb, a.beta != nullptr, chunk(c), h, cols, 0.0f);
        }
    }
    // misaligned rows, whole-wave teams with several chunks per lane: does
    // this wave's chunk c hold the row's first or last chunk (its lanes hold
    // k = k0 .. k0 + 63)?  With one chunk per lane nearly every wave does:
    // those plans keep the two-block read.
    auto edge_of = [&](int c) {
        const int k0 = t.s * kWave + W * c;
        return k0 == 0 || (k0 < nv && nv <= k0 + kWave);
    };
    auto gamma_of = [&](int c, int k) {
        if constexpr (NARROW && NP >= 1) return gpre[c];
        if constexpr (!AL && NCH >= 2) {
            return param_load_wide<PM>(rg, a.gamma != nullptr, k, h, 1.0f, edge_of(c));
        } else {
            return param_load<AL, PM>(rg, a.gamma != nullptr, k, h, cols, 1.0f);
        }
    };
    auto beta_of = [&](int c, int k) {
        if constexpr (NARROW && NP == 2) return bpre[c];
        if constexpr (!AL && NCH >= 2) {
            return param_load_wide<PM>(rb, a.beta != nullptr, k, h, 0.0f, edge_of(c));
        } else {
            return param_load<AL, PM>(rb, a.beta != nullptr, k, h, cols, 0.0f);
        }
    };

    constexpr int AUX = LR_NT_LOADS ? kAuxNt : kAuxDefault;
    float4 v[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) v[c] = res_ld4<AUX>(rx, xo + chunk(c) * 16);
    if constexpr (RES) {
        // the residual: on aligned rows, and on misaligned rows when its
        // tensor starts at x's phase (so every residual row sits at its x
        // row's phase), the same 16-byte reads as x; otherwise one float at a
        // time.  The choice is uniform and outside the loops, so that every
        // path issues all its loads before the first use.
        float4 q[NCH];
        if constexpr (AL) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) q[c] = res_ld4<AUX>(rr, ro + chunk(c) * 16);
        } else if (phase_of(reinterpret_cast<uintptr_t>(a.residual)) == phase_of(reinterpret_cast<uintptr_t>(a.x))) {
            const BufRes rm = make_res(a.residual + (rx_base - a.x), rx_bytes);
#pragma unroll
            for (int c = 0; c < NCH; ++c) q[c] = res_ld4<AUX>(rm, xo + chunk(c) * 16);
        } else {
#pragma unroll
            for (int c = 0; c < NCH; ++c) q[c] = elem_chunk(rr, chunk(c), h, cols, ro);
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            v[c] = make_float4(v[c].x + q[c].x, v[c].y + q[c].y, v[c].z + q[c].z, v[c].w + q[c].w);
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int k = chunk(c);
        if constexpr (!(ID == 0.0f && AL && !NARROW)) {  // else past the end: zeros, the add identity
            v[c] = (k < nv) ? v[c] : splat4(ID);
            if (!AL) mask_chunk(v[c], k, h, cols, ID);
        }
    }

    if constexpr (NARROW && NP >= 1) {
        // the parameters are used only in the store loop's `k < nv` branch;
        // without this the compiler moves their loads down there
        auto pin = [](float4& q) {
            float x = q.x, y = q.y, z = q.z, w = q.w;
            asm volatile("" : "+v"(x), "+v"(y), "+v"(z), "+v"(w));
            q = make_float4(x, y, z, w);
        };
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            pin(gpre[c]);
            if constexpr (NP == 2) pin(bpre[c]);
        }
    }

    float sel = 0.0f;
    if constexpr (OP == kCrossEntropy && NARROW) {
        // the labelled logit (element lab of the row: byte xo + 4 (h + lab)
        // of the rows' resource), 0 for a label outside [0, cols)
        const bool in = lab >= 0 && lab < (int64_t)cols;
        const float g = res_ld1(rx, xo + (h + (in ? (int)lab : 0)) * 4);
        sel = in ? g : 0.0f;
    } else if constexpr (OP == kCrossEntropy) {
        if (active && t.w == 0) sel = gather_label(a, xr, row);
    }

    if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        // each wave folds (max, sum of exp) over its own chunks with no
        // barrier; one exchange merges the S pairs.  Two dependent team
        // reductions (max, then the sum) cost a second workgroup barrier,
        // 0.07-0.3 us per launch at 768 x 6144 on MI355X.
        float m = ID;
#pragma unroll
        for (int c = 0; c < NCH; ++c) m = fmax2(fmax2(m, fmax2(v[c].x, v[c].y)), fmax2(v[c].z, v[c].w));
        m = group_allreduce<MaxOp, LW>(m);
        // a wave whose elements are all -inf (masked, or past the row's end)
        // shifts by 0 instead of by its maximum: its exponentials are then
        // exp(-inf) = 0 (its outputs +0, not -inf * 0), and it brings
        // (-inf, 0) to the merge
        const float mm = (m == -INFINITY) ? 0.0f : m;
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            v[c].x = fast_exp(v[c].x - mm);
            v[c].y = fast_exp(v[c].y - mm);
            v[c].z = fast_exp(v[c].z - mm);
            v[c].w = fast_exp(v[c].w - mm);
            s += (v[c].x + v[c].y) + (v[c].z + v[c].w);
        }
        s = group_allreduce<AddOp, LW>(s);
        const MaxSum ms = team_maxsum(m, s, red[0], red[1], S, t);
        if constexpr (OP == kCrossEntropy) {
            if (active && t.w == 0) a.losses[row] = fast_log(ms.s) + (ms.m - sel);
        } else {
            // y = exp(x - m_w) * exp(m_w - M) / s
            const float r = (m == -INFINITY) ? 0.0f : fast_exp(m - ms.m) * fast_rcp(ms.s);
            float* yr = a.y + row * (int64_t)cols;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int k = chunk(c);
                if (k < nv) {
                    const float4 o = make_float4(v[c].x * r, v[c].y * r, v[c].z * r, v[c].w * r);
                    store_chunk<AL>(yr, a.y_same_phase, k, h, cols, o);
                }
            }
        }
    } else if constexpr (OP == kRowSum) {
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) sum += (v[c].x + v[c].y) + (v[c].z + v[c].w);
        sum = row_reduce<AddOp, LW>(sum, red[0], S, t);
        if (active && t.w == 0) a.sums[row] = sum;
    } else if constexpr (OP == kRowMinMax) {
        float lo = ID, hi = ID;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            lo = fminnum(fminnum(lo, fminnum(v[c].x, v[c].y)), fminnum(v[c].z, v[c].w));
            hi = fmaxnum(fmaxnum(hi, fmaxnum(v[c].x, v[c].y)), fmaxnum(v[c].z, v[c].w));
        }
        finish_minmax<LW>(a, lo, hi, red[0], red[1], S, t, active, row);
    } else if constexpr (OP == kRmsNorm) {
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            ss += (v[c].x * v[c].x + v[c].y * v[c].y) + (v[c].z * v[c].z + v[c].w * v[c].w);
        ss = row_reduce<AddOp, LW>(ss, red[0], S, t);
        const float r = fast_rsqrt(ss * a.inv_cols + a.eps);
        float* yr = a.y + row * (int64_t)cols;
        // every gamma chunk is requested at once, then every output formed,
        // then every chunk stored back to back, so that no wait for a gamma
        // chunk comes after a store (768 x 6144 on MI355X: 6.83 us at six
        // waves per row, against 6.91 us for a load, wait and store per chunk
        // at nine).  LayerNorm keeps the per-chunk loop, which measured
        // faster for it (6.93 against 7.00 us).
        float4 o[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const float4 g = gamma_of(c, chunk(c));
            o[c] = make_float4(v[c].x * r * g.x, v[c].y * r * g.y, v[c].z * r * g.z, v[c].w * r * g.w);
        }
        pin_chunks(o);
        if constexpr (AL && !NARROW) {
            // through a resource over the row: a chunk past its end is dropped
            const BufRes ry = make_res(yr, nv * 16);
#pragma unroll
            for (int c = 0; c < NCH; ++c) res_st4(ry, chunk(c) * 16, o[c]);
        } else {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int k = chunk(c);
                if (k < nv) store_chunk<AL>(yr, a.y_same_phase, k, h, cols, o[c]);
            }
        }
    } else {  // LayerNorm, fused residual LayerNorm
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) sum += (v[c].x + v[c].y) + (v[c].z + v[c].w);
        if constexpr (RES) {
            if (a.sum_out != nullptr) {
                float* sr = a.sum_out + row * (int64_t)cols;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const int k = chunk(c);
                    if (k < nv) store_chunk<AL>(sr, a.s_same_phase, k, h, cols, v[c]);
                }
            }
        }
        // the centred statistics: mean, then the sum of squared deviations
        float qs;
        bool two_pass = true;
        if constexpr (!NARROW) two_pass = S == 1;
        if (two_pass) {
            // one wave (or a sub-wave team) holds the row: the mean, then
            // the centred sum of squares, each reduced without an exchange
            sum = row_reduce<AddOp, LW>(sum, red[0], S, t);
            const float mu = sum * a.inv_cols;
            qs = 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int k = chunk(c);
                float4 d = make_float4(v[c].x - mu, v[c].y - mu, v[c].z - mu, v[c].w - mu);
                if (k >= nv) d = splat4(0.0f);
                if (!AL) mask_chunk(d, k, h, cols, 0.0f);
                v[c] = d;
                qs += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
            }
            qs = row_reduce<AddOp, LW>(qs, red[1], S, t);
        } else if constexpr (!NARROW) {
            // S waves, one exchange: each wave centres its own elements on
            // its own mean m_w (rounded) and reduces the centred sum of
            // squares q_w and the centred sum c_w; the exchange brings every
            // wave's (m_w, q_w, c_w, n_w), and the pairwise update of Chan,
            // Golub and LeVeque merges them exactly, the rounding of m_w
            // included: sum (x - mu)^2 = sum_w q_w + d_w (2 c_w + n_w d_w),
            // d_w = m_w - mu, mu = sum_w (n_w m_w + c_w) / cols.  Against
            // the mean and the centred sum of squares exchanged one after
            // the other: one workgroup barrier less (LayerNorm 768 x 6144 at
            // six waves per row on MI355X: 6.78 -> 6.74 us).
            const float sw = wave_allreduce<AddOp>(sum);
            // aligned rows: a wave whose every slot lies inside the row (its
            // last chunk, t.s * 64 + 63 + W * (NCH - 1), below nv; a
            // wave-uniform test) holds exactly 256 NCH elements, which it
            // centres without the per-element selects that zero the slots
            // past the row; when that count is a power of two its mean is a
            // multiply, which equals the division bit for bit.  Same-box A/B
            // on MI355X for the selects: 768 x 6144 6.73 -> 6.71 us, 1024 x
            // 4096 6.57 -> 6.52, 512 x 12288 8.95 -> 8.87, 2048 x 8192 25.23 ->
            // 25.16.
            constexpr int kInside = kWave * kVec * NCH;
            const bool inside = AL && t.s * kWave + kWave - 1 + W * (NCH - 1) < nv;
            int nw;
            float mw, q = 0.0f, cw = 0.0f;
            if (inside) {
                nw = kInside;
                mw = (kInside & (kInside - 1)) == 0 ? sw * (1.0f / kInside) : sw / (float)kInside;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const float4 d = make_float4(v[c].x - mw, v[c].y - mw, v[c].z - mw, v[c].w - mw);
                    q += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
                    cw += (d.x + d.y) + (d.z + d.w);
                }
            } else {
                nw = active ? wave_elems(t.s, W, NCH, h, cols) : 0;
                mw = nw > 0 ? sw / (float)nw : 0.0f;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const int k = chunk(c);
                    float4 d = make_float4(v[c].x - mw, v[c].y - mw, v[c].z - mw, v[c].w - mw);
                    if (k >= nv) d = splat4(0.0f);
                    if (!AL) mask_chunk(d, k, h, cols, 0.0f);
                    q += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
                    cw += (d.x + d.y) + (d.z + d.w);
                }
            }
            wave_allreduce2<AddOp>(q, cw);
            float4* slot = reinterpret_cast<float4*>(&red[0][0]);
            if (t.lane == 0) slot[t.q * S + t.s] = make_float4(mw, q, cw, (float)nw);
            __syncthreads();
            const bool in = t.lane < S;
            const float4 e = in ? slot[t.q * S + t.lane] : splat4(0.0f);
            const float mu = team_merge<AddOp>(__builtin_fmaf(e.w, e.x, e.z)) * a.inv_cols;
            const float dw = e.x - mu;
            qs = team_merge<AddOp>(in ? e.y + dw * (2.0f * e.z + e.w * dw) : 0.0f);
#pragma unroll
            for (int c = 0; c < NCH; ++c) v[c] = make_float4(v[c].x - mu, v[c].y - mu, v[c].z - mu, v[c].w - mu);
        }
        const float r = fast_rsqrt(qs * a.inv_cols + a.eps);
        float* yr = a.y + row * (int64_t)cols;
        // aligned rows of teams of several waves: every gamma and beta chunk
        // is requested at once, every output formed, then the chunks stored
        // back to back, as RMSNorm does (768 x 6144 at six waves per row on
        // MI355X: 6.78 -> 6.73 us; 1024 x 4096 at two: 6.15 -> 5.76 us).  A
        // one-wave team keeps the load, wait and store per chunk: there the
        // burst cost 5.17 -> 7.06 us (4096 x 1024), and in the fused residual
        // LayerNorm, which keeps the loop too, 10.20 -> 12.25 us.
        bool burst = false;
        if constexpr (OP == kLayerNorm && AL && !NARROW) burst = S > 1;
        if (burst) {
            if constexpr (OP == kLayerNorm && AL && !NARROW) {
                float4 o[NCH];
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const float4 g = gamma_of(c, chunk(c));
                    const float4 b = beta_of(c, chunk(c));
                    o[c] = make_float4(v[c].x * r * g.x + b.x, v[c].y * r * g.y + b.y, v[c].z * r * g.z + b.z,
                                       v[c].w * r * g.w + b.w);
                }
                pin_chunks(o);
                const BufRes ry = make_res(yr, nv * 16);
#pragma unroll
                for (int c = 0; c < NCH; ++c) res_st4(ry, chunk(c) * 16, o[c]);
            }
        } else {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int k = chunk(c);
                if (k < nv) {
                    const float4 g = gamma_of(c, k);
                    const float4 b = beta_of(c, k);
                    const float4 o = make_float4(v[c].x * r * g.x + b.x, v[c].y * r * g.y + b.y,
                                                 v[c].z * r * g.z + b.z, v[c].w * r * g.w + b.w);
                    store_chunk<AL>(yr, a.y_same_phase, k, h, cols, o);
                }
            }
        }
    }
}

template <int OP, int NCH, bool AL, int PM>
__global__ void __launch_bounds__(cache_max_threads(NCH))
k_cache(LR_ENTRY_PARAMS) {
    // two exchanges of one float per wave, or one of four (LayerNorm)
    __shared__ __attribute__((aligned(16))) float red[4][kMaxWaves];
    cache_body<OP, NCH, AL, PM, kWave>(LR_ENTRY_KARGS, red);
}

// Sub-wave teams: LW lanes per row, 64 / LW rows per wave, S = 1.
template <int OP, int NCH, bool AL, int PM, int LW>
__global__ void __launch_bounds__(1024)
k_cache_narrow(LR_ENTRY_PARAMS) {
    __shared__ float red[4][kMaxWaves];  // untouched: no cross-wave exchange
    cache_body<OP, NCH, AL, PM, LW>(LR_ENTRY_KARGS, red);
}

// ===========================================================================
// STREAM family: the row is walked in trips of U chunks per worker; passes
// that need it again reload it.  Softmax and cross-entropy fold (max,
// sum of exp) online in one pass (Milakov and Gimelshein's online normaliser)
// and merge the per-worker pairs at the end.
// ===========================================================================
template <int OP, bool AL>
__device__ __forceinline__ void load_trip(float4 (&v)[kStreamUnroll], const float4* xa, BufRes rr, int k0,
                                          int W, int nv, int h, int cols, float id) {
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
        const int k = k0 + W * u;
        v[u] = (k < nv) ? ld4(xa + k) : splat4(id);
        if constexpr (OP == kAddLayerNorm) {  // + residual (FP32); id is 0
            const float4 q = AL ? res_ld4<LR_NT_LOADS ? kAuxNt : kAuxDefault>(rr, k * 16) : elem_chunk(rr, k, h, cols);
            if (k < nv) v[u] = make_float4(v[u].x + q.x, v[u].y + q.y, v[u].z + q.z, v[u].w + q.w);
        }
        if (!AL) mask_chunk(v[u], k, h, cols, id);
    }
}

template <int OP, bool AL>
__global__ void __launch_bounds__(1024) k_stream(LR_ENTRY_PARAMS) {
    const KArgs a = LR_ENTRY_KARGS;
    __shared__ float red[2][kMaxWaves];
    constexpr int U = kStreamUnroll;
    constexpr float ID = op_identity<OP>();
    const int S = a.S;
    const int W = kWave * S;
    const Team t = team_of_wave(wave_id(), (int)threadIdx.x & (kWave - 1), S, a.team_magic);
    const int64_t row = row_of(blockIdx.x, a.Q, t.q);
    const bool active = row < a.rows;
    const int cols = a.cols;
    const float* xr = a.x + (active ? row : 0) * (int64_t)cols;
    const int h = AL ? 0 : phase_of(reinterpret_cast<uintptr_t>(xr));
    const int nv = active ? (AL ? cols / kVec : chunks_of(h, cols)) : 0;
    const float4* xa = reinterpret_cast<const float4*>(xr - h);
    float* yr = a.y + (active ? row : 0) * (int64_t)cols;
    const int64_t roff = (active ? row : 0) * (int64_t)cols;
    const BufRes rr = make_res(OP == kAddLayerNorm ? a.residual + roff : nullptr,
                               OP == kAddLayerNorm && active ? (AL ? nv * 16 : cols * 4) : 0);

    float sel = 0.0f;
    if constexpr (OP == kCrossEntropy) {
        if (active && t.w == 0) sel = gather_label(a, xr, row);
    }

    if constexpr (OP == kSoftmax || OP == kCrossEntropy) {
        float m = -INFINITY, s = 0.0f;
        for (int k0 = t.w; k0 < nv; k0 += W * U) {
            float4 v[U];
            load_trip<OP, AL>(v, xa, rr, k0, W, nv, h, cols, ID);
            float tm = m;
#pragma unroll
            for (int u = 0; u < U; ++u)
                tm = fmax2(fmax2(tm, fmax2(v[u].x, v[u].y)), fmax2(v[u].z, v[u].w));
            // while every element so far is -inf (masked), shift by 0: the
            // exponentials are then exp(-inf) = 0 and s stays 0
            const float mm = (tm == -INFINITY) ? 0.0f : tm;
            s *= fast_exp(m - mm);  // m = -inf until a finite element: s is 0 anyway
            m = tm;
#pragma unroll
            for (int u = 0; u < U; ++u)
                s += (fast_exp(v[u].x - mm) + fast_exp(v[u].y - mm)) +
                     (fast_exp(v[u].z - mm) + fast_exp(v[u].w - mm));
        }
        const float M = team_reduce<MaxOp>(m, red[0], S, t);
        // a worker with no elements has m = -inf and s = 0
        const float sc = (m == -INFINITY) ? 0.0f : s * fast_exp(m - M);
        const float tot = team_reduce<AddOp>(sc, red[1], S, t);
        if constexpr (OP == kCrossEntropy) {
            if (active && t.w == 0) a.losses[row] = fast_log(tot) + (M - sel);
        } else {
            const float r = fast_rcp(tot);
            for (int k0 = t.w; k0 < nv; k0 += W * U) {
                float4 v[U];
                load_trip<OP, AL>(v, xa, rr, k0, W, nv, h, cols, ID);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int k = k0 + W * u;
                    if (k < nv) {
                        const float4 o = make_float4(fast_exp(v[u].x - M) * r, fast_exp(v[u].y - M) * r,
                                                     fast_exp(v[u].z - M) * r, fast_exp(v[u].w - M) * r);
                        store_chunk<AL>(yr, a.y_same_phase, k, h, cols, o);
                    }
                }
            }
        }
    } else if constexpr (OP == kRowSum) {
        float sum = 0.0f;
        for (int k0 = t.w; k0 < nv; k0 += W * U) {
            float4 v[U];
            load_trip<OP, AL>(v, xa, rr, k0, W, nv, h, cols, ID);
#pragma unroll
            for (int u = 0; u < U; ++u) sum += (v[u].x + v[u].y) + (v[u].z + v[u].w);
        }
        sum = team_reduce<AddOp>(sum, red[0], S, t);
        if (active && t.w == 0) a.sums[row] = sum;
    } else if constexpr (OP == kRowMinMax) {
        float lo = ID, hi = ID;
        for (int k0 = t.w; k0 < nv; k0 += W * U) {
            float4 v[U];
            load_trip<OP, AL>(v, xa, rr, k0, W, nv, h, cols, ID);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                lo = fminnum(fminnum(lo, fminnum(v[u].x, v[u].y)), fminnum(v[u].z, v[u].w));
                hi = fmaxnum(fmaxnum(hi, fmaxnum(v[u].x, v[u].y)), fmaxnum(v[u].z, v[u].w));
            }
        }
        finish_minmax(a, lo, hi, red[0], red[1], S, t, active, row);
    } else if constexpr (OP == kRmsNorm) {
        float ss = 0.0f;
        for (int k0 = t.w; k0 < nv; k0 += W * U) {
            float4 v[U];
            load_trip<OP, AL>(v, xa, rr, k0, W, nv, h, cols, ID);
#pragma unroll
            for (int u = 0; u < U; ++u)
                ss += (v[u].x * v[u].x + v[u].y * v[u].y) + (v[u].z * v[u].z + v[u].w * v[u].w);
        }
        ss = team_reduce<AddOp>(ss, red[0], S, t);
        const float r = fast_rsqrt(ss * a.inv_cols + a.eps);
        for (int k0 = t.w; k0 < nv; k0 += W * U) {
            float4 v[U];
            load_trip<OP, AL>(v, xa, rr, k0, W, nv, h, cols, ID);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + W * u;
                if (k < nv) {
                    const float4 g = param_chunk<AL>(a.gamma, k, h, cols, 1.0f);
                    const float4 o = make_float4(v[u].x * r * g.x, v[u].y * r * g.y,
                                                 v[u].z * r * g.z, v[u].w * r * g.w);
                    store_chunk<AL>(yr, a.y_same_phase, k, h, cols, o);
                }
            }
        }
    } else {  // LayerNorm, fused residual LayerNorm
        float sum = 0.0f;
        for (int k0 = t.w; k0 < nv; k0 += W * U) {
            float4 v[U];
            load_trip<OP, AL>(v, xa, rr, k0, W, nv, h, cols, ID);
#pragma unroll
            for (int u = 0; u < U; ++u) sum += (v[u].x + v[u].y) + (v[u].z + v[u].w);
        }
        sum = team_reduce<AddOp>(sum, red[0], S, t);
        const float mu = sum * a.inv_cols;
        float qs = 0.0f;
        for (int k0 = t.w; k0 < nv; k0 += W * U) {
            float4 v[U];
            load_trip<OP, AL>(v, xa, rr, k0, W, nv, h, cols, ID);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + W * u;
                float4 d = make_float4(v[u].x - mu, v[u].y - mu, v[u].z - mu, v[u].w - mu);
                if (k >= nv) d = splat4(0.0f);
                if (!AL) mask_chunk(d, k, h, cols, 0.0f);
                qs += (d.x * d.x + d.y * d.y) + (d.z * d.z + d.w * d.w);
            }
        }
        qs = team_reduce<AddOp>(qs, red[1], S, t);
        const float r = fast_rsqrt(qs * a.inv_cols + a.eps);
        for (int k0 = t.w; k0 < nv; k0 += W * U) {
            float4 v[U];
            load_trip<OP, AL>(v, xa, rr, k0, W, nv, h, cols, ID);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = k0 + W * u;
                if (k < nv) {
                    const float4 g = param_chunk<AL>(a.gamma, k, h, cols, 1.0f);
                    const float4 b = param_chunk<AL>(a.beta, k, h, cols, 0.0f);
                    const float4 o = make_float4((v[u].x - mu) * r * g.x + b.x, (v[u].y - mu) * r * g.y + b.y,
                                                 (v[u].z - mu) * r * g.z + b.z, (v[u].w - mu) * r * g.w + b.w);
                    store_chunk<AL>(yr, a.y_same_phase, k, h, cols, o);
                    // the sum is written in this last pass only, so an output
                    // that is x or the residual itself is not read after it
                    if (OP == kAddLayerNorm && a.sum_out != nullptr)
                        store_chunk<AL>(a.sum_out + roff, a.s_same_phase, k, h, cols, v[u]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launch by plan: selects the compiled instance and launches it on `s`.
// ---------------------------------------------------------------------------
template <int OP, int NCH, bool AL, int PM>
hipError_t launch_cache_inst(const KArgs& a, const lr_plan& p, hipStream_t s) {
    hipLaunchKernelGGL((k_cache<OP, NCH, AL, PM>), dim3((unsigned)p.blocks), dim3(p.threads_per_block), 0, s,
                       LR_ENTRY_ARGS(a));
    return hipGetLastError();
}

template <int OP, int NCH, bool AL, int PM, int LW>
hipError_t launch_narrow_inst(const KArgs& a, const lr_plan& p, hipStream_t s) {
    hipLaunchKernelGGL((k_cache_narrow<OP, NCH, AL, PM, LW>), dim3((unsigned)p.blocks), dim3(p.threads_per_block), 0,
                       s, LR_ENTRY_ARGS(a));
    return hipGetLastError();
}

template <int OP, bool AL, int PM, int LW>
hipError_t launch_narrow_nch(const KArgs& a, const lr_plan& p, hipStream_t s) {
    switch (p.chunks_per_lane) {
        case 1: return launch_narrow_inst<OP, 1, AL, PM, LW>(a, p, s);
        case 2: return launch_narrow_inst<OP, 2, AL, PM, LW>(a, p, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP, bool AL, int PM>
hipError_t launch_cache_nch(const KArgs& a, const lr_plan& p, hipStream_t s) {
    switch (p.lanes_per_row) {
        case 4: return launch_narrow_nch<OP, AL, PM, 4>(a, p, s);
        case 8: return launch_narrow_nch<OP, AL, PM, 8>(a, p, s);
        case 16: return launch_narrow_nch<OP, AL, PM, 16>(a, p, s);
        case 32: return launch_narrow_nch<OP, AL, PM, 32>(a, p, s);
        default: break;  // whole-wave teams
    }
    switch (p.chunks_per_lane) {
        case 1: return launch_cache_inst<OP, 1, AL, PM>(a, p, s);
        case 2: return launch_cache_inst<OP, 2, AL, PM>(a, p, s);
        case 3: return launch_cache_inst<OP, 3, AL, PM>(a, p, s);
        case 4: return launch_cache_inst<OP, 4, AL, PM>(a, p, s);
        case 6: return launch_cache_inst<OP, 6, AL, PM>(a, p, s);
        case 8: return launch_cache_inst<OP, 8, AL, PM>(a, p, s);
        case 12: return launch_cache_inst<OP, 12, AL, PM>(a, p, s);
        case 16: return launch_cache_inst<OP, 16, AL, PM>(a, p, s);
        case 24: return launch_cache_inst<OP, 24, AL, PM>(a, p, s);
        case 32: return launch_cache_inst<OP, 32, AL, PM>(a, p, s);
        default: return hipErrorInvalidValue;
    }
}

// Selects the parameter mode from which parameters are present.
template <int OP, bool AL>
hipError_t launch_cache_pm(const KArgs& a, const lr_plan& p, hipStream_t s) {
    if constexpr (num_params<OP>() == 0) {
        return launch_cache_nch<OP, AL, kParNone>(a, p, s);
    } else {
        const bool all = a.gamma != nullptr && (OP == kRmsNorm || a.beta != nullptr);
        const bool none = a.gamma == nullptr && (OP == kRmsNorm || a.beta == nullptr);
        if (all) return launch_cache_nch<OP, AL, kParAll>(a, p, s);
        if (none) return launch_cache_nch<OP, AL, kParNone>(a, p, s);
        return launch_cache_nch<OP, AL, kParRuntime>(a, p, s);
    }
}

template <int OP>
hipError_t launch_op(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    if (p.family == LR_FAMILY_CACHE) {
        return aligned ? launch_cache_pm<OP, true>(a, p, s) : launch_cache_pm<OP, false>(a, p, s);
    }
    if (p.family == LR_FAMILY_STREAM) {
        if (aligned)
            hipLaunchKernelGGL((k_stream<OP, true>), dim3((unsigned)p.blocks), dim3(p.threads_per_block), 0, s,
                               LR_ENTRY_ARGS(a));
        else
            hipLaunchKernelGGL((k_stream<OP, false>), dim3((unsigned)p.blocks), dim3(p.threads_per_block), 0, s,
                               LR_ENTRY_ARGS(a));
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

}  // namespace lr
