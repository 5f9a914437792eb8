// Thread -> (row, element) mapping shared by the kernels and the host
// coverage replay (lr_coverage_check), so that the replay checks the very
// functions the kernels are built from.
//
// Mapping algebra of "TIRx Metal reduction lowering", section 4, re-derived
// for 64-lane wavefronts:  W = 64*S workers cooperate on one row, a
// workgroup packs Q rows (64*S*Q threads), worker w owns the 16-byte chunks
// k = w + W*c (blocked-cyclic ownership with V = 4, section 4.4), and a chunk
// covers the four consecutive floats 4k .. 4k+3 of the row's 16-byte aligned
// grid.  A row that does not start on a 16-byte boundary sits `phase`
// floats into its first chunk; grid slots outside [0, cols) are not
// elements of the row and take the reduction identity.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define LR_HD __host__ __device__ __forceinline__
#else
#define LR_HD inline
#endif

namespace lr {

constexpr int kWave = 64;       // lanes per wavefront (gfx950)
constexpr int kVec = 4;         // floats per 128-bit chunk
constexpr int kMaxWaves = 16;   // 1024 threads per workgroup
constexpr int kSlab = 256;      // ordered family: floats folded per LDS slab
constexpr int kTreeStack = 32;  // ordered family, tree policy: subtrees kept per wave (2^32 slabs)
constexpr int kMaxSplits = 64;  // split family: segments per row (one wave lane per partial)

// Ordered reduction policies (the lr_reduction_policy codes).
enum Policy : int { kPolUnordered = 0, kPolFoldLeft = 1, kPolTree = 2, kPolFoldRight = 3 };

struct Team {
    int q;     // packed row within the workgroup
    int w;     // worker within the row team, 0 .. 64*S-1
    int s;     // wavefront within the row team
    int lane;  // lane within the wavefront
};

// Multiplier that turns the division of a wave index by S into a multiply
// and a shift: floor(i / S) == (i * team_magic(S)) >> 16 for 0 <= i < 16 and
// 1 <= S <= 16 (ceil(2^16/S) exceeds 2^16/S by less than 1, and i times that
// excess stays below 2^16/S, so the quotient never reaches the next integer).
LR_HD int team_magic(int S) { return (65536 + S - 1) / S; }

// Team of lane `lane` of wave `wave` of a workgroup whose row teams are S
// waves wide.  Every field but `w` and `lane` is uniform over the wave.
LR_HD Team team_of_wave(int wave, int lane, int S, int magic) {
    const int q = (wave * magic) >> 16;
    const int s = wave - q * S;
    return Team{q, s * kWave + lane, s, lane};
}

LR_HD Team team_of(int tid, int S) { return team_of_wave(tid / kWave, tid % kWave, S, team_magic(S)); }

// Sub-wave teams of L = 4, 8, 16 or 32 lanes (CACHE family, narrow rows):
// lane group lane / L of wave `wave` serves packed row wave * (64 / L) +
// lane / L, as worker lane % L.
constexpr int kNarrowLanes[] = {4, 8, 16, 32};

LR_HD bool narrow_lanes(int L) { return L == 4 || L == 8 || L == 16 || L == 32; }

LR_HD Team team_of_group(int wave, int lane, int L) { return Team{wave * (kWave / L) + lane / L, lane % L, 0, lane}; }

LR_HD int64_t row_of(int64_t block, int Q, int q) { return block * Q + q; }

// Floats between the 16-byte boundary at or below `addr` and `addr`.
LR_HD int phase_of(uintptr_t addr) { return (int)((addr & 15u) >> 2); }

// 16-byte chunks of the aligned grid that touch a row of `cols` floats.
LR_HD int chunks_of(int phase, int cols) { return (phase + cols + kVec - 1) / kVec; }

// Chunk owned by worker w at stripe slot c.
LR_HD int chunk_index(int w, int W, int c) { return w + W * c; }

// Row element held in float j of chunk k (may fall outside [0, cols)).
LR_HD int elem_index(int k, int j, int phase) { return kVec * k + j - phase; }

LR_HD bool elem_valid(int e, int cols) { return (unsigned)e < (unsigned)cols; }

// Chunk k holds four row elements (no guard needed for it).
LR_HD bool chunk_full(int k, int phase, int cols) {
    return kVec * k - phase >= 0 && kVec * k + kVec - phase <= cols;
}

// Elements of a row (phase, cols) held by wavefront s of a whole-wave team
// of W = 64 S workers with nch chunks each: its stripe slot c covers grid
// positions 4 b .. 4 b + 255, b = 64 s + W c, and the row occupies grid
// positions phase .. phase + cols - 1.
LR_HD int wave_elems(int s, int W, int nch, int phase, int cols) {
    int n = 0;
    for (int c = 0; c < nch; ++c) {
        const int p = kVec * (s * kWave + W * c);
        const int lo = p > phase ? p : phase;
        const int hi = p + kVec * kWave < phase + cols ? p + kVec * kWave : phase + cols;
        n += hi > lo ? hi - lo : 0;
    }
    return n;
}

// Split family: a row's nv chunks are cut into G segments of L = ceil(nv/G)
// chunks; segment g holds chunks [k0, k1) (the last ones may be short or
// empty).  Worker w of the segment's workgroup owns chunks k0 + w + W*c.
struct SegmentBounds {
    int k0, k1;
};

LR_HD SegmentBounds segment_bounds(int nv, int G, int g) {
    const int L = (nv + G - 1) / G;
    const int k0 = g * L < nv ? g * L : nv;
    const int k1 = k0 + L < nv ? k0 + L : nv;
    return SegmentBounds{k0, k1};
}

// Ordered family: one wavefront per row; lane l loads element
// kSlab*slab + 64*i + l, i = 0..3, into slot 64*i + l of its LDS slab.
LR_HD int ordered_elem(int slab, int i, int lane) { return kSlab * slab + kWave * i + lane; }

}  // namespace lr
