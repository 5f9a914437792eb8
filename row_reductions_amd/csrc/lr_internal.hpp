// Internal interface between the C-ABI layer (lr_abi.cpp), the planner
// (lr_planner.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "lr.h"

namespace lr {

// Kernel arguments (passed by value).  Unused pointers are null.
struct KArgs {
    const float* x;         // input rows (logits for cross-entropy)
    float* y;               // output rows (softmax, norms)
    const float* gamma;     // per-column scale or null
    const float* beta;      // per-column shift or null
    const int64_t* labels;  // cross-entropy labels
    float* losses;          // cross-entropy per-row loss
    int64_t rows;
    int32_t cols;
    float eps;
    float inv_cols;         // 1/cols rounded to FP32 (unordered policy only)
    int32_t S;              // waves per row
    int32_t Q;              // rows per workgroup
    int32_t y_same_phase;   // y rows start at the same 16-byte phase as x rows
    int32_t team_magic;     // team_magic(S): wave index / S as a multiply
    const float* residual;  // fused residual LayerNorm: second input, else null
    float* sum_out;         // fused residual LayerNorm: x + residual out, or null
    int32_t r_same_phase;   // residual rows start at the same 16-byte phase as x rows
    int32_t s_same_phase;   // sum_out rows start at the same 16-byte phase as x rows
    float* sums;            // row sum: one float per row
    float* mins;            // row minimum (or null)
    float* maxs;            // row maximum (or null)
    int32_t splits;         // split family: segments per row (G), else 0
    float* ws;              // split family: 2 floats per segment, rows*G*2 floats
};

// Compiled cache-family chunk counts (chunks_per_lane), ascending.
constexpr int kCacheChunks[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32};
constexpr int kNumCacheChunks = sizeof(kCacheChunks) / sizeof(kCacheChunks[0]);
constexpr int kStreamUnroll = 4;
// Chunk counts (whole rows) of the one-lane-per-row ORDERED instances, ascending.
constexpr int kLaneChunks[] = {1, 2, 4, 8, 16};
constexpr int kNumLaneChunks = sizeof(kLaneChunks) / sizeof(kLaneChunks[0]);
// Chunk counts of the sub-wave CACHE instances (lanes_per_row 4 .. 32), ascending.
constexpr int kNarrowChunks[] = {1, 2};
constexpr int kNumNarrowChunks = sizeof(kNarrowChunks) / sizeof(kNarrowChunks[0]);
// Split-family chunk counts (the stripe of one segment), ascending.
constexpr int kSplitChunks[] = {1, 2, 3, 4, 6, 8};
constexpr int kNumSplitChunks = sizeof(kSplitChunks) / sizeof(kSplitChunks[0]);

// Largest workgroup a cache instance is compiled for (launch bounds); the
// register stripe grows with the chunk count, so the bound shrinks.
constexpr int cache_max_threads(int nch) { return nch <= 8 ? 1024 : (nch <= 16 ? 512 : 256); }

bool cache_chunks_compiled(int nch);

// Workspace bytes a plan needs for `rows` rows (0 unless it splits rows).
int64_t plan_workspace_bytes(const lr_plan& p, int64_t rows);

// Work-items one kernel dispatch may carry.  The dispatch packet holds a
// 32-bit grid size; staying at 2^31 also keeps blockIdx * blockDim inside a
// signed 32-bit int.
constexpr int64_t kMaxDispatchItems = int64_t(1) << 31;

// Rows one dispatch of plan `p` covers for a call over `rows` rows (at least
// 1, at most `rows`); a multiple of rows_per_block whenever it is below rows.
int64_t dispatch_rows(const lr_plan& p, int64_t rows);

// `p` resized to a piece of n rows (its grid: ceil(n / Q) workgroups, or
// n * splits for the split family).
lr_plan piece_plan(const lr_plan& p, int64_t n);

// Per-op launchers (one translation unit per op; CACHE, STREAM and SPLIT).  `aligned` selects the
// instance for 16-byte aligned rows and parameter vectors.
hipError_t launch_softmax(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_rmsnorm(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_layernorm(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_cross_entropy(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_add_layernorm(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_row_sum(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_row_minmax(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
// Row copy through the CACHE family's load/store path (k_copy_rows.hip).
hipError_t launch_copy_rows(const float* x, float* y, int64_t rows, int cols, const lr_plan& p, bool sync,
                            hipStream_t s);
hipError_t launch_ordered(int op, int policy, const KArgs& a, const lr_plan& p, hipStream_t s);
// The ordered policies with one lane per row (lanes_per_row = 1: narrow
// rows, one wavefront of 64 rows per workgroup).
hipError_t launch_ordered_lane(int op, int policy, const KArgs& a, const lr_plan& p, hipStream_t s);
// TREE family (ordered_tree on the cache layout), one translation unit per op.
hipError_t launch_tree_softmax(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_tree_cross_entropy(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_tree_rmsnorm(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_tree_layernorm(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_tree_add_layernorm(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_tree_row_sum(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);
hipError_t launch_tree_row_minmax(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s);

// The current device's address of lr_run_f32_noalloc's device array
// (lr_noalloc.hip), looked up on the first call on that device.
lr_status noalloc_scratch(void** out);

// Longest row the TREE family takes (128 slabs of 256 floats).
constexpr int kTreeMaxCols = 128 * 256;

}  // namespace lr
