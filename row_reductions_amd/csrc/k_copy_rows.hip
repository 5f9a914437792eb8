// Row copy through the CACHE family's data path: the floor under a whole
// reduction launch's time.  One workgroup per row, lane w of the S-wave team
// reading chunks w, w + W, .. (W = 64 S) with the same 16-byte buffer reads
// and writing them back with the same streamed stores, with no arithmetic
// and no parameter read between the two.  SYNC: every wave waits for its
// reads and the workgroup meets at one barrier before the first store, as
// the reductions' cross-wave exchange makes them do; without it each wave
// stores as soon as its own reads land.  Its four arguments arrive
// preloaded in scalar registers, as the operations' leading arguments do.
#include "lr_device.hpp"
#include "lr_internal.hpp"

namespace lr {
namespace {

template <int NCH, bool SYNC>
__global__ void __launch_bounds__(1024) k_copy_rows(const float* x, float* y, int cols, int S) {
    const int W = kWave * S;
    const int w = (int)threadIdx.x;  // one row per workgroup: the worker is the thread
    const int64_t off = (int64_t)blockIdx.x * cols;
    const int nv = cols / kVec;
    const BufRes rx = make_res(x + off, nv * 16);
    const BufRes ry = make_res(y + off, nv * 16);
    constexpr int AUX = LR_NT_LOADS ? kAuxNt : kAuxDefault;
    float4 v[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) v[c] = res_ld4<AUX>(rx, chunk_index(w, W, c) * 16);
    if constexpr (SYNC) {
        __builtin_amdgcn_s_waitcnt(0);  // every counter at zero: the wave's reads have landed
        __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) res_st4(ry, chunk_index(w, W, c) * 16, v[c]);
}

template <int NCH>
hipError_t go(const float* x, float* y, int64_t rows, int cols, int S, bool sync, hipStream_t s) {
    if (sync) {
        hipLaunchKernelGGL((k_copy_rows<NCH, true>), dim3((unsigned)rows), dim3(kWave * S), 0, s, x, y, cols, S);
    } else {
        hipLaunchKernelGGL((k_copy_rows<NCH, false>), dim3((unsigned)rows), dim3(kWave * S), 0, s, x, y, cols, S);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_copy_rows(const float* x, float* y, int64_t rows, int cols, const lr_plan& p, bool sync,
                            hipStream_t s) {
    const int S = p.waves_per_row;
    switch (p.chunks_per_lane) {
        case 1: return go<1>(x, y, rows, cols, S, sync, s);
        case 2: return go<2>(x, y, rows, cols, S, sync, s);
        case 3: return go<3>(x, y, rows, cols, S, sync, s);
        case 4: return go<4>(x, y, rows, cols, S, sync, s);
        case 6: return go<6>(x, y, rows, cols, S, sync, s);
        case 8: return go<8>(x, y, rows, cols, S, sync, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lr
