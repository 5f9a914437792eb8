// Unordered-policy kernels of one operation: every CACHE chunk count, the
// STREAM family and the SPLIT family, each for aligned and misaligned rows
// (lr_kernels.hpp, lr_split.hpp).
#include "lr_split.hpp"

namespace lr {

hipError_t launch_cross_entropy(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    return launch_unordered<kCrossEntropy>(a, p, aligned, s);
}

}  // namespace lr
