// Unordered-policy kernels of the row minimum and maximum: every CACHE chunk count, the
// STREAM family and the SPLIT family, each for aligned and misaligned rows
// (lr_kernels.hpp, lr_split.hpp).
#include "lr_split.hpp"

namespace lr {

hipError_t launch_row_minmax(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    return launch_unordered<kRowMinMax>(a, p, aligned, s);
}

}  // namespace lr
