// Unordered-policy kernels of the row minimum and maximum: every CACHE chunk count and the
// STREAM family, each for aligned and misaligned rows (lr_kernels.hpp).
#include "lr_kernels.hpp"

namespace lr {

hipError_t launch_row_minmax(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    return launch_op<kRowMinMax>(a, p, aligned, s);
}

}  // namespace lr
