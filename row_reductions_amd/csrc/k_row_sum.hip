// Unordered-policy kernels of the row sum: every CACHE chunk count and the
// STREAM family, each for aligned and misaligned rows (lr_kernels.hpp).
#include "lr_kernels.hpp"

namespace lr {

hipError_t launch_row_sum(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    return launch_op<kRowSum>(a, p, aligned, s);
}

}  // namespace lr
