// Unordered-policy kernels of the row sum: every CACHE chunk count, the
// STREAM family and the SPLIT family, each for aligned and misaligned rows
// (lr_kernels.hpp, lr_split.hpp).
#include "lr_split.hpp"

namespace lr {

hipError_t launch_row_sum(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    return launch_unordered<kRowSum>(a, p, aligned, s);
}

}  // namespace lr
