// Unordered-policy kernels of the fused residual LayerNorm: every CACHE chunk
// count and the STREAM family, each for aligned and misaligned rows
// (lr_kernels.hpp).
#include "lr_split.hpp"

namespace lr {

hipError_t launch_add_layernorm(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    return launch_unordered<kAddLayerNorm>(a, p, aligned, s);
}

}  // namespace lr
