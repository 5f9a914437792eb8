// ordered_tree (TREE family) kernels of one operation (lr_tree.hpp), built
// without contraction and with IEEE division and square root.
#pragma clang fp contract(off)

#include "lr_tree.hpp"

namespace lr {

hipError_t launch_tree_layernorm(const KArgs& a, const lr_plan& p, bool aligned, hipStream_t s) {
    return launch_tree_op<kLayerNorm>(a, p, aligned, s);
}

}  // namespace lr
