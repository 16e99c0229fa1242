// Instantiations of the fused kernel for partials PartF32, activations ActBF16, N = 1..4.
#include "arfuse_table.hpp"

namespace arf {
launch_fn lookup_f32_bf16_n01_04(int n, bool rpw, int waves, int c) {
    return pick_shards<PartF32, ActBF16, 1, 4>(n, rpw, waves, c);
}
}  // namespace arf
