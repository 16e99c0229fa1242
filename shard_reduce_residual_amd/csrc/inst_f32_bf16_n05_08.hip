// Instantiations of the fused kernel for partials PartF32, activations ActBF16, N = 5..8.
#include "arfuse_table.hpp"

namespace arf {
launch_fn lookup_f32_bf16_n05_08(int n, bool rpw, int waves, int c) {
    return pick_shards<PartF32, ActBF16, 5, 8>(n, rpw, waves, c);
}
}  // namespace arf
