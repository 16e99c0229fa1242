// Instantiations of the fused and held-row kernels for partials PartF32, activations ActBF16, N = 9..12.
#include "arfuse_table.hpp"

namespace arf {
launch_fn lookup_f32_bf16_n09_12(int n, bool rpw, int waves, int c) {
    return pick_shards<PartF32, ActBF16, 9, 12>(n, rpw, waves, c);
}
held_launch_fn held_f32_bf16_n09_12(int n, int c, bool quant, int waves) {
    return pick_held_shards<PartF32, ActBF16, 9, 12>(n, c, quant, waves);
}
}  // namespace arf
