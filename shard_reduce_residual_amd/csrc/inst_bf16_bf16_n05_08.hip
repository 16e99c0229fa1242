// Instantiations of the fused and held-row kernels for partials ActBF16, activations ActBF16, N = 5..8.
#include "arfuse_table.hpp"

namespace arf {
launch_fn lookup_bf16_bf16_n05_08(int n, bool rpw, int waves, int c) {
    return pick_shards<ActBF16, ActBF16, 5, 8>(n, rpw, waves, c);
}
held_launch_fn held_bf16_bf16_n05_08(int n, int c, bool quant, int waves) {
    return pick_held_shards<ActBF16, ActBF16, 5, 8>(n, c, quant, waves);
}
}  // namespace arf
