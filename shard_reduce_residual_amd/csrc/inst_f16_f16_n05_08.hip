// Instantiations of the fused and held-row kernels for partials ActF16, activations ActF16, N = 5..8.
#include "arfuse_table.hpp"

namespace arf {
launch_fn lookup_f16_f16_n05_08(int n, bool rpw, int waves, int c) {
    return pick_shards<ActF16, ActF16, 5, 8>(n, rpw, waves, c);
}
held_launch_fn held_f16_f16_n05_08(int n, int c, bool quant, int waves) {
    return pick_held_shards<ActF16, ActF16, 5, 8>(n, c, quant, waves);
}
}  // namespace arf
