// Instantiations of the fused kernel for partials of type ActBF16 and activations of type ActBF16.
#include "arfuse_table.hpp"

namespace arf {
launch_fn lookup_bf16_bf16(int nmax, bool row_per_wave, int waves, int c) {
    return pick_launcher<ActBF16, ActBF16>(nmax, row_per_wave, waves, c);
}
}  // namespace arf
