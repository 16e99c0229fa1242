// Instantiations of the fused kernel for partials of type PartF32 and activations of type ActBF16.
#include "arfuse_table.hpp"

namespace arf {
launch_fn lookup_f32_bf16(int nmax, bool row_per_wave, int waves, int c) {
    return pick_launcher<PartF32, ActBF16>(nmax, row_per_wave, waves, c);
}
}  // namespace arf
