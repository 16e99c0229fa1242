// Instantiations of the fused kernel for partials of type PartF32 and activations of type ActF16.
#include "arfuse_table.hpp"

namespace arf {
launch_fn lookup_f32_f16(int nmax, bool row_per_wave, int waves, int c) {
    return pick_launcher<PartF32, ActF16>(nmax, row_per_wave, waves, c);
}
}  // namespace arf
