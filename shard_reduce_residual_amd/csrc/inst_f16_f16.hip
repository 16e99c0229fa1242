// Instantiations of the fused kernel for partials of type ActF16 and activations of type ActF16.
#include "arfuse_table.hpp"

namespace arf {
launch_fn lookup_f16_f16(int nmax, bool row_per_wave, int waves, int c) {
    return pick_launcher<ActF16, ActF16>(nmax, row_per_wave, waves, c);
}
}  // namespace arf
