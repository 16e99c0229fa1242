// arfuse_table.hpp -- the instantiated launch geometries of the fused kernel, and the
// lookup from (shard bound, path, wavefronts per workgroup, chunks per lane) to a
// launcher. One translation unit per (partial type, activation type) includes this.
//
// Menu: shard bound NMAX in {1, 2, 4, 8, 16}; one row per wavefront with 4 wavefronts
// per workgroup and C in {1, 2, 4, 8}; one row per workgroup with WAVES in {2, 4, 8, 16}
// and C in {1, 2, 4, 8}.
#pragma once

#include "arfuse_device.hpp"

namespace arf {

template <class PT, class AT, int NM, int W>
launch_fn pick_block_c(int c) {
    switch (c) {
        case 1: return &launch_fused<PT, AT, NM, 1, W, false>;
        case 2: return &launch_fused<PT, AT, NM, 2, W, false>;
        case 4: return &launch_fused<PT, AT, NM, 4, W, false>;
        case 8: return &launch_fused<PT, AT, NM, 8, W, false>;
        default: return nullptr;
    }
}

template <class PT, class AT, int NM>
launch_fn pick_geometry(bool row_per_wave, int waves, int c) {
    if (row_per_wave) {
        if (waves != 4) return nullptr;
        switch (c) {
            case 1: return &launch_fused<PT, AT, NM, 1, 4, true>;
            case 2: return &launch_fused<PT, AT, NM, 2, 4, true>;
            case 4: return &launch_fused<PT, AT, NM, 4, 4, true>;
            case 8: return &launch_fused<PT, AT, NM, 8, 4, true>;
            default: return nullptr;
        }
    }
    switch (waves) {
        case 2: return pick_block_c<PT, AT, NM, 2>(c);
        case 4: return pick_block_c<PT, AT, NM, 4>(c);
        case 8: return pick_block_c<PT, AT, NM, 8>(c);
        case 16: return pick_block_c<PT, AT, NM, 16>(c);
        default: return nullptr;
    }
}

template <class PT, class AT>
launch_fn pick_launcher(int nmax, bool row_per_wave, int waves, int c) {
    switch (nmax) {
        case 1: return pick_geometry<PT, AT, 1>(row_per_wave, waves, c);
        case 2: return pick_geometry<PT, AT, 2>(row_per_wave, waves, c);
        case 4: return pick_geometry<PT, AT, 4>(row_per_wave, waves, c);
        case 8: return pick_geometry<PT, AT, 8>(row_per_wave, waves, c);
        case 16: return pick_geometry<PT, AT, 16>(row_per_wave, waves, c);
        default: return nullptr;
    }
}

// Defined in the per-type translation units.
launch_fn lookup_bf16_bf16(int nmax, bool row_per_wave, int waves, int c);
launch_fn lookup_f16_f16(int nmax, bool row_per_wave, int waves, int c);
launch_fn lookup_f32_bf16(int nmax, bool row_per_wave, int waves, int c);
launch_fn lookup_f32_f16(int nmax, bool row_per_wave, int waves, int c);

}  // namespace arf
