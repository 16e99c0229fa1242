// arfuse_table.hpp -- the instantiated launch geometries of the fused kernel and of the
// held-row kernel, and the lookup from (shard count, path, wavefronts per workgroup,
// chunks per lane) to a launcher. Each inst_*.hip translation unit instantiates one element-type pair for a
// range of shard counts, so the 1024 kernels compile in parallel.
//
// Menu: shard count N in 1..16 (exact: no per-shard branch, so the loads of a whole row
// are scheduled freely); one row per wavefront (4 wavefronts per workgroup) with C in
// {1, 2, 4, 8}; one row per workgroup with WAVES in {4, 8, 16} and C in {1, 2, 4, 8}.
// Every geometry has one kernel per (N, C); only its prefetch depth differs by geometry.
#pragma once

#include "arfuse_device.hpp"

namespace arf {

// Shards in flight per row. The 8-wave row-per-workgroup geometry is the plan's choice
// when a launch has fewer than two rows per CU and rows of more than 256 chunks; there the
// time is load latency rather than HBM throughput, so its kernels keep up to three shards
// in flight (bounded by the load registers, C * pieces * 4 VGPRs per slot) instead of one.
// The 4-wave geometry with one 16-byte piece per lane (rows of up to 256 chunks, 16-bit
// partials) keeps three in flight from 8 shards: 16 shards of 64 x 2048 under graph replay
// 3.68 -> 3.41 us, 8 x 16384 x 2048 rows by index 124.2 -> 122.9 us, 2 shards unchanged
// (same outputs).
template <class PT, int C, int W, int N>
constexpr int block_depth() {
    constexpr int pc = C * PartTraits<PT>::kPieces;
    if (W == 4) return pc == 1 && N >= 8 ? 4 : 2;
    return W != 8 ? 2 : (pc <= 4 ? 4 : (pc <= 8 ? 3 : 2));
}

template <class PT, class AT, int N, int W>
launch_fn pick_block_c(int c) {
    switch (c) {
        case 1: return &launch_fused<PT, AT, N, 1, W, false, block_depth<PT, 1, W, N>()>;
        case 2: return &launch_fused<PT, AT, N, 2, W, false, block_depth<PT, 2, W, N>()>;
        case 4: return &launch_fused<PT, AT, N, 4, W, false, block_depth<PT, 4, W, N>()>;
        case 8: return &launch_fused<PT, AT, N, 8, W, false, block_depth<PT, 8, W, N>()>;
        default: return nullptr;
    }
}

template <class PT, class AT, int N>
launch_fn pick_geometry(bool row_per_wave, int waves, int c) {
    if (row_per_wave) {
        if (waves != 4) return nullptr;
        switch (c) {
            case 1: return &launch_fused<PT, AT, N, 1, 4, true>;
            case 2: return &launch_fused<PT, AT, N, 2, 4, true>;
            case 4: return &launch_fused<PT, AT, N, 4, 4, true>;
            case 8: return &launch_fused<PT, AT, N, 8, 4, true>;
            default: return nullptr;
        }
    }
    switch (waves) {
        case 4: return pick_block_c<PT, AT, N, 4>(c);
        case 8: return pick_block_c<PT, AT, N, 8>(c);
        case 16: return pick_block_c<PT, AT, N, 16>(c);
        default: return nullptr;
    }
}

template <class PT, class AT, int NLO, int NHI>
launch_fn pick_shards(int n, bool row_per_wave, int waves, int c) {
    if constexpr (NLO <= NHI) {
        if (n == NLO) return pick_geometry<PT, AT, NLO>(row_per_wave, waves, c);
        return pick_shards<PT, AT, NLO + 1, NHI>(n, row_per_wave, waves, c);
    } else {
        return nullptr;
    }
}

// Held-row kernels: 4 wavefronts with C in {1, 2, 4, 8}, in the general form (any quantised
// copy) for all shard counts and in the form without a quantised copy for 1..4 shards
// (and for fp32 partials with C in {1, 2, 4}, all shard counts); and, for 16-bit partials,
// 8 wavefronts (2 per SIMD) with C in {1, 2, 4} in both forms (all shard counts).
template <class PT, class AT, int N, int W, bool QUANT, int CMAX>
held_launch_fn pick_held_c(int c) {
    switch (c) {
        case 1: return &launch_held<PT, AT, N, 1, W, QUANT>;
        case 2: return &launch_held<PT, AT, N, 2, W, QUANT>;
        case 4: return &launch_held<PT, AT, N, 4, W, QUANT>;
        case 8: if constexpr (CMAX >= 8) return &launch_held<PT, AT, N, 8, W, QUANT>;
                return nullptr;
        default: return nullptr;
    }
}

template <class PT, class AT, int N>
held_launch_fn pick_held(int c, bool quant, int waves) {
    if constexpr (N <= 4) {
        if (!quant && waves == 4) return pick_held_c<PT, AT, N, 4, false, 8>(c);
    } else if constexpr (PartTraits<PT>::kPieces == 2) {
        if (!quant && waves == 4 && c <= 4) return pick_held_c<PT, AT, N, 4, false, 4>(c);
    }
    if constexpr (PartTraits<PT>::kPieces == 1) {
        if (waves == 8) {
            if (quant) return pick_held_c<PT, AT, N, 8, true, 4>(c);
            return pick_held_c<PT, AT, N, 8, false, 4>(c);
        }
    }
    return waves == 4 ? pick_held_c<PT, AT, N, 4, true, 8>(c) : nullptr;
}

template <class PT, class AT, int NLO, int NHI>
held_launch_fn pick_held_shards(int n, int c, bool quant, int waves) {
    if constexpr (NLO <= NHI) {
        if (n == NLO) return pick_held<PT, AT, NLO>(c, quant, waves);
        return pick_held_shards<PT, AT, NLO + 1, NHI>(n, c, quant, waves);
    } else {
        return nullptr;
    }
}

// Defined in the inst_<partial>_<activation>_n<lo>_<hi>.hip translation units.
#define ARF_DECLARE_LOOKUPS(PD, AD)                                              \
    launch_fn lookup_##PD##_##AD##_n01_04(int n, bool rpw, int waves, int c);    \
    launch_fn lookup_##PD##_##AD##_n05_08(int n, bool rpw, int waves, int c);    \
    launch_fn lookup_##PD##_##AD##_n09_12(int n, bool rpw, int waves, int c);    \
    launch_fn lookup_##PD##_##AD##_n13_16(int n, bool rpw, int waves, int c);    \
    held_launch_fn held_##PD##_##AD##_n01_04(int n, int c, bool quant, int waves);           \
    held_launch_fn held_##PD##_##AD##_n05_08(int n, int c, bool quant, int waves);           \
    held_launch_fn held_##PD##_##AD##_n09_12(int n, int c, bool quant, int waves);           \
    held_launch_fn held_##PD##_##AD##_n13_16(int n, int c, bool quant, int waves);
ARF_DECLARE_LOOKUPS(bf16, bf16)
ARF_DECLARE_LOOKUPS(f16, f16)
ARF_DECLARE_LOOKUPS(f32, bf16)
ARF_DECLARE_LOOKUPS(f32, f16)
#undef ARF_DECLARE_LOOKUPS

}  // namespace arf
