// arfuse_device.hpp -- gfx950 device code of libarfuse.
//
// One fused, single-pass kernel: every byte of the partials and the residual is read
// from HBM once, every output is written once. The method (TensorRT-LLM page
// "allReduceFusionKernels.cu": allreduce_sum fp32 branch, fused_op/add128, rms_norm;
// oneshot-sync post-barrier loop for the [N][tokens][hidden] layout) is reproduced in
// its rounding order: fp32 rank-order sum -> cast to the activation type -> residual add
// in the activation type -> mean of squares -> (x * inv) * gamma -> cast.
//
// Design for CDNA4 (not a translation of the page's cluster/DSMEM kernel):
//  * A row (token) belongs to one wavefront (small hidden) or one workgroup (large
//    hidden); the page needed up to 8 cooperating CTAs per token, here one workgroup of
//    up to 16 wave64s covers hidden = 65536.
//  * Each lane owns C 16-byte chunks (8 elements) at chunk index j*G + lane (G lanes per
//    row), so each load instruction of a wavefront covers 1 KiB of contiguous HBM.
//  * All global traffic uses raw buffer instructions with a per-row resource whose size
//    is the row's bytes: lanes past the end of a ragged row read zeros and their stores
//    are dropped by the hardware range check, so there is no tail branch.
//  * Streaming data (partials, residual, outputs) carries the non-temporal hint; gamma is
//    shared by all rows and uses the default policy.
//  * The mean of squares is accumulated in fp64 per lane (squares of 16-bit values are
//    exact in fp64), reduced across the wavefront with DPP lane moves and readlane, and
//    across wavefronts through LDS, in a fixed order: the result does not depend on timing.
//  * The normalised row stays in registers (packed 16-bit) between the two reductions of
//    the per-token fp8 scale, so nothing is re-read from HBM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arf {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Resource word 3 for raw (untyped, stride 0) buffers on gfx9-family GPUs: data format
// 32 bits, no swizzle. With stride 0 the range check compares the byte offset against
// the record count, which is how ragged rows are handled.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of the buffer builtins on gfx940-family GPUs: bit 1 = NT.
constexpr int kAuxStream = 2;
constexpr int kAuxDefault = 0;

enum QuantMode : int32_t { kQuantNone = 0, kQuantTensor = 1, kQuantToken = 2, kQuantMx = 3 };

struct Params {
    const void* partials;
    const void* residual_in;   // NULL in reduce-only mode (its loads then read nothing)
    void* residual_out;        // nullable; the reduced values in reduce-only mode
    const void* gamma;
    void* norm_out;            // nullable
    uint8_t* quant_out;        // used when quant_mode != kQuantNone
    const float* scale_in;
    void* scale_out;           // float [tokens] (per token) or E8M0 bytes [tokens][hidden/32]
    int64_t tokens;            // rows of every buffer (shard stride tokens * hidden)
    int64_t row_begin;         // first row of this launch
    int64_t row_end;           // one past the last row of this launch
    int32_t hidden;
    int32_t n_shards;
    float eps;
    int32_t quant_mode;
    int32_t acc_partial;       // round every partial sum to the partial type
    int32_t reduce_only;       // store the reduced value and stop
    int32_t held_rows;         // held-row kernel: rows a workgroup holds at once (K)
    // Row claims (one row per workgroup only): workgroups with index >= claim_static take
    // their row from one of claim_split counters in the order they start; NULL: row =
    // row_begin + workgroup index.
    uint32_t* claim;           // counter k at claim + 64 k, each 0 at launch and left at 0
    int64_t claim_static;      // workgroups below this index keep row_begin + index
    uint32_t claim_count;      // workgroups that claim (gridDim.x - claim_static), a
                               // multiple of 8 << claim_shift
    uint32_t claim_shift;      // 2^claim_shift counters share the claims (0..2)
};

struct ActBF16 {};
struct ActF16 {};
struct PartF32 {};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferWord3);
}

// ---- 16-bit <-> fp32 -----------------------------------------------------------------

__device__ __forceinline__ void unpack8(ActBF16, u32x4 v, float f[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
}

// The halves are taken with integer shifts: bit-casting a vector element to a half2
// vector here was compiled into a load of the first dword only (hipcc of ROCm 7.2).
__device__ __forceinline__ void unpack8(ActF16, u32x4 v, float f[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = v[i];
        f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
        f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    }
}

// fp32 -> 16-bit, round to nearest even (gfx950 converts bf16 pairs in one instruction).
__device__ __forceinline__ u32x4 pack8(ActBF16, const float f[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x2 a = {f[2 * i], f[2 * i + 1]};
        v[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2));
    }
    return v;
}

__device__ __forceinline__ u32x4 pack8(ActF16, const float f[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x2 a = {f[2 * i], f[2 * i + 1]};
        v[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, f16x2));
    }
    return v;
}

// ---- fp32 -> OCP E4M3 ------------------------------------------------------------------
// Magnitudes above 448 are clamped first (saturating conversion; NaN is kept), with one
// median-of-three, then the hardware converter rounds to nearest even. Four values -> one
// dword, lowest byte first.
__device__ __forceinline__ float e4m3_sat(float v) {
    const float c = __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
    return v != v ? v : c;
}

__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(a), e4m3_sat(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(c), e4m3_sat(d), w, true);
    return (uint32_t)w;
}

// ---- OCP MX FP4 ------------------------------------------------------------------------------
// E8M0 code of a block whose largest magnitude is amax (finite, >= 0): 127 + clamp(
// floor(log2 amax) - 2, -127, 127), 0 for a zero block. frexp's exponent e has
// amax = m * 2^e with m in [0.5, 1), so floor(log2 amax) = e - 1 (denormals included).
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
    if (!(amax > 0.0f)) return 0u;
    int shared = __builtin_amdgcn_frexp_expf(amax) - 1 - 2;
    shared = shared < -127 ? -127 : (shared > 127 ? 127 : shared);
    return (uint32_t)(shared + 127);
}

// E2M1 codes, nibble i holding the code of v[i]: gfx950's packed conversion (two values per
// instruction, into the byte the select names, the other bytes kept), with a scale of 1 (the
// caller has applied the block scale, an exact power of two). It rounds to nearest even over
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}, a tie going to the even code (0.25 -> 0, 0.75 -> 1.0, 1.25 ->
// 1.0, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4), saturates at 6, sends infinities and NaN to
// +-6, and keeps the sign in bit 3 (zeros included). A GPU test checks it against the
// oracle's encoder on every fp32 value of magnitude 2^-4 to 8 and on specials and samples
// beyond; it replaced a chain of seven comparisons per element.
__device__ __forceinline__ uint32_t e2m1_pack4(float v0, float v1, float v2, float v3) {
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v0, v1, 1.0f, 0);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v2, v3, 1.0f, 1);
}
__device__ __forceinline__ uint32_t e2m1_pack8(const float v[8]) {
    uint32_t w = e2m1_pack4(v[0], v[1], v[2], v[3]);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
}

// ---- cross-lane reductions (wave64) ------------------------------------------------------

// Data-parallel-primitive (DPP) lane moves: a VALU operand modifier, no LDS round trip.
// Within each row of 16 lanes: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1]
// (lane ^ 2), row_half_mirror (lane i <-> 7 - i in each group of 8), row_mirror (lane i <->
// 15 - i in each row). After xor-1, xor-2 and half-mirror steps every lane of a group of 8
// holds the same combination of the group's values; after row_mirror, of the row's.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the 64 lanes: a DPP butterfly inside each row of 16 (every lane of a row ends
// with the same value, since each step adds the same two operands in either order), then
// the four row sums in a fixed order. The result is the same in every lane and on every
// run.
__device__ __forceinline__ double wave_sum(double v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppMirror>(v);
    return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

// Maximum over the 64 lanes (fmaxf: a NaN operand is skipped), the same pattern.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    const float a = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0)),
                          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16)));
    const float b = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32)),
                          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48)));
    return fmaxf(a, b);
}

// ---- the fused kernel -------------------------------------------------------------------
//
// PT: partial element type tag (ActBF16 / ActF16 / PartF32); AT: activation tag.
// N: number of shards (exact). C: chunks per lane. WAVES: wavefronts per workgroup.
// ROW_PER_WAVE: each wavefront owns one row (else the whole workgroup owns one row).
// DEPTH: shards in flight while one is added.
//
// The row is streamed shard by shard ("shard-major"): the lanes of the row read shard r's
// whole row (C chunks each), add it into fp32 accumulators in rank order, and meanwhile the
// loads of the next DEPTH-1 shards are in flight; the residual row follows the last shard.
// At any moment a row therefore touches one or two long sequential streams instead of N+1
// interleaved ones, which measured a few per cent faster in HBM than chunk-by-chunk order.
template <class PT> struct PartTraits {
    static constexpr int kPieces = 1;   // 16-byte loads per chunk per shard
    static constexpr int kBytes = 2;
};
template <> struct PartTraits<PartF32> {
    static constexpr int kPieces = 2;
    static constexpr int kBytes = 4;
};

template <class AT>
__device__ __forceinline__ void load_partial_chunk(AT, u32x4 const (&v)[1], float f[8]) {
    unpack8(AT{}, v[0], f);
}
template <class AT>
__device__ __forceinline__ void load_partial_chunk(AT, u32x4 const (&v)[2], float f[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = __uint_as_float(v[0][i]);
        f[4 + i] = __uint_as_float(v[1][i]);
    }
}

// Row layout of a lane's 8 elements in chunk j (G lanes per row, lane gl):
//  * 16-bit partials: elements [8c, 8c+8) with c = j*G + gl -- one 16-byte access per
//    shard and per 16-bit row, each wavefront instruction covering 1 KiB;
//  * fp32 partials ("split"): two quads [4u, 4u+4) with u = (2j+w)*G + gl, w = 0, 1 --
//    every 16-byte partial load is again 1 KiB contiguous per wavefront instruction
//    (instead of 16 of every 32 bytes), and the 16-bit rows use 8-byte accesses.
template <bool SPLIT, int G>
struct Layout {
    // byte offset of the w-th 16-byte partial piece of chunk j
    __device__ static uint32_t part(int j, int w, int gl) {
        return SPLIT ? (uint32_t)((2 * j + w) * G + gl) * 16u
                     : (uint32_t)(j * G + gl) * 16u;
    }
    template <int AUX>
    __device__ static u32x4 load_act(__amdgpu_buffer_rsrc_t r, int j, int gl) {
        if constexpr (SPLIT) {
            const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(
                r, (uint32_t)((2 * j) * G + gl) * 8u, 0, AUX);
            const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(
                r, (uint32_t)((2 * j + 1) * G + gl) * 8u, 0, AUX);
            return u32x4{a[0], a[1], b[0], b[1]};
        } else {
            return __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(j * G + gl) * 16u, 0,
                                                         AUX);
        }
    }
    __device__ static void store_act(u32x4 v, __amdgpu_buffer_rsrc_t r, int j, int gl) {
        if constexpr (SPLIT) {
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{v[0], v[1]}, r,
                                                  (uint32_t)((2 * j) * G + gl) * 8u, 0,
                                                  kAuxStream);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{v[2], v[3]}, r,
                                                  (uint32_t)((2 * j + 1) * G + gl) * 8u, 0,
                                                  kAuxStream);
        } else {
            __builtin_amdgcn_raw_buffer_store_b128(v, r, (uint32_t)(j * G + gl) * 16u, 0,
                                                   kAuxStream);
        }
    }
    // MXFP4 codes and block scales of chunk j. In the 16-bit layout a 32-element block
    // is 4 consecutive lanes (8 elements each); in the split layout it is 8 consecutive
    // lanes' quads of the same half w. y: the lane's 8 cast outputs.
    __device__ static void store_mx(const float y[8], __amdgpu_buffer_rsrc_t q,
                                    __amdgpu_buffer_rsrc_t sc, int j, int gl) {
        if constexpr (SPLIT) {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                float a = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) a = fmaxf(a, __builtin_fabsf(y[4 * w + e]));
                a = fmaxf(a, dpp<kDppXor1>(a));   // the 8 lanes of the block
                a = fmaxf(a, dpp<kDppXor2>(a));
                a = fmaxf(a, dpp<kDppHalfMirror>(a));
                const uint32_t code = mx_scale_code(a);
                const float inv = __builtin_amdgcn_ldexpf(1.0f, 127 - (int)code);
                const uint32_t packed = e2m1_pack4(y[4 * w] * inv, y[4 * w + 1] * inv,
                                                   y[4 * w + 2] * inv, y[4 * w + 3] * inv);
                const uint32_t u = (uint32_t)((2 * j + w) * G + gl);
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)packed, q, u * 2u, 0,
                                                      kAuxStream);
                if ((gl & 7) == 0)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, sc, u / 8u, 0,
                                                         kAuxStream);
            }
        } else {
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, __builtin_fabsf(y[e]));
            a = fmaxf(a, dpp<kDppXor1>(a));   // the 4 lanes of the block
            a = fmaxf(a, dpp<kDppXor2>(a));
            const uint32_t code = mx_scale_code(a);
            const float inv = __builtin_amdgcn_ldexpf(1.0f, 127 - (int)code);
            float ys[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ys[e] = y[e] * inv;
            const uint32_t packed = e2m1_pack8(ys);
            const uint32_t c = (uint32_t)(j * G + gl);
            __builtin_amdgcn_raw_buffer_store_b32(packed, q, c * 4u, 0, kAuxStream);
            if ((gl & 3) == 0)
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, sc, c / 4u, 0, kAuxStream);
        }
    }
    // 8 fp8 codes of chunk j (q[0]: the first four elements, q[1]: the last four)
    __device__ static void store_codes(u32x2 q, __amdgpu_buffer_rsrc_t r, int j, int gl) {
        if constexpr (SPLIT) {
            __builtin_amdgcn_raw_buffer_store_b32(q[0], r, (uint32_t)((2 * j) * G + gl) * 4u,
                                                  0, kAuxStream);
            __builtin_amdgcn_raw_buffer_store_b32(q[1], r,
                                                  (uint32_t)((2 * j + 1) * G + gl) * 4u, 0,
                                                  kAuxStream);
        } else {
            __builtin_amdgcn_raw_buffer_store_b64(q, r, (uint32_t)(j * G + gl) * 8u, 0,
                                                  kAuxStream);
        }
    }
};

template <class PT, class AT, int N, int C, int WAVES, bool ROW_PER_WAVE, int DEPTH = 2>
__global__ __launch_bounds__(WAVES * 64) void fused_reduce_add_rmsnorm(Params p) {
    static_assert(N >= 1 && C >= 1 && DEPTH >= 2, "bad instantiation");
    constexpr int PW = PartTraits<PT>::kPieces;
    constexpr int G = ROW_PER_WAVE ? 64 : WAVES * 64;   // lanes per row
    using L = Layout<(PW == 2), G>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    int64_t row;
    int gl;
    if constexpr (ROW_PER_WAVE) {
        row = p.row_begin + (int64_t)blockIdx.x * WAVES + __builtin_amdgcn_readfirstlane(wave);
        if (row >= p.row_end) return;   // whole wavefront leaves; no workgroup barrier here
        gl = lane;
    } else {
        row = p.row_begin + (int64_t)blockIdx.x;
        gl = threadIdx.x;
        if (p.claim && (int64_t)blockIdx.x >= p.claim_static) {
            // Past the static prefix, rows go to workgroups in the order they start: the
            // rows in flight then stay one compact window of the launch however far the
            // XCDs drift apart, and a faster XCD takes more rows. One relaxed device-scope
            // increment per workgroup. The claims are spread over S = 2^claim_shift
            // counters, 256 bytes apart, since one counter serves only so many claims per
            // microsecond: counter k hands out rows k, k + S, k + 2S, ... to the
            // workgroups i past the prefix with (i / 8) mod S == k, a group of 8
            // consecutive workgroups (one per XCD) at a time, so that every counter serves
            // every XCD. Each counter has claim_count / S claimants; the last increment of
            // each returns it to 0 for the next launch on the same stream. The claimants
            // outnumber the rows left: the surplus finds no row and exits. (Shifts, not a
            // division by S: the claim is on the workgroup's critical path.)
            __shared__ int64_t s_row;
            if (threadIdx.x == 0) {
                const uint32_t sh = p.claim_shift;
                const uint32_t i = blockIdx.x - (uint32_t)p.claim_static;
                const uint32_t k = (i >> 3) & ((1u << sh) - 1u);
                uint32_t* ctr = p.claim + k * 64u;
                const uint32_t c = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                if (c == (p.claim_count >> sh) - 1u)
                    __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_row = p.claim_static + (int64_t)(((uint64_t)c << sh) + k);
            }
            __syncthreads();
            row = p.row_begin + s_row;
            if (row >= p.row_end) return;   // uniform: the whole workgroup leaves
        }
    }

    const uint32_t H = (uint32_t)p.hidden;
    const uint32_t act_row = H * 2u;
    const uint32_t part_row = H * (uint32_t)PartTraits<PT>::kBytes;
    const int64_t act_off = row * (int64_t)act_row;

    const auto r_in = make_rsrc((const char*)p.residual_in + act_off, p.residual_in ? act_row : 0u);
    const auto r_out = make_rsrc((char*)p.residual_out + act_off, p.residual_out ? act_row : 0u);
    const auto y_out = make_rsrc((char*)p.norm_out + act_off, p.norm_out ? act_row : 0u);
    const auto g_in = make_rsrc(p.gamma, act_row);
    // The per-tensor scale is read before any store: read after the output stores, its
    // load waited for all of them to complete (one memory counter covers loads and
    // stores) and then for its own round trip, on the critical path of short launches.
    // It cannot alias an output (the host rejects that overlap).
    const float scale_tensor = p.quant_mode == kQuantTensor ? p.scale_in[0] : 0.0f;

    __amdgpu_buffer_rsrc_t part[N];
#pragma unroll
    for (int r = 0; r < N; ++r)
        part[r] = make_rsrc((const char*)p.partials +
                                ((int64_t)r * p.tokens + row) * (int64_t)part_row,
                            part_row);

    // ---- pass over HBM: rank-order fp32 sum of the shards
    u32x4 buf[DEPTH][C][PW];
    u32x4 rv[C];
    float acc[C][8];
    auto issue_shard = [&](int r, int slot) {
#pragma unroll
        for (int j = 0; j < C; ++j)
#pragma unroll
            for (int w = 0; w < PW; ++w)
                buf[slot][j][w] = __builtin_amdgcn_raw_buffer_load_b128(
                    part[r], L::part(j, w, gl), 0, kAuxStream);
    };
    auto issue_residual = [&]() {
#pragma unroll
        for (int j = 0; j < C; ++j) rv[j] = L::template load_act<kAuxStream>(r_in, j, gl);
    };
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d)
        if (d < N) issue_shard(d, d);
    if (N < DEPTH - 1) issue_residual();
#pragma unroll
    for (int r = 0; r < N; ++r) {
        if (r + DEPTH - 1 < N) issue_shard(r + DEPTH - 1, (r + DEPTH - 1) % DEPTH);
        else if (r + DEPTH - 1 == N) issue_residual();
        const int slot = r % DEPTH;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            float t[8];
            load_partial_chunk(AT{}, buf[slot][j], t);
            if (r == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[j][e] = t[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[j][e] = acc[j][e] + t[e];
                if constexpr (PW == 1) {
                    // the other branch of the page's sum: each partial sum rounded to the
                    // (16-bit) partial type; a select, so the load schedule is unchanged
                    float rnd[8];
                    unpack8(PT{}, pack8(PT{}, acc[j]), rnd);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[j][e] = p.acc_partial ? rnd[e] : acc[j][e];
                }
            }
        }
    }

    if (p.reduce_only) {   // one rank's share of the token-slice exchange
#pragma unroll
        for (int j = 0; j < C; ++j) L::store_act(pack8(AT{}, acc[j]), r_out, j, gl);
        return;
    }

    // ---- cast, residual add, cast, store; sum of squares of the stored value
    double ss = 0.0;
    u32x4 xr[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
        float s[8], res[8], sum[8];
        unpack8(AT{}, pack8(AT{}, acc[j]), s);   // reduced value in the activation type
        unpack8(AT{}, rv[j], res);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] = s[e] + res[e];
        const u32x4 rr = pack8(AT{}, sum);       // residual_out
        L::store_act(rr, r_out, j, gl);
        xr[j] = rr;
        float x[8];
        unpack8(AT{}, rr, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fma((double)x[e], (double)x[e], ss);
    }

    u32x4 gv[C];
#pragma unroll
    for (int j = 0; j < C; ++j) gv[j] = L::template load_act<kAuxDefault>(g_in, j, gl);

    // ---- mean of squares across the row
    ss = wave_sum(ss);
    if constexpr (!ROW_PER_WAVE) {
        __shared__ double s_ss[WAVES];
        if (lane == 0) s_ss[wave] = ss;
        __syncthreads();
        ss = 0.0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) ss += s_ss[w];
    }
    const float inv = (float)(1.0 / __builtin_sqrt(ss / (double)H + (double)p.eps));

    // ---- normalise, store, and keep the cast result for the fp8 copy
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < C; ++j) {
        float x[8], g[8], y[8];
        unpack8(AT{}, xr[j], x);
        unpack8(AT{}, gv[j], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = x[e] * inv;
            y[e] = v * g[e];
        }
        const u32x4 yr = pack8(AT{}, y);
        L::store_act(yr, y_out, j, gl);
        xr[j] = yr;
        if (p.quant_mode == kQuantToken) {
            float yc[8];
            unpack8(AT{}, yr, yc);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, __builtin_fabsf(yc[e]));
        }
    }
    if (p.quant_mode == kQuantNone) return;

    // ---- MXFP4 copy: blocks of 32 share 2^(floor(log2 amax) - 2); E2M1 codes of y / X
    if (p.quant_mode == kQuantMx) {
        const auto q_mx = make_rsrc(p.quant_out + row * (int64_t)(H / 2), H / 2);
        const auto s_mx = make_rsrc((uint8_t*)p.scale_out + row * (int64_t)(H / 32), H / 32);
#pragma unroll
        for (int j = 0; j < C; ++j) {
            float y[8];
            unpack8(AT{}, xr[j], y);
            L::store_mx(y, q_mx, s_mx, j, gl);
        }
        return;
    }

    // ---- fp8 copy: q = E4M3(y * (1/scale))
    float scale;
    if (p.quant_mode == kQuantToken) {
        amax = wave_max(amax);
        if constexpr (!ROW_PER_WAVE) {
            __shared__ float s_max[WAVES];
            if (lane == 0) s_max[wave] = amax;
            __syncthreads();
            amax = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) amax = fmaxf(amax, s_max[w]);
        }
        scale = amax / 448.0f;
        if (gl == 0) static_cast<float*>(p.scale_out)[row] = scale;
    } else {
        scale = scale_tensor;
    }
    const float inv_scale = scale > 0.0f ? 1.0f / scale : 0.0f;
    const auto q_out = make_rsrc(p.quant_out + row * (int64_t)H, H);
#pragma unroll
    for (int j = 0; j < C; ++j) {
        float y[8];
        unpack8(AT{}, xr[j], y);
        u32x2 q;
        q[0] = e4m3x4(y[0] * inv_scale, y[1] * inv_scale, y[2] * inv_scale, y[3] * inv_scale);
        q[1] = e4m3x4(y[4] * inv_scale, y[5] * inv_scale, y[6] * inv_scale, y[7] * inv_scale);
        L::store_codes(q, q_out, j, gl);
    }
}

// ---- the held-row kernel ----------------------------------------------------------------
//
// Persistent workgroups (at most one per compute unit, of 4 or 8 wavefronts: WAVES / 4 per
// SIMD), each owning whole rows. A workgroup
// works in batches of up to K rows:
//  * read half: it streams its rows (shards shard-major, then the residual; the first D-1
//    shards of the next row are loaded while the current row finishes) and keeps each row's
//    rounded residual r in LDS, plus each wavefront's part of sum(r^2);
//  * write half: for each held row it stores residual_out, recomputes y = cast((r*inv)*gamma)
//    from r, inv and gamma, and stores norm_out and the quantised copy.
// When the whole launch fits in one batch per workgroup, HBM sees one long stretch of reads
// and then one of writes, instead of reads and writes interleaved row by row (a bus
// turnaround each time). Workgroup g takes rows g, g + G, g + 2G, ... in batches of K, so at
// any moment the chip works on one compact window of rows.
//
// The arithmetic, and its order, is that of fused_reduce_add_rmsnorm's row-per-workgroup
// form with the same number of wavefronts: the outputs are the same bits. The write half
// uses the 16-bit layout for every partial type (lane gl owns 8 consecutive elements per
// chunk, 16-byte stores): the LDS image of a row is its HBM byte image, and only the lane
// that computes an element changes; the sum of squares is taken in the read layout and the
// per-token maximum does not depend on the order.
//
// LDS (size set by the host): K rows of hidden*2 bytes, then K*WAVES fp64 partial sums of
// squares and K*WAVES fp32 maxima. Only hidden/8 <= C * WAVES * 64 is supported (the host
// checks).
template <class PT, class AT, int N, int C, int WAVES, bool QUANT>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4)))
void fused_held_rows(Params p) {
    constexpr int PW = PartTraits<PT>::kPieces;
    constexpr int G = WAVES * 64;              // lanes per row
    // segments in flight (D - 1 <= N): one ahead for fp32 partials, two for 16-bit ones (a
    // sweep of 9 held-region shapes: one ahead 1.6-4% faster with fp32 partials, up to 10%
    // slower with 16-bit ones)
    constexpr int DS = PW == 2 ? 2 : 3;
    constexpr int D = N + 1 < DS ? N + 1 : DS;
    constexpr bool SPLIT = PW == 2;
    using L = Layout<SPLIT, G>;
    using LW = Layout<false, G>;
    extern __shared__ __align__(16) char s_dyn[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int gl = threadIdx.x;
    const int K = p.held_rows;
    const uint32_t H = (uint32_t)p.hidden;
    const uint32_t act_row = H * 2u;
    const uint32_t part_row = H * (uint32_t)PartTraits<PT>::kBytes;
    const uint32_t n_pieces = SPLIT ? H / 4u : H / 8u;   // 8- or 16-byte pieces of a 16-bit row
    double* s_ss = reinterpret_cast<double*>(s_dyn + (size_t)K * act_row);
    float* s_mx = reinterpret_cast<float*>(s_ss + K * WAVES);

    const auto g_in = make_rsrc(p.gamma, act_row);
    u32x4 gv[C];
#pragma unroll
    for (int j = 0; j < C; ++j) gv[j] = LW::template load_act<kAuxDefault>(g_in, j, gl);
    // QUANT = false: the instantiation for calls without a quantised copy. Without the
    // quantisation paths the kernel needs fewer scalar registers: the general form spills
    // 74 of them into vector-register lanes, reloaded inside the row loop (4 fp32 shards of
    // 2048 x 7168: 53.5 -> 51.4 us).
    const int32_t qmode = QUANT ? p.quant_mode : (int32_t)kQuantNone;
    const float scale_tensor = qmode == kQuantTensor ? p.scale_in[0] : 0.0f;

    auto hold_store = [&](char* row, int j, u32x4 v) {   // chunk j of the read layout
        if constexpr (SPLIT) {
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                const uint32_t u = (uint32_t)((2 * j + w) * G + gl);
                if (u < n_pieces)
                    *reinterpret_cast<u32x2*>(row + u * 8u) = w ? u32x2{v[2], v[3]} : u32x2{v[0], v[1]};
            }
        } else {
            const uint32_t c = (uint32_t)(j * G + gl);
            if (c < n_pieces) *reinterpret_cast<u32x4*>(row + c * 16u) = v;
        }
    };
    auto hold_load = [&](const char* row, int j) {   // chunk j of the 16-bit layout
        u32x4 v = {0u, 0u, 0u, 0u};
        const uint32_t c = (uint32_t)(j * G + gl);
        if (c < H / 8u) v = *reinterpret_cast<const u32x4*>(row + c * 16u);
        return v;
    };
    // The same without the zero fill: a lane past the row's end reads chunk 0 instead. For
    // the write half only, whose stores past the row's end the range check drops (an MXFP4
    // block never straddles the end, since hidden % 32 == 0): with no branch per chunk the
    // reads of a row issue together.
    auto hold_load_any = [&](const char* row, int j) {
        const uint32_t c = (uint32_t)(j * G + gl);
        return *reinterpret_cast<const u32x4*>(row + (c < H / 8u ? c : 0u) * 16u);
    };
    auto shard_rsrc = [&](int64_t row, int r, bool valid) {
        return make_rsrc((const char*)p.partials + ((int64_t)r * p.tokens + row) * (int64_t)part_row,
                         valid ? part_row : 0u);
    };
    auto row_inv = [&](int k) {
        double ss = 0.0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) ss += s_ss[k * WAVES + w];
        return (float)(1.0 / __builtin_sqrt(ss / (double)H + (double)p.eps));
    };

    // Workgroup g's i-th row is row_begin + T(i), T(i) = (i / K)*G*K + (i % K)*G + g; rows
    // of a batch are consecutive i. T(i) >= rows: no more rows (T grows with i).
    const int64_t rows = p.row_end - p.row_begin;
    const int64_t grid = gridDim.x;
    auto ticket = [&](int64_t i) { return (i / K) * (grid * K) + (i % K) * grid + blockIdx.x; };
    int64_t seq = 0;               // rows taken so far: the current row is T(seq)
    int64_t cur = ticket(0), nxt = ticket(1);

    // Shard segments of the current row. Slots [0, D-1) arrive loaded ahead: the next row's
    // first D-1 shards are issued into them once the current row has consumed them, so no
    // copy between registers (which would wait for the loads in flight) is needed.
    u32x4 sb[N][C][PW];
    while (cur < rows) {
        // ---- read half: up to K rows in, r held in LDS
        {
            const auto row0 = p.row_begin + cur;
#pragma unroll
            for (int d = 0; d < D - 1; ++d) {
                const auto rs = shard_rsrc(row0, d, true);
#pragma unroll
                for (int j = 0; j < C; ++j)
#pragma unroll
                    for (int w = 0; w < PW; ++w)
                        sb[d][j][w] = __builtin_amdgcn_raw_buffer_load_b128(rs, L::part(j, w, gl), 0, kAuxStream);
            }
        }
        int kn = 0;
        for (;;) {
            const int k = kn;
            const int64_t row = p.row_begin + cur;
            const bool nvalid = k + 1 < K && nxt < rows;   // the next row joins this batch
            const int64_t nrow = p.row_begin + (nxt < rows ? nxt : cur);
            __amdgpu_buffer_rsrc_t part[N];
#pragma unroll
            for (int r = 0; r < N; ++r) part[r] = shard_rsrc(row, r, true);
            const auto r_in = make_rsrc((const char*)p.residual_in + row * (int64_t)act_row, act_row);
            u32x4 rv[C];
            float acc[C][8];
            double ss = 0.0;
            char* hrow = s_dyn + (size_t)k * act_row;
#pragma unroll
            for (int s = 0; s <= N; ++s) {
                const int t = s + D - 1;   // segment issued now: shard t, the residual (t == N),
                if (t < N) {               // or shard t - N - 1 of the next row, into its
                                           // slot (consumed at step t - N - 1 < s)
#pragma unroll
                    for (int j = 0; j < C; ++j)
#pragma unroll
                        for (int w = 0; w < PW; ++w)
                            sb[t][j][w] = __builtin_amdgcn_raw_buffer_load_b128(part[t], L::part(j, w, gl), 0, kAuxStream);
                } else if (t == N) {
#pragma unroll
                    for (int j = 0; j < C; ++j) rv[j] = L::template load_act<kAuxStream>(r_in, j, gl);
                } else {
                    const auto rs = shard_rsrc(nrow, t - N - 1, nvalid);
#pragma unroll
                    for (int j = 0; j < C; ++j)
#pragma unroll
                        for (int w = 0; w < PW; ++w)
                            sb[t - N - 1][j][w] = __builtin_amdgcn_raw_buffer_load_b128(rs, L::part(j, w, gl), 0, kAuxStream);
                }
                if (s < N) {
#pragma unroll
                    for (int j = 0; j < C; ++j) {
                        float f[8];
                        load_partial_chunk(AT{}, sb[s][j], f);
                        if (s == 0) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) acc[j][e] = f[e];
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) acc[j][e] = acc[j][e] + f[e];
                            if constexpr (PW == 1) {
                                float rnd[8];
                                unpack8(PT{}, pack8(PT{}, acc[j]), rnd);
#pragma unroll
                                for (int e = 0; e < 8; ++e) acc[j][e] = p.acc_partial ? rnd[e] : acc[j][e];
                            }
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < C; ++j) {
                        float sv[8], res[8], sum[8];
                        unpack8(AT{}, pack8(AT{}, acc[j]), sv);
                        unpack8(AT{}, rv[j], res);
#pragma unroll
                        for (int e = 0; e < 8; ++e) sum[e] = sv[e] + res[e];
                        const u32x4 rr = pack8(AT{}, sum);
                        hold_store(hrow, j, rr);
                        float x[8];
                        unpack8(AT{}, rr, x);
#pragma unroll
                        for (int e = 0; e < 8; ++e) ss = __builtin_fma((double)x[e], (double)x[e], ss);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);   // keep the ring: D-1 segments in flight
            }
            ss = wave_sum(ss);
            if (lane == 0) s_ss[k * WAVES + wave] = ss;
            kn = k + 1;
            cur = nxt;
            nxt = ticket(++seq + 1);
            if (!nvalid) break;
        }
        __syncthreads();

        // inv of held row k is formed by lane k of every wavefront, in parallel: one chain of
        // fp64 divide and square root per wavefront instead of one per row, which with one
        // wavefront per SIMD nothing else would hide. Rows beyond the 64th (small hidden
        // sizes only) form theirs in turn. Same operations, so the same bits.
        const float inv_lane = lane < kn ? row_inv(lane) : 0.0f;
        auto inv_of = [&](int k) {
            return k < 64 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                          __builtin_bit_cast(int, inv_lane), k))
                          : row_inv(k);
        };

        // ---- per-token maxima of the cast outputs (needed before the first code is written)
        if (qmode == kQuantToken) {
            for (int k = 0; k < kn; ++k) {
                const float inv = inv_of(k);
                const char* hrow = s_dyn + (size_t)k * act_row;
                float amax = 0.0f;
#pragma unroll
                for (int j = 0; j < C; ++j) {
                    float x[8], g[8], y[8], yc[8];
                    unpack8(AT{}, hold_load(hrow, j), x);
                    unpack8(AT{}, gv[j], g);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float v = x[e] * inv;
                        y[e] = v * g[e];
                    }
                    unpack8(AT{}, pack8(AT{}, y), yc);
#pragma unroll
                    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, __builtin_fabsf(yc[e]));
                }
                amax = wave_max(amax);
                if (lane == 0) s_mx[k * WAVES + wave] = amax;
            }
            __syncthreads();
        }

        // ---- write half (the batch's rows are T(seq - kn) .. T(seq - 1))
        for (int k = 0; k < kn; ++k) {
            const int64_t row = p.row_begin + ticket(seq - kn + k);
            const int64_t act_off = row * (int64_t)act_row;
            const auto r_out = make_rsrc((char*)p.residual_out + act_off, p.residual_out ? act_row : 0u);
            const auto y_out = make_rsrc((char*)p.norm_out + act_off, p.norm_out ? act_row : 0u);
            const char* hrow = s_dyn + (size_t)k * act_row;
            const float inv = inv_of(k);
            float inv_scale = 0.0f;
            if (qmode == kQuantToken) {
                float amax = 0.0f;
#pragma unroll
                for (int w = 0; w < WAVES; ++w) amax = fmaxf(amax, s_mx[k * WAVES + w]);
                const float scale = amax / 448.0f;
                if (gl == 0) static_cast<float*>(p.scale_out)[row] = scale;
                inv_scale = scale > 0.0f ? 1.0f / scale : 0.0f;
            } else if (qmode == kQuantTensor) {
                inv_scale = scale_tensor > 0.0f ? 1.0f / scale_tensor : 0.0f;
            }
            const auto q_out = make_rsrc(p.quant_out + row * (int64_t)H, p.quant_out ? H : 0u);
            const auto q_mx = make_rsrc(p.quant_out + row * (int64_t)(H / 2), p.quant_out ? H / 2 : 0u);
            const auto s_mxo = make_rsrc((uint8_t*)p.scale_out + row * (int64_t)(H / 32), p.scale_out ? H / 32 : 0u);
            u32x4 rrs[C];
#pragma unroll
            for (int j = 0; j < C; ++j) rrs[j] = hold_load_any(hrow, j);
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const u32x4 rr = rrs[j];
                LW::store_act(rr, r_out, j, gl);
                float x[8], g[8], y[8];
                unpack8(AT{}, rr, x);
                unpack8(AT{}, gv[j], g);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float v = x[e] * inv;
                    y[e] = v * g[e];
                }
                const u32x4 yr = pack8(AT{}, y);
                LW::store_act(yr, y_out, j, gl);
                if (qmode == kQuantNone) continue;
                float yc[8];
                unpack8(AT{}, yr, yc);
                if (qmode == kQuantMx) {
                    LW::store_mx(yc, q_mx, s_mxo, j, gl);
                } else {
                    u32x2 q;
                    q[0] = e4m3x4(yc[0] * inv_scale, yc[1] * inv_scale, yc[2] * inv_scale, yc[3] * inv_scale);
                    q[1] = e4m3x4(yc[4] * inv_scale, yc[5] * inv_scale, yc[6] * inv_scale, yc[7] * inv_scale);
                    LW::store_codes(q, q_out, j, gl);
                }
            }
        }
        __syncthreads();   // the next batch reuses the LDS rows
    }
}

// Host-side launcher for one instantiation; returns the launch's own status. `lds` bytes of
// dynamic LDS are reserved per workgroup (the kernel does not use them): a reservation caps
// how many workgroups share a compute unit.
template <class PT, class AT, int N, int C, int WAVES, bool ROW_PER_WAVE, int DEPTH = 2>
hipError_t launch_fused(const Params& p, uint32_t grid, uint32_t lds, hipStream_t stream) {
    Params arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(
            &fused_reduce_add_rmsnorm<PT, AT, N, C, WAVES, ROW_PER_WAVE, DEPTH>),
        dim3(grid), dim3(WAVES * 64), args, lds, stream);
}

typedef hipError_t (*launch_fn)(const Params&, uint32_t, uint32_t, hipStream_t);

// Held-row kernel launcher: `lds` bytes of dynamic LDS per workgroup.
template <class PT, class AT, int N, int C, int WAVES, bool QUANT>
hipError_t launch_held(const Params& p, uint32_t grid, uint32_t lds, hipStream_t stream) {
    Params arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&fused_held_rows<PT, AT, N, C, WAVES, QUANT>),
        dim3(grid), dim3(WAVES * 64), args, lds, stream);
}

typedef hipError_t (*held_launch_fn)(const Params&, uint32_t, uint32_t, hipStream_t);

}  // namespace arf
