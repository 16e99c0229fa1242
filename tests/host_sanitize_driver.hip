// Host-side driver for the sanitized build of libarfuse's dispatcher (CPU only): every
// entry point with invalid arguments, every status string, the launch plan over a grid of
// sizes and CU counts, and the geometry override. The kernel lookup tables are replaced by
// stubs, so nothing is launched; where a call passes validation it needs a device, and on
// a host without one it must return ARF_ERR_HIP.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "arfuse.h"
#include "arfuse_table.hpp"

namespace arf {
#define ARF_STUB(PD, AD, R)                                                         \
    launch_fn lookup_##PD##_##AD##_##R(int, bool, int, int) { return nullptr; }     \
    held_launch_fn held_##PD##_##AD##_##R(int, int, bool, int) { return nullptr; }
#define ARF_STUBS(PD, AD) \
    ARF_STUB(PD, AD, n01_04) ARF_STUB(PD, AD, n05_08) ARF_STUB(PD, AD, n09_12) ARF_STUB(PD, AD, n13_16)
ARF_STUBS(bf16, bf16)
ARF_STUBS(f16, f16)
ARF_STUBS(f32, bf16)
ARF_STUBS(f32, f16)
}  // namespace arf

static int g_checks = 0, g_fail = 0;
static int64_t div_up_i64(int64_t a, int64_t b) { return (a + b - 1) / b; }
#define EXPECT(cond)                                                        \
    do {                                                                    \
        ++g_checks;                                                         \
        if (!(cond)) {                                                      \
            ++g_fail;                                                       \
            std::printf("FAILED line %d: %s\n", __LINE__, #cond);           \
        }                                                                   \
    } while (0)

int main() {
    int devices = 0;
    const bool have_device = hipGetDeviceCount(&devices) == hipSuccess && devices > 0;
    // fake, well-aligned, disjoint addresses: validation never dereferences them
    char* base = reinterpret_cast<char*>(uintptr_t(1) << 40);
    void* P = base;                         // partials
    void* R = base + (1 << 24);             // residual_in
    void* RO = base + (2 << 24);            // residual_out
    void* G = base + (3 << 24);             // gamma
    void* NO = base + (4 << 24);            // norm_out
    uint8_t* Q = reinterpret_cast<uint8_t*>(base + (5 << 24));
    float* S = reinterpret_cast<float*>(base + (6 << 24));

    EXPECT(arf_version() == ARF_VERSION);
    for (int s = -3; s < 12; ++s) EXPECT(arf_status_string(s) != nullptr && std::strlen(arf_status_string(s)) > 0);

    // the non-quant entry point
    EXPECT(arf_reduce_add_rmsnorm(P, 0, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_reduce_add_rmsnorm(P, 17, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, -1, 64, 0, 0, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, int64_t(1) << 31, 64, 0, 0, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 60, 0, 0, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 65544, 0, 0, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 1, 0, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_DTYPE);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 2, 2, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_DTYPE);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 0, 0, R, RO, G, -1.0f, NO, nullptr) == ARF_ERR_VALUE);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 0, 0, R, RO, G, 1.0f / 0.0f, NO, nullptr) == ARF_ERR_VALUE);
    EXPECT(arf_reduce_add_rmsnorm(nullptr, 2, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_NULL);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 0, 0, R, nullptr, G, 1e-6f, nullptr, nullptr) == ARF_ERR_NO_OUTPUT);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 0, 0, R, base + (2 << 24) + 8, G, 1e-6f, NO, nullptr) == ARF_ERR_ALIGN);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 0, 0, R, base + 64, G, 1e-6f, NO, nullptr) == ARF_ERR_ALIAS);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 0, 0, R, RO, G, 1e-6f, RO, nullptr) == ARF_ERR_ALIAS);
    EXPECT(arf_reduce_add_rmsnorm(P, 2, 0, 64, 0, 0, nullptr, nullptr, nullptr, 0.0f, nullptr, nullptr) == ARF_OK);

    // quantised copies
    EXPECT(arf_reduce_add_rmsnorm_quant(P, 2, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, Q, 5, S, S, nullptr) == ARF_ERR_VALUE);
    EXPECT(arf_reduce_add_rmsnorm_quant(P, 2, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, Q, ARF_QUANT_MXFP4, S, S, nullptr) == ARF_ERR_VALUE);
    EXPECT(arf_reduce_add_rmsnorm_quant(P, 2, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, nullptr, ARF_QUANT_PER_TOKEN, nullptr, S, nullptr) == ARF_ERR_NULL);
    EXPECT(arf_reduce_add_rmsnorm_quant(P, 2, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, Q, ARF_QUANT_PER_TENSOR, nullptr, nullptr, nullptr) == ARF_ERR_NULL);
    EXPECT(arf_reduce_add_rmsnorm_quant(P, 2, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, Q, ARF_QUANT_PER_TOKEN, nullptr,
                                        reinterpret_cast<float*>(base + (6 << 24) + 2), nullptr) == ARF_ERR_ALIGN);
    EXPECT(arf_reduce_add_rmsnorm_quant(P, 2, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, reinterpret_cast<uint8_t*>(NO) + 64, ARF_QUANT_PER_TOKEN, nullptr, S, nullptr) == ARF_ERR_ALIAS);

    // the general form
    arf_params a;
    std::memset(&a, 0, sizeof a);
    a.struct_size = sizeof a; a.n_shards = 2; a.partials = P; a.tokens = 4; a.row_begin = 0; a.row_count = -1;
    a.hidden = 64; a.residual_in = R; a.residual_out = RO; a.gamma = G; a.eps = 1e-6f; a.norm_out = NO;
    EXPECT(arf_fused_epilogue(nullptr, nullptr) == ARF_ERR_NULL);
    arf_params b = a; b.struct_size = sizeof a - 8; EXPECT(arf_fused_epilogue(&b, nullptr) == ARF_ERR_VALUE);
    b = a; b.row_begin = 5; EXPECT(arf_fused_epilogue(&b, nullptr) == ARF_ERR_SHAPE);
    b = a; b.row_begin = 3; b.row_count = 2; EXPECT(arf_fused_epilogue(&b, nullptr) == ARF_ERR_SHAPE);
    b = a; b.row_begin = 4; b.row_count = -1; b.partials = nullptr; EXPECT(arf_fused_epilogue(&b, nullptr) == ARF_OK);
    b = a; b.accumulate = 2; EXPECT(arf_fused_epilogue(&b, nullptr) == ARF_ERR_VALUE);
    b = a; b.quant_out = Q; b.quant_mode = 9; EXPECT(arf_fused_epilogue(&b, nullptr) == ARF_ERR_VALUE);
    b = a; b.quant_out = Q; b.quant_mode = ARF_QUANT_MXFP4; b.scale_out = S; b.hidden = 40; EXPECT(arf_fused_epilogue(&b, nullptr) == ARF_ERR_SHAPE);
    b = a; b.quant_out = Q; b.quant_mode = ARF_QUANT_MXFP4; b.scale_out = nullptr; EXPECT(arf_fused_epilogue(&b, nullptr) == ARF_ERR_NULL);

    // reduce only
    EXPECT(arf_reduce_rows(P, 2, 4, 0, -1, 64, 0, 0, 0, nullptr, nullptr) == ARF_ERR_NULL);
    EXPECT(arf_reduce_rows(P, 2, 4, 3, 2, 64, 0, 0, 0, RO, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_reduce_rows(P, 2, 4, 0, -1, 64, 0, 0, 7, RO, nullptr) == ARF_ERR_VALUE);
    EXPECT(arf_reduce_rows(P, 2, 4, 4, -1, 64, 0, 0, 0, nullptr, nullptr) == ARF_OK);

    // utilities
    EXPECT(arf_e4m3_encode(nullptr, Q, -1, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_e4m3_encode(nullptr, Q, 0, nullptr) == ARF_OK);
    EXPECT(arf_e4m3_encode(nullptr, Q, 4, nullptr) == ARF_ERR_NULL);
    EXPECT(arf_e4m3_encode(reinterpret_cast<float*>(base + 2), Q, 4, nullptr) == ARF_ERR_ALIGN);
    EXPECT(arf_e2m1_encode(nullptr, Q, -1, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_e2m1_encode(nullptr, Q, 0, nullptr) == ARF_OK);
    EXPECT(arf_e2m1_encode(nullptr, Q, 4, nullptr) == ARF_ERR_NULL);
    EXPECT(arf_e2m1_encode(reinterpret_cast<float*>(base + 2), Q, 4, nullptr) == ARF_ERR_ALIGN);
    EXPECT(arf_stream_copy(RO, P, 24, nullptr) == ARF_ERR_SHAPE);
    EXPECT(arf_stream_copy(P, base + 16, 64, nullptr) == ARF_ERR_ALIAS);
    EXPECT(arf_stream_mix(nullptr, 0, nullptr, 0, 0, nullptr) == ARF_OK);
    EXPECT(arf_stream_mix(RO, 32, nullptr, 32, 0, nullptr) == ARF_ERR_NULL);
    EXPECT(arf_stream_mix(RO, 16, P, 16, int64_t(1) << 40, nullptr) == ARF_ERR_SHAPE);

    // calls that pass validation need a device
    if (!have_device) {
        EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 0, 0, R, RO, G, 1e-6f, NO, nullptr) == ARF_ERR_HIP);
        EXPECT(arf_reduce_add_rmsnorm(P, 2, 4, 64, 0, 0, R, R, G, 1e-6f, nullptr, nullptr) == ARF_ERR_HIP);
        EXPECT(arf_fused_epilogue(&a, nullptr) == ARF_ERR_HIP);
        EXPECT(arf_reduce_rows(P, 2, 4, 1, 2, 64, 2, 0, 1, RO, nullptr) == ARF_ERR_HIP);
        EXPECT(arf_stream_copy(RO, P, 64, nullptr) == ARF_ERR_HIP);
        int32_t out[4];
        EXPECT(arf_get_plan(2, 4, 64, 0, 0, out) == ARF_ERR_HIP);
    }

    // the plan over sizes and CU counts: the row is covered, the geometry is in the menu
    const int cus_list[] = {1, 2, 3, 80, 256, 304, 1024};
    const int64_t tok_list[] = {0, 1, 2, 3, 4, 5, 63, 64, 255, 256, 511, 512, 513, 2047, 2048, 8191,
                                8192, 65535, 1 << 20, (int64_t(1) << 31) - 1};
    for (int cus : cus_list)
        for (int64_t t : tok_list)
            for (int h = 8; h <= ARF_MAX_HIDDEN; h += (h < 1024 ? 8 : (h < 8192 ? 136 : 2056))) {
                for (int n : {3, 8}) {
                    int32_t o[4];
                    if (arf_get_plan(n, t, h, ARF_BF16, cus, o) != ARF_OK) { EXPECT(false); continue; }
                    const int64_t lanes = o[0] == 1 ? 64 : 64 * (int64_t)o[1];
                    EXPECT(o[0] == 1 || o[0] == 2 || o[0] == 3 || o[0] == 4);
                    EXPECT(o[2] == 1 || o[2] == 2 || o[2] == 4 || o[2] == 8);
                    EXPECT(o[0] == 2 ? (o[1] == 4 || o[1] == 8 || o[1] == 16)
                                     : o[0] == 3 ? (o[1] == 8 && o[2] <= 4)   // bf16: 8 wavefronts
                                                 : o[1] == 4);
                    EXPECT(lanes * o[2] * 8 >= h);
                    // held rows: one workgroup per compute unit, the whole launch in one batch
                    // of at most 160 KiB of LDS per workgroup; claimed rows: a static prefix
                    // of per_cu workgroups per CU, then claimants for the rows left plus
                    // max(64, rows/16), rounded up to a multiple of 8 * split, in one dispatch
                    const int64_t surplus = t / 16 > 64 ? t / 16 : 64;
                    int64_t g = o[0] == 1 ? (t + 3) / 4 : o[0] == 2 ? t : (t < cus ? t : cus);
                    if (o[0] == 4) {
                        const int64_t row_bytes = (int64_t)n * h * 2 + 6LL * h;
                        int split = 0, per_cu = 0;
                        if ((t >= 16LL * cus && row_bytes >= 128 * 1024) ||
                            (t >= 8LL * cus && row_bytes >= 256 * 1024)) {
                            split = row_bytes >= 256 * 1024 ? 1 : 2; per_cu = 2;
                        } else if (t >= 32LL * cus && h / 8 >= 256 && row_bytes >= 32 * 1024) {
                            split = row_bytes >= 96 * 1024 ? 2 : 4;
                            per_cu = split;
                        }
                        EXPECT(split > 0);
                        const int64_t first = t < (int64_t)per_cu * cus ? t : (int64_t)per_cu * cus;
                        const int64_t unit = 8LL * (split > 0 ? split : 1);
                        g = first + div_up_i64(t - first + surplus, unit) * unit;
                        EXPECT(g * 256 <= (int64_t)UINT32_MAX);
                    }
                    EXPECT((int64_t)(uint32_t)o[3] == g);
                    // every launch of one row per workgroup or wavefront fits the work-item
                    // limit of one dispatch, or is split by the caller into row ranges
                    if (o[0] != 2 && o[0] != 1) EXPECT((int64_t)(uint32_t)o[3] * lanes <= (int64_t)UINT32_MAX);
                    if (o[0] == 3) {
                        EXPECT(t >= 3LL * cus && h >= 4096 && h <= 8192);
                        EXPECT(div_up_i64(t, cus) * (2LL * h + 12LL * o[1]) <= 160 * 1024);
                    }
                }
            }
    int32_t o[4];
    EXPECT(arf_get_plan(3, 8, 64, ARF_BF16, 256, nullptr) == ARF_ERR_NULL);
    EXPECT(arf_get_plan(0, 8, 64, ARF_BF16, 256, o) == ARF_ERR_SHAPE);
    EXPECT(arf_get_plan(3, 8, 64, 5, 256, o) == ARF_ERR_DTYPE);

    // the override: accepted values force the geometry; others are refused
    EXPECT(arf_set_path_override(1, 0, 0) == ARF_OK);
    EXPECT(arf_get_plan(3, 100, 1024, ARF_BF16, 256, o) == ARF_OK && o[0] == 1 && o[3] == 25);
    EXPECT(arf_get_plan(3, 100, 8192, ARF_BF16, 256, o) == ARF_ERR_VALUE);
    EXPECT(arf_set_path_override(2, 16, 8) == ARF_OK);
    EXPECT(arf_get_plan(3, 100, 65536, ARF_BF16, 256, o) == ARF_OK && o[1] == 16 && o[2] == 8);
    EXPECT(arf_set_path_override(2, 4, 1) == ARF_OK);
    EXPECT(arf_get_plan(3, 100, 4096, ARF_BF16, 256, o) == ARF_ERR_VALUE);
    // held rows forced: 8 wavefronts for 16-bit partials (4 for fp32), grid min(rows,
    // CUs); refused where a row needs more than 8 chunks per lane
    EXPECT(arf_set_path_override(3, 0, 0) == ARF_OK);
    EXPECT(arf_get_plan(8, 100, 16384, ARF_BF16, 256, o) == ARF_OK && o[0] == 3 && o[1] == 8 && o[2] == 4 && o[3] == 100);
    EXPECT(arf_get_plan(8, 100, 16384, ARF_F32, 256, o) == ARF_OK && o[0] == 3 && o[1] == 4 && o[2] == 8 && o[3] == 100);
    EXPECT(arf_get_plan(8, 8192, 1024, ARF_BF16, 256, o) == ARF_OK && o[0] == 3 && o[2] == 1 && o[3] == 256);
    EXPECT(arf_get_plan(8, 100, 16392, ARF_BF16, 256, o) == ARF_ERR_VALUE);
    EXPECT(arf_set_path_override(3, 4, 2) == ARF_OK);
    EXPECT(arf_get_plan(8, 100, 4096, ARF_BF16, 256, o) == ARF_OK && o[0] == 3 && o[2] == 2);
    EXPECT(arf_get_plan(8, 100, 4104, ARF_BF16, 256, o) == ARF_ERR_VALUE);
    // claimed rows forced: every row claimed, any row count (claimants rounded up to a
    // multiple of 8 * split: 4 counters below 96 KiB per row, 2 below 256 KiB, else 1);
    // beyond one dispatch, path 2
    EXPECT(arf_set_path_override(4, 0, 0) == ARF_OK);
    EXPECT(arf_get_plan(8, 100, 4096, ARF_BF16, 256, o) == ARF_OK && o[0] == 4 && o[1] == 4 && o[2] == 2 && o[3] == 192);
    EXPECT(arf_get_plan(8, 100, 8192, ARF_BF16, 256, o) == ARF_OK && o[0] == 4 && o[1] == 4 && o[2] == 4 && o[3] == 176);
    EXPECT(arf_get_plan(8, 0, 4096, ARF_BF16, 256, o) == ARF_OK && o[0] == 4 && o[3] == 64);
    EXPECT(arf_get_plan(8, (int64_t(1) << 31) - 1, 4096, ARF_BF16, 256, o) == ARF_OK && o[0] == 2);
    EXPECT(arf_get_plan(8, 100, 18016, ARF_BF16, 256, o) == ARF_OK && o[0] == 4 && o[1] == 16 && o[2] == 4);
    EXPECT(arf_set_path_override(2, 0, 0) == ARF_OK);
    EXPECT(arf_get_plan(8, 100, 65536, ARF_BF16, 256, o) == ARF_OK && o[0] == 2 && o[1] == 16 && o[2] == 8);
    EXPECT(arf_set_path_override(4, 0, 0) == ARF_OK);
    EXPECT(arf_set_path_override(4, 16, 8) == ARF_OK);
    EXPECT(arf_get_plan(3, 100, 65536, ARF_BF16, 256, o) == ARF_OK && o[0] == 4 && o[1] == 16 && o[2] == 8);
    EXPECT(arf_get_plan(3, 100, 65544, ARF_BF16, 256, o) == ARF_ERR_SHAPE);
    const int bad[][3] = {{5, 0, 0}, {-1, 0, 0}, {0, 4, 0}, {0, 0, 2}, {1, 8, 0}, {2, 3, 0}, {2, 4, 3}, {2, 32, 1}, {3, 16, 0}, {3, 0, 3}, {4, 2, 0}, {4, 0, 3}};
    for (const auto& v : bad) EXPECT(arf_set_path_override(v[0], v[1], v[2]) == ARF_ERR_VALUE);
    EXPECT(arf_set_path_override(0, 0, 0) == ARF_OK);
    EXPECT(arf_get_plan(8, 8192, 16384, ARF_BF16, 256, o) == ARF_OK && o[0] == 4 && o[1] == 4 && o[2] == 8 && o[3] == 8704);
    EXPECT(arf_get_plan(8, 2047, 16384, ARF_BF16, 256, o) == ARF_OK && o[0] == 2);
    EXPECT(arf_get_plan(8, 4096, 8192, ARF_BF16, 256, o) == ARF_OK && o[0] == 4);
    EXPECT(arf_get_plan(8, 8191, 4096, ARF_BF16, 256, o) == ARF_OK && o[0] == 2);
    EXPECT(arf_get_plan(8, 8192, 4096, ARF_BF16, 256, o) == ARF_OK && o[0] == 4 && o[3] == 8704);
    EXPECT(arf_get_plan(8, 8192, 2048, ARF_BF16, 256, o) == ARF_OK && o[0] == 4 && o[2] == 1 && o[3] == 8704);
    EXPECT(arf_get_plan(4, 16384, 2048, ARF_BF16, 256, o) == ARF_OK && o[0] == 1);   // 28 KiB per row
    EXPECT(arf_get_plan(16, 16384, 1024, ARF_BF16, 256, o) == ARF_OK && o[0] == 1);  // 128 chunks
    EXPECT(arf_get_plan(4, 8192, 8192, ARF_BF16, 256, o) == ARF_OK && o[0] == 4 && o[3] == 8704);
    EXPECT(arf_get_plan(4, 8192, 7168, ARF_F32, 256, o) == ARF_OK && o[0] == 4 && o[3] == 8704);
    // held rows by default only in their measured range
    EXPECT(arf_get_plan(4, 2048, 7168, ARF_F32, 256, o) == ARF_OK && o[0] == 3 && o[2] == 4 && o[3] == 256);
    EXPECT(arf_get_plan(8, 2048, 7168, ARF_BF16, 256, o) == ARF_OK && o[0] == 3 && o[1] == 8);
    EXPECT(arf_get_plan(8, 2048, 7168, ARF_F32, 256, o) == ARF_OK && o[0] == 3 && o[1] == 4);
    EXPECT(arf_get_plan(16, 2048, 7168, ARF_F32, 256, o) == ARF_OK && o[0] != 3);
    EXPECT(arf_get_plan(4, 767, 7168, ARF_F32, 256, o) == ARF_OK && o[0] == 2);
    EXPECT(arf_get_plan(4, 1536, 7168, ARF_F32, 256, o) == ARF_OK && o[0] == 3);
    EXPECT(arf_get_plan(4, 4096, 7168, ARF_F32, 256, o) == ARF_OK && o[0] == 4);   // two batches: claimed rows
    EXPECT(arf_get_plan(2, 4096, 4096, ARF_BF16, 256, o) == ARF_OK && o[0] == 3);
    EXPECT(arf_get_plan(2, 4096, 4088, ARF_BF16, 256, o) == ARF_OK && o[0] != 3);
    EXPECT(arf_get_plan(2, 4864, 4096, ARF_BF16, 256, o) == ARF_OK && o[0] == 3);   // 19 rows per CU fit
    EXPECT(arf_get_plan(2, 4865, 4096, ARF_BF16, 256, o) == ARF_OK && o[0] != 3);

    std::printf("%s %d checks, %d failed%s\n", g_fail ? "FAILED" : "ok", g_checks, g_fail,
                have_device ? " (device present: launching calls skipped)" : "");
    return g_fail ? 1 : 0;
}
