/* Drives every oracle entry point on small seeded inputs, for an ASan/UBSan build
 * (tests/test_oracle_sanitized.py). Exit status 0 and a line "ok <checksum>" on success.
 * Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/arf_oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return state;
}
static float uni(void) { return (float)((next() >> 11) * (1.0 / 9007199254740992.0)) * 4.0f - 2.0f; }

static uint64_t sum_bytes(const void* p, size_t n)
{
    const uint8_t* b = (const uint8_t*)p;
    uint64_t h = 1469598103934665603ull;
    for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 1099511628211ull;
    return h;
}

int main(void)
{
    const int32_t N = 5, H = 96;
    const int64_t T = 7;
    uint64_t check = 0;
    for (int32_t pdt = 0; pdt < 3; ++pdt) {
        for (int32_t adt = 0; adt < 2; ++adt) {
            if (pdt != adt && pdt != ARFO_F32) continue;
            const size_t sp = pdt == ARFO_F32 ? 4 : 2;
            void* part = malloc((size_t)N * T * H * sp);
            uint16_t* res = malloc((size_t)T * H * 2);
            uint16_t* gam = malloc((size_t)H * 2);
            uint16_t* rout = malloc((size_t)T * H * 2);
            uint16_t* nout = malloc((size_t)T * H * 2);
            uint8_t* q = malloc((size_t)T * H);
            float* sc = malloc((size_t)T * 4);
            uint8_t* mxs = malloc((size_t)T * H / 32);
            for (int64_t i = 0; i < (int64_t)N * T * H; ++i) {
                float v = uni();
                if (pdt == ARFO_F32) ((float*)part)[i] = v;
                else ((uint16_t*)part)[i] = pdt == ARFO_BF16 ? arfo_f32_to_bf16(v) : arfo_f32_to_f16(v);
            }
            for (int64_t i = 0; i < T * H; ++i)
                res[i] = adt == ARFO_BF16 ? arfo_f32_to_bf16(uni()) : arfo_f32_to_f16(uni());
            for (int32_t i = 0; i < H; ++i)
                gam[i] = adt == ARFO_BF16 ? arfo_f32_to_bf16(1.0f + 0.25f * uni())
                                          : arfo_f32_to_f16(1.0f + 0.25f * uni());
            const float scale = 0.01f;
            for (int32_t mode = -1; mode <= ARFO_MXFP4; ++mode) {
                for (int32_t acc = 0; acc < 2; ++acc) {
                    for (int32_t thr = 1; thr <= 3; thr += 2) {
                        arfo_args a = {part, N, T, H, pdt, adt, acc, 1, 5, res, rout, gam,
                                       1e-6f, nout, mode < 0 ? NULL : q, mode, &scale,
                                       mode == ARFO_MXFP4 ? (void*)mxs : (void*)sc, thr};
                        memset(rout, 0, (size_t)T * H * 2);
                        memset(nout, 0, (size_t)T * H * 2);
                        if (arfo_run(&a) != 0) { printf("arfo_run failed\n"); return 1; }
                        check ^= sum_bytes(rout, (size_t)T * H * 2) + 3 * sum_bytes(nout, (size_t)T * H * 2);
                    }
                }
            }
            if (arfo_reduce_rows(part, N, T, H, pdt, adt, ARFO_ACC_PARTIAL, 2, -1, rout, 2) != 0) {
                printf("arfo_reduce_rows failed\n");
                return 1;
            }
            check ^= sum_bytes(rout, (size_t)T * H * 2);
            if (arfo_reduce_add_rmsnorm(part, N, T, H, pdt, adt, res, res, gam, 0.0f, nout, 4) != 0 ||
                arfo_reduce_add_rmsnorm_quant(part, N, T, H, pdt, adt, res, NULL, gam, 1e-5f, NULL,
                                              q, ARFO_PER_TOKEN, NULL, sc, 2) != 0) {
                printf("wrapper failed\n");
                return 1;
            }
            check ^= sum_bytes(q, (size_t)T * H);
            free(part); free(res); free(gam); free(rout); free(nout); free(q); free(sc); free(mxs);
        }
    }
    for (int v = 0; v < 70000; ++v) {   /* every 16-bit pattern through the decoders */
        check += (uint64_t)arfo_f32_to_e4m3(arfo_bf16_to_f32((uint16_t)v));
        check += (uint64_t)arfo_f32_to_e2m1(arfo_f16_to_f32((uint16_t)v));
        check += (uint64_t)arfo_mx_scale_code(arfo_bf16_to_f32((uint16_t)(v & 0x7FFF)));
    }
    printf("ok %llu\n", (unsigned long long)check);
    return 0;
}
