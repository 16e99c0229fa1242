/*
 * c_abi_consumer.c -- a plain C99 program that uses libarfuse through include/arfuse.h
 * alone (test infrastructure: it also links the CPU oracle to check the results).
 *
 *   c_abi_consumer cpu   status strings and argument checks through the C ABI; no device
 *                        work (every call is rejected before the library touches HIP)
 *   c_abi_consumer gpu   device buffers from hipMalloc, the fused calls on the legacy
 *                        default stream and on a stream created here, every output
 *                        compared with the oracle's: residual_out bit for bit, norm_out
 *                        within 1 ulp, fp8 codes within 1 code, per-token scales bit for
 *                        bit in the rows whose norm_out is
 *
 * Inputs are drawn from splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", 2014) and built directly as bit patterns of the element type, so no
 * conversion arithmetic sits between the generator and either side.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "arf_oracle.h"
#include "arfuse.h"

static int failures = 0;

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            printf("FAIL %s:%d: ", __FILE__, __LINE__);   \
            printf(__VA_ARGS__);                          \
            printf("\n");                                 \
            ++failures;                                   \
        }                                                 \
    } while (0)

static uint64_t splitmix64(uint64_t* s) {
    uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* 16-bit values with a random sign, exponent in [e_lo, e_lo + 7] and random mantissa:
   bf16 (7 mantissa bits) or fp16 (10 mantissa bits). */
static void fill16(uint16_t* x, size_t n, uint64_t seed, int act_dtype, int e_lo, int positive) {
    const int mbits = act_dtype == ARF_BF16 ? 7 : 10;
    for (size_t i = 0; i < n; ++i) {
        const uint64_t r = splitmix64(&seed);
        const uint32_t sign = positive ? 0u : (uint32_t)(r & 1u);
        const uint32_t e = (uint32_t)e_lo + (uint32_t)((r >> 1) & 7u);
        const uint32_t m = (uint32_t)(r >> 8) & ((1u << mbits) - 1u);
        x[i] = (uint16_t)((sign << 15) | (e << mbits) | m);
    }
}

/* fp32 values: random sign, exponent 2^-8 .. 2^0, random 23-bit mantissa. */
static void fill32(uint32_t* x, size_t n, uint64_t seed) {
    for (size_t i = 0; i < n; ++i) {
        const uint64_t r = splitmix64(&seed);
        x[i] = ((uint32_t)(r & 1u) << 31) | ((119u + (uint32_t)((r >> 1) & 7u)) << 23) |
               ((uint32_t)(r >> 8) & 0x7FFFFFu);
    }
}

static int32_t ord16(uint16_t b) { return (b & 0x8000u) ? -(int32_t)(b & 0x7FFFu) : (int32_t)b; }
static int32_t ord8(uint8_t b) { return (b & 0x80u) ? -(int32_t)(b & 0x7Fu) : (int32_t)b; }

static void* dev_copy(const void* host, size_t bytes) {
    void* d = NULL;
    if (hipMalloc(&d, bytes) != hipSuccess) return NULL;
    if (host && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
    return d;
}

typedef struct {
    const char* name;
    int32_t n, hidden, pdt, adt, mode; /* mode < 0: no quantised copy */
    int64_t tokens;
    int in_place;                      /* residual_out == residual_in */
    int own_stream;                    /* a stream created here, else the legacy default */
    uint64_t seed;
} gpu_case;

static void run_case(const gpu_case* c) {
    const size_t th = (size_t)c->tokens * (size_t)c->hidden;
    const size_t sp = c->pdt == ARF_F32 ? 4 : 2;
    const size_t part_bytes = (size_t)c->n * th * sp;
    void* part = malloc(part_bytes);
    uint16_t* res = malloc(th * 2);
    uint16_t* gam = malloc((size_t)c->hidden * 2);
    if (!part || !res || !gam) { CHECK(0, "%s: host allocation", c->name); return; }
    if (c->pdt == ARF_F32) fill32((uint32_t*)part, (size_t)c->n * th, c->seed);
    else fill16((uint16_t*)part, (size_t)c->n * th, c->seed, c->adt, c->adt == ARF_BF16 ? 120 : 9, 0);
    fill16(res, th, c->seed + 1, c->adt, c->adt == ARF_BF16 ? 120 : 9, 0);
    fill16(gam, (size_t)c->hidden, c->seed + 2, c->adt, c->adt == ARF_BF16 ? 124 : 13, 1);
    const float eps = 1e-6f, scale_tensor = 0.0125f;

    /* the oracle, on the host */
    uint16_t* o_rout = malloc(th * 2);
    uint16_t* o_nout = malloc(th * 2);
    uint8_t* o_q = malloc(th);
    float* o_sc = malloc((size_t)c->tokens * 4);
    arfo_args a;
    memset(&a, 0, sizeof(a));
    a.partials = part; a.n_shards = c->n; a.tokens = c->tokens; a.hidden = c->hidden;
    a.partial_dtype = c->pdt; a.act_dtype = c->adt; a.accumulate = ARFO_ACC_F32;
    a.row_begin = 0; a.row_count = -1; a.residual_in = res; a.residual_out = o_rout;
    a.gamma = gam; a.eps = eps; a.norm_out = o_nout;
    a.quant_mode = c->mode < 0 ? -1 : (c->mode == ARF_QUANT_PER_TENSOR ? ARFO_PER_TENSOR : ARFO_PER_TOKEN);
    a.quant_out = c->mode < 0 ? NULL : o_q;
    a.scale_in = c->mode == ARF_QUANT_PER_TENSOR ? &scale_tensor : NULL;
    a.scale_out = c->mode == ARF_QUANT_PER_TOKEN ? o_sc : NULL;
    a.n_threads = 8;
    CHECK(arfo_run(&a) == ARFO_OK, "%s: oracle", c->name);

    /* the library, on the device */
    void* d_part = dev_copy(part, part_bytes);
    void* d_res = dev_copy(res, th * 2);
    void* d_gam = dev_copy(gam, (size_t)c->hidden * 2);
    void* d_rout = c->in_place ? d_res : dev_copy(NULL, th * 2);
    void* d_nout = dev_copy(NULL, th * 2);
    void* d_q = dev_copy(NULL, th);
    void* d_sc = dev_copy(NULL, (size_t)c->tokens * 4);
    void* d_sin = dev_copy(&scale_tensor, 4);
    if (!d_part || !d_res || !d_gam || !d_rout || !d_nout || !d_q || !d_sc || !d_sin) {
        CHECK(0, "%s: device allocation", c->name);
        return;
    }
    hipStream_t st = NULL;
    if (c->own_stream) CHECK(hipStreamCreate(&st) == hipSuccess, "%s: stream", c->name);
    arf_status s;
    if (c->mode < 0)
        s = arf_reduce_add_rmsnorm(d_part, c->n, c->tokens, c->hidden, c->pdt, c->adt, d_res,
                                   d_rout, d_gam, eps, d_nout, (void*)st);
    else
        s = arf_reduce_add_rmsnorm_quant(d_part, c->n, c->tokens, c->hidden, c->pdt, c->adt,
                                         d_res, d_rout, d_gam, eps, d_nout, (uint8_t*)d_q,
                                         c->mode, (const float*)d_sin, (float*)d_sc, (void*)st);
    CHECK(s == ARF_OK, "%s: %s", c->name, arf_status_string(s));
    CHECK(hipDeviceSynchronize() == hipSuccess, "%s: synchronise", c->name);

    uint16_t* g_rout = malloc(th * 2);
    uint16_t* g_nout = malloc(th * 2);
    uint8_t* g_q = malloc(th);
    float* g_sc = malloc((size_t)c->tokens * 4);
    CHECK(hipMemcpy(g_rout, d_rout, th * 2, hipMemcpyDeviceToHost) == hipSuccess, "copy");
    CHECK(hipMemcpy(g_nout, d_nout, th * 2, hipMemcpyDeviceToHost) == hipSuccess, "copy");
    CHECK(hipMemcpy(g_q, d_q, th, hipMemcpyDeviceToHost) == hipSuccess, "copy");
    CHECK(hipMemcpy(g_sc, d_sc, (size_t)c->tokens * 4, hipMemcpyDeviceToHost) == hipSuccess, "copy");

    size_t res_diff = 0, norm_off = 0, code_off = 0, scale_diff = 0;
    int32_t worst_norm = 0, worst_code = 0;
    for (int64_t t = 0; t < c->tokens; ++t) {
        int row_equal = 1;
        for (int32_t i = 0; i < c->hidden; ++i) {
            const size_t k = (size_t)t * (size_t)c->hidden + (size_t)i;
            if (g_rout[k] != o_rout[k]) ++res_diff;
            const int32_t dn = abs(ord16(g_nout[k]) - ord16(o_nout[k]));
            if (dn) row_equal = 0;
            if (dn > 1) ++norm_off;
            if (dn > worst_norm) worst_norm = dn;
            if (c->mode >= 0) {
                const int32_t dq = abs(ord8(g_q[k]) - ord8(o_q[k]));
                if (dq > 1) ++code_off;
                if (dq > worst_code) worst_code = dq;
            }
        }
        if (c->mode == ARF_QUANT_PER_TOKEN && row_equal &&
            memcmp(&g_sc[t], &o_sc[t], 4) != 0)
            ++scale_diff;
    }
    CHECK(res_diff == 0, "%s: residual_out differs in %zu elements", c->name, res_diff);
    CHECK(norm_off == 0, "%s: norm_out beyond 1 ulp in %zu elements", c->name, norm_off);
    CHECK(code_off == 0, "%s: fp8 codes beyond 1 code in %zu elements", c->name, code_off);
    CHECK(scale_diff == 0, "%s: %zu per-token scales differ", c->name, scale_diff);
    printf("case %s: %d x %lld x %d, residual bit-exact, norm_out max %d ulp, codes max %d\n",
           c->name, c->n, (long long)c->tokens, c->hidden, worst_norm, worst_code);
    fflush(stdout);

    if (st) hipStreamDestroy(st);
    hipFree(d_part); hipFree(d_res); hipFree(d_gam); hipFree(d_nout); hipFree(d_q);
    hipFree(d_sc); hipFree(d_sin);
    if (!c->in_place) hipFree(d_rout);
    free(part); free(res); free(gam); free(o_rout); free(o_nout); free(o_q); free(o_sc);
    free(g_rout); free(g_nout); free(g_q); free(g_sc);
}

static void cpu_checks(void) {
    static uint16_t buf[4][4 * 64] __attribute__((aligned(16)));
    static uint8_t q[4 * 64] __attribute__((aligned(16)));
    static float sc[4] __attribute__((aligned(16)));
    void *part = buf[0], *res = buf[1], *gam = buf[2], *out = buf[3];
    CHECK(arf_version() == ARF_VERSION, "version %d", (int)arf_version());
    for (int s = ARF_OK; s <= ARF_ERR_HIP; ++s) {
        const char* str = arf_status_string(s);
        CHECK(str && strlen(str) > 0, "status string %d", s);
    }
    /* rejected before any HIP call */
    CHECK(arf_reduce_add_rmsnorm(NULL, 1, 4, 64, ARF_BF16, ARF_BF16, res, out, gam, 1e-6f, NULL, NULL) == ARF_ERR_NULL, "null partials");
    CHECK(arf_reduce_add_rmsnorm(part, 1, 4, 60, ARF_BF16, ARF_BF16, res, out, gam, 1e-6f, NULL, NULL) == ARF_ERR_SHAPE, "hidden 60");
    CHECK(arf_reduce_add_rmsnorm(part, ARF_MAX_SHARDS + 1, 4, 64, ARF_BF16, ARF_BF16, res, out, gam, 1e-6f, NULL, NULL) == ARF_ERR_SHAPE, "17 shards");
    CHECK(arf_reduce_add_rmsnorm(part, 1, 4, 64, ARF_BF16, ARF_F32, res, out, gam, 1e-6f, NULL, NULL) == ARF_ERR_DTYPE, "fp32 activations");
    CHECK(arf_reduce_add_rmsnorm(part, 1, 4, 64, ARF_BF16, ARF_F16, res, out, gam, 1e-6f, NULL, NULL) == ARF_ERR_DTYPE, "bf16 partials, fp16 activations");
    CHECK(arf_reduce_add_rmsnorm(part, 1, 4, 64, ARF_BF16, ARF_BF16, res, out, gam, -1.0f, NULL, NULL) == ARF_ERR_VALUE, "negative eps");
    CHECK(arf_reduce_add_rmsnorm(part, 1, 4, 64, ARF_BF16, ARF_BF16, res, NULL, gam, 1e-6f, NULL, NULL) == ARF_ERR_NO_OUTPUT, "no output");
    CHECK(arf_reduce_add_rmsnorm((char*)part + 2, 1, 4, 64, ARF_BF16, ARF_BF16, res, out, gam, 1e-6f, NULL, NULL) == ARF_ERR_ALIGN, "misaligned partials");
    CHECK(arf_reduce_add_rmsnorm(part, 1, 4, 64, ARF_BF16, ARF_BF16, res, part, gam, 1e-6f, NULL, NULL) == ARF_ERR_ALIAS, "output over the partials");
    CHECK(arf_reduce_add_rmsnorm(NULL, 1, 0, 64, ARF_BF16, ARF_BF16, NULL, NULL, NULL, 1e-6f, NULL, NULL) == ARF_OK, "empty call");
    CHECK(arf_reduce_add_rmsnorm_quant(part, 1, 4, 64, ARF_BF16, ARF_BF16, res, out, gam, 1e-6f, NULL, q, 7, NULL, sc, NULL) == ARF_ERR_VALUE, "quant mode 7");
    CHECK(arf_reduce_add_rmsnorm_quant(part, 1, 4, 64, ARF_BF16, ARF_BF16, res, out, gam, 1e-6f, NULL, q, ARF_QUANT_PER_TOKEN, NULL, NULL, NULL) == ARF_ERR_NULL, "per-token without scale_out");
    CHECK(arf_set_path_override(5, 0, 0) == ARF_ERR_VALUE, "override path 5");
    CHECK(arf_set_path_override(0, 0, 0) == ARF_OK, "override reset");
    int32_t plan[4] = {0, 0, 0, 0};
    CHECK(arf_get_plan(8, 8192, 16384, ARF_BF16, 256, plan) == ARF_OK && plan[0] == 4, "plan of 8 x 8192 x 16384");
    CHECK(arf_get_plan(8, 8192, 2048, ARF_BF16, 256, plan) == ARF_OK && plan[0] == 4, "plan of 8 x 8192 x 2048");
    CHECK(arf_get_plan_quant(4, 2048, 7168, ARF_F32, ARF_QUANT_PER_TENSOR, 256, plan) == ARF_OK && plan[0] == 3, "per-tensor plan of 4 x 2048 x 7168");
    CHECK(arf_get_plan_quant(4, 2048, 7168, ARF_F32, ARF_QUANT_PER_TOKEN, 256, plan) == ARF_OK && plan[0] == 2, "per-token plan of 4 x 2048 x 7168");
    CHECK(arf_get_plan_quant(4, 2048, 7168, ARF_F32, ARF_QUANT_NONE, 256, plan) == ARF_OK && plan[0] == 3, "plan without a copy");
    CHECK(arf_get_plan_quant(4, 2048, 7168, ARF_F32, 9, 256, plan) == ARF_ERR_VALUE, "plan with copy mode 9");
    CHECK(arf_e2m1_encode(NULL, NULL, 0, NULL) == ARF_OK, "empty e2m1 conversion");
}

int main(int argc, char** argv) {
    if (argc != 2 || (strcmp(argv[1], "cpu") != 0 && strcmp(argv[1], "gpu") != 0)) {
        fprintf(stderr, "usage: %s cpu|gpu\n", argv[0]);
        return 2;
    }
    cpu_checks();
    if (strcmp(argv[1], "gpu") == 0) {
        static const gpu_case cases[] = {
            /* name, n, hidden, pdt, adt, mode, tokens, in_place, own_stream, seed */
            {"ragged fp16, per-tensor fp8", 2, 1032, ARF_F16, ARF_F16, ARF_QUANT_PER_TENSOR, 37, 0, 0, 101},
            {"bf16, per-token fp8, own stream", 8, 4096, ARF_BF16, ARF_BF16, ARF_QUANT_PER_TOKEN, 300, 0, 1, 202},
            {"fp32 partials 2048 x 7168, in place (held rows)", 4, 7168, ARF_F32, ARF_BF16, -1, 2048, 1, 0, 303},
            {"bf16 2048 x 16384, per-token fp8, own stream (claimed rows)", 8, 16384, ARF_BF16, ARF_BF16, ARF_QUANT_PER_TOKEN, 2048, 0, 1, 404},
            {"bf16 8192 x 2048, per-token fp8, own stream (claims over 4 counters)", 8, 2048, ARF_BF16, ARF_BF16, ARF_QUANT_PER_TOKEN, 8192, 0, 1, 505},
        };
        for (size_t i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i) {
            printf("running %s\n", cases[i].name);
            fflush(stdout);
            run_case(&cases[i]);
        }
    }
    if (failures) {
        printf("%d checks failed\n", failures);
        return 1;
    }
    printf("ok %s\n", argv[1]);
    return 0;
}
