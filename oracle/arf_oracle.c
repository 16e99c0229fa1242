/*
 * arf_oracle.c -- TEST INFRASTRUCTURE ONLY (see arf_oracle.h).
 *
 * Plain scalar reference for the fused epilogue of the tensor-parallel all-reduce:
 * rank-ordered fp32 sum of the N partials, residual add, RMSNorm, optional fp8-e4m3 copy.
 * Only tests/, the smoke entry and the benchmark's CPU-baseline leg may load this code.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fPIC -shared -pthread (x86-64, SSE
 * arithmetic, so every `float` operation below is one IEEE binary32 operation with one
 * rounding, and no multiply-add is ever contracted).
 *
 * Step numbering (O1..O6) follows the order in which the method computes, per token t and
 * hidden index i. Sources:
 *   [SUM]   TensorRT-LLM page "allReduceFusionKernels.cu", function allreduce_sum,
 *           fp32-accumulation branch (the default per use_fp32_acc).
 *   [SUM-P] same function, other branch: the packs are added with add128 in DType, so
 *           every partial sum is rounded to the partial type.
 *   [ADD]   same page, fused_op and add128 (residual add in the activation type).
 *   [NORM]  same page, rms_norm.
 *   [LAYOUT] same page, oneshot-sync kernel post-barrier loop (shard r of a token's
 *           access at r * (tokens*hidden/8) + idx), and the FlashInfer page for
 *           trtllm_create_ipc_workspace_for_all_reduce_fusion (tp_size x tokens x hidden
 *           buffers; 4-byte elements with use_fp32_lamport).
 *   [OFP8]  OCP 8-bit Floating Point Specification (OFP8) rev 1.0, E4M3 encoding.
 *   [MX]    OCP Microscaling Formats (MX) v1.0: MXFP4 = blocks of 32 FP4 (E2M1) elements
 *           sharing one E8M0 scale X = 2^(floor(log2(max |V|)) - emax_elem), emax_elem = 2,
 *           elements quantised from V / X (round to nearest even, saturating).
 */
#include "arf_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* Rounding to a narrower binary format, from the definition.                           */
/* ------------------------------------------------------------------------------------ */

/*
 * Round the finite value x (which is an exact binary32 value, held in a double) to the
 * nearest value of a binary format with `mbits` stored mantissa bits and minimum normal
 * exponent `emin` (gradual underflow below it), ties to the even neighbour. The spacing
 * of representable values in the binade of x is 2^(max(floor(log2|x|), emin) - mbits);
 * dividing by that power of two is exact, nearbyint() rounds ties to even in the default
 * rounding mode, and multiplying back is exact. The result may be one binade up (carry)
 * and may exceed the format's largest finite value: the caller decides overflow.
 */
static double round_to_format(double x, int mbits, int emin)
{
    if (x == 0.0) return x;
    int e;
    (void)frexp(fabs(x), &e);  /* |x| = f * 2^e with f in [0.5, 1) */
    int ex = e - 1;            /* floor(log2 |x|) */
    if (ex < emin) ex = emin;
    double quantum = ldexp(1.0, ex - mbits);
    double r = nearbyint(x / quantum);
    return r * quantum;
}

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* bfloat16: 8 exponent bits (bias 127), 7 mantissa bits; a bf16 value is the top half of
   the binary32 value with the same number. Largest finite (2 - 2^-7) * 2^127. */
uint16_t arfo_f32_to_bf16(float x)
{
    uint32_t u = f32_bits(x);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);          /* quiet NaN */
    if (isinf(x)) return (uint16_t)(u >> 16);
    double r = round_to_format((double)x, 7, -126);
    const double maxf = ldexp(255.0, 120);                          /* (2-2^-7)*2^127 */
    if (fabs(r) > maxf) return (uint16_t)((u & 0x80000000u) ? 0xFF80u : 0x7F80u);
    /* r is exactly representable in binary32 with its low 16 bits zero */
    return (uint16_t)(f32_bits((float)r) >> 16) | (uint16_t)((u >> 16) & 0x8000u);
}

float arfo_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* IEEE binary16: 5 exponent bits (bias 15), 10 mantissa bits, emin = -14, largest finite
   65504, smallest subnormal 2^-24. */
uint16_t arfo_f32_to_f16(float x)
{
    uint32_t u = f32_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u | ((u >> 13) & 0x01FFu));
    if (isinf(x)) return (uint16_t)(sign | 0x7C00u);
    double r = fabs(round_to_format((double)x, 10, -14));
    if (r > 65504.0) return (uint16_t)(sign | 0x7C00u);
    if (r == 0.0) return sign;
    int e;
    (void)frexp(r, &e);
    int ex = e - 1;
    if (ex < -14) {                                   /* subnormal: r = m * 2^-24 */
        uint16_t m = (uint16_t)ldexp(r, 24);
        return (uint16_t)(sign | m);
    }
    uint16_t m = (uint16_t)(ldexp(r, -ex) * 1024.0 - 1024.0);
    return (uint16_t)(sign | ((uint16_t)(ex + 15) << 10) | m);
}

float arfo_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ef = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (ef == 0x1F) {
        if (m) return bits_f32(((uint32_t)sign << 31) | 0x7FC00000u | ((uint32_t)m << 13));
        v = INFINITY;
    } else if (ef == 0) {
        v = ldexp((double)m, -24);
    } else {
        v = ldexp((double)(1024 + m), ef - 25);
    }
    return (float)(sign ? -v : v);
}

/* OCP OFP8 E4M3 [OFP8]: 4 exponent bits (bias 7), 3 mantissa bits, emin = -6, no
   infinities, NaN = S.1111.111, largest finite 1.75 * 2^8 = 448, smallest subnormal
   2^-9. Conversion here is round-to-nearest-even with saturation: anything whose rounded
   magnitude exceeds 448 (including infinity) becomes +-448. */
uint8_t arfo_f32_to_e4m3(float x)
{
    uint8_t sign = (uint8_t)((f32_bits(x) >> 24) & 0x80u);
    if (isnan(x)) return (uint8_t)(sign | 0x7Fu);
    if (isinf(x)) return (uint8_t)(sign | 0x7Eu);
    double r = fabs(round_to_format((double)x, 3, -6));
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    int e;
    (void)frexp(r, &e);
    int ex = e - 1;
    if (ex < -6) {                                    /* subnormal: r = m * 2^-9 */
        uint8_t m = (uint8_t)ldexp(r, 9);
        return (uint8_t)(sign | m);
    }
    uint8_t m = (uint8_t)(ldexp(r, -ex) * 8.0 - 8.0);
    return (uint8_t)(sign | (uint8_t)((ex + 7) << 3) | m);
}

float arfo_e4m3_to_f32(uint8_t q)
{
    int sign = (q >> 7) & 1;
    int ef = (q >> 3) & 0xF;
    int m = q & 0x7;
    double v;
    if (ef == 0xF && m == 0x7) return bits_f32(((uint32_t)sign << 31) | 0x7FC00000u);
    if (ef == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), ef - 10);
    return (float)(sign ? -v : v);
}

/* OCP MX FP4 E2M1 [MX]: 2 exponent bits (bias 1), 1 mantissa bit, emin = 0, largest
   finite 1.5 * 2^2 = 6, smallest subnormal 0.5, no infinities or NaN. Round to nearest even,
   saturating to +-6 (infinities too; NaN is not produced by the method and maps to +-6). */
uint8_t arfo_f32_to_e2m1(float x)
{
    uint8_t sign = (uint8_t)((f32_bits(x) >> 28) & 0x8u);
    if (isnan(x) || isinf(x)) return (uint8_t)(sign | 0x7u);
    double r = fabs(round_to_format((double)x, 1, 0));
    if (r > 6.0) r = 6.0;
    if (r == 0.0) return sign;
    int e;
    (void)frexp(r, &e);
    int ex = e - 1;
    if (ex < 0) return (uint8_t)(sign | 0x1u);            /* subnormal: 0.5 */
    uint8_t m = (uint8_t)(ldexp(r, -ex) * 2.0 - 2.0);
    return (uint8_t)(sign | (uint8_t)((ex + 1) << 1) | m);
}

float arfo_e2m1_to_f32(uint8_t q)
{
    int sign = (q >> 3) & 1;
    int ef = (q >> 1) & 0x3;
    int m = q & 0x1;
    double v = ef == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, ef - 1);
    return (float)(sign ? -v : v);
}

uint8_t arfo_mx_scale_code(float amax)
{
    if (!(amax > 0.0f)) return 0;
    int e;
    (void)frexp((double)amax, &e);
    int shared = (e - 1) - 2;                             /* floor(log2 amax) - emax_elem */
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
    return (uint8_t)(shared + 127);
}

void arfo_f32_to_bf16_n(const float* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = arfo_f32_to_bf16(x[i]);
}
void arfo_f32_to_f16_n(const float* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = arfo_f32_to_f16(x[i]);
}
void arfo_f32_to_e4m3_n(const float* x, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = arfo_f32_to_e4m3(x[i]);
}

void arfo_f32_to_e2m1_n(const float* x, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = arfo_f32_to_e2m1(x[i]);
}

/* ------------------------------------------------------------------------------------ */
/* Element access.                                                                      */
/* ------------------------------------------------------------------------------------ */

static float act_to_f32(uint16_t v, int32_t act)
{
    return act == ARFO_BF16 ? arfo_bf16_to_f32(v) : arfo_f16_to_f32(v);
}

static uint16_t f32_to_act(float x, int32_t act)
{
    return act == ARFO_BF16 ? arfo_f32_to_bf16(x) : arfo_f32_to_f16(x);
}

static float partial_at(const void* p, int32_t dtype, int64_t idx)
{
    if (dtype == ARFO_F32) return ((const float*)p)[idx];
    return act_to_f32(((const uint16_t*)p)[idx], dtype);
}

/* ------------------------------------------------------------------------------------ */
/* One token (row).                                                                      */
/* ------------------------------------------------------------------------------------ */

typedef struct {
    const void* partials;
    int32_t n_shards;
    int64_t tokens;
    int32_t hidden;
    int32_t pdt, adt;
    int32_t acc;              /* ARFO_ACC_F32 | ARFO_ACC_PARTIAL */
    uint16_t* sums_out;       /* reduce only when non-NULL */
    const uint16_t* residual_in;
    uint16_t* residual_out;
    const uint16_t* gamma;
    float eps;
    uint16_t* norm_out;
    uint8_t* quant_out;       /* NULL when no quantised copy is asked for */
    int32_t mode;
    const float* scale_in;
    void* scale_out;
} job_t;

/* Round an fp32 value to the partial type (identity for fp32 partials). */
static float to_partial_type(float x, int32_t pdt)
{
    if (pdt == ARFO_F32) return x;
    return act_to_f32(f32_to_act(x, pdt), pdt);
}

/* O1-O2 for one element: the reduced value in the activation type. */
static uint16_t reduce_element(const job_t* j, int64_t shard_stride, int64_t idx)
{
    /* O1 [SUM]: start from rank 0's value and add ranks 1..N-1 one at a time, in fp32;
       or [SUM-P] in the partial type: each partial sum is rounded to that type. One fp32
       addition followed by one rounding to a p-bit type gives the correctly rounded sum
       of the two values, since 24 >= 2p + 2 (double rounding is innocuous). */
    float acc = partial_at(j->partials, j->pdt, idx);
    for (int32_t r = 1; r < j->n_shards; ++r) {
        acc = acc + partial_at(j->partials, j->pdt, (int64_t)r * shard_stride + idx);
        if (j->acc == ARFO_ACC_PARTIAL) acc = to_partial_type(acc, j->pdt);
    }
    /* O2 [SUM]: the reduced value is cast back to the activation type. */
    return f32_to_act(acc, j->adt);
}

static void one_token(const job_t* j, int64_t t, uint16_t* rrow, uint16_t* yrow)
{
    const int64_t H = j->hidden;
    const int64_t shard_stride = j->tokens * H;      /* [LAYOUT]: dense [N][T][H] */
    const int64_t row = t * H;

    if (j->sums_out) {
        for (int64_t i = 0; i < H; ++i) j->sums_out[row + i] = reduce_element(j, shard_stride, row + i);
        return;
    }
    for (int64_t i = 0; i < H; ++i) {
        uint16_t s = reduce_element(j, shard_stride, row + i);
        /* O3 [ADD]: residual add in the activation type: the exact sum of two 16-bit
           values, rounded once (one binary32 add is exact-then-rounded to 24 bits and a
           second rounding to 8 or 11 bits cannot differ from a direct one, since
           24 >= 2p + 2 for p = 8 and p = 11). */
        float sum = act_to_f32(s, j->adt) + act_to_f32(j->residual_in[row + i], j->adt);
        rrow[i] = f32_to_act(sum, j->adt);
    }
    if (j->residual_out)
        for (int64_t i = 0; i < H; ++i) j->residual_out[row + i] = rrow[i];

    /* O4 [NORM]: mean of squares of the ROUNDED residual, then 1/sqrt(mean + eps). The
       page sums squares in fp32 across threads and blocks (an implementation-defined
       order); here the sum is sequential in fp64 (each square of a 16-bit value is exact
       in fp64), and the inverse root is computed in fp64 and rounded once to fp32. */
    double ss = 0.0;
    for (int64_t i = 0; i < H; ++i) {
        double x = (double)act_to_f32(rrow[i], j->adt);
        ss += x * x;
    }
    float inv = (float)(1.0 / sqrt(ss / (double)H + (double)j->eps));

    /* O5 [NORM]: y = (x * inv) * gamma in fp32, cast to the activation type. */
    for (int64_t i = 0; i < H; ++i) {
        float x = act_to_f32(rrow[i], j->adt);
        float g = act_to_f32(j->gamma[i], j->adt);
        float v = x * inv;
        v = v * g;
        yrow[i] = f32_to_act(v, j->adt);
    }
    if (j->norm_out)
        for (int64_t i = 0; i < H; ++i) j->norm_out[row + i] = yrow[i];

    /* O6': MXFP4 copy of the cast normalised output [MX]: per block of 32 elements,
       X = 2^(floor(log2 max|y|) - 2) (E8M0), codes E2M1(y / X); y / X is a power-of-two
       scaling, exact in fp64. */
    if (j->quant_out && j->mode == ARFO_MXFP4) {
        uint8_t* qrow = j->quant_out + t * (H / 2);
        uint8_t* srow = (uint8_t*)j->scale_out + t * (H / 32);
        for (int64_t b = 0; b < H / 32; ++b) {
            float amax = 0.0f;
            for (int64_t i = 32 * b; i < 32 * b + 32; ++i) {
                float a = fabsf(act_to_f32(yrow[i], j->adt));
                if (a > amax) amax = a;
            }
            uint8_t code = arfo_mx_scale_code(amax);
            srow[b] = code;
            double inv_x = ldexp(1.0, 127 - (int)code);       /* 1 / 2^(code - 127) */
            for (int64_t i = 32 * b; i < 32 * b + 32; i += 2) {
                uint8_t lo = arfo_f32_to_e2m1((float)((double)act_to_f32(yrow[i], j->adt) * inv_x));
                uint8_t hi = arfo_f32_to_e2m1((float)((double)act_to_f32(yrow[i + 1], j->adt) * inv_x));
                qrow[i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
        return;
    }
    /* O6: fp8-e4m3 copy of the cast normalised output, v = y * (1/scale). */
    if (j->quant_out) {
        float scale;
        if (j->mode == ARFO_PER_TOKEN) {
            float amax = 0.0f;
            for (int64_t i = 0; i < H; ++i) {
                float a = fabsf(act_to_f32(yrow[i], j->adt));
                if (a > amax) amax = a;
            }
            scale = amax / 448.0f;
            ((float*)j->scale_out)[t] = scale;
        } else {
            scale = j->scale_in[0];
        }
        float inv_scale = scale > 0.0f ? 1.0f / scale : 0.0f;
        for (int64_t i = 0; i < H; ++i)
            j->quant_out[row + i] = arfo_f32_to_e4m3(act_to_f32(yrow[i], j->adt) * inv_scale);
    }
}

/* ------------------------------------------------------------------------------------ */
/* Row split over threads: contiguous blocks of tokens, one token per thread at a time. */
/* ------------------------------------------------------------------------------------ */

typedef struct {
    const job_t* job;
    int64_t t0, t1;
    int failed;
} slice_t;

static void* run_slice(void* arg)
{
    slice_t* s = (slice_t*)arg;
    const int64_t H = s->job->hidden;
    uint16_t* rrow = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
    uint16_t* yrow = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
    if (!rrow || !yrow) {
        s->failed = 1;
    } else {
        for (int64_t t = s->t0; t < s->t1; ++t) one_token(s->job, t, rrow, yrow);
    }
    free(rrow);
    free(yrow);
    return NULL;
}

static int run_job(const job_t* j, int64_t row_begin, int64_t row_count, int32_t n_threads)
{
    if (row_count == 0) return ARFO_OK;
    if (n_threads < 1) n_threads = 1;
    if ((int64_t)n_threads > row_count) n_threads = (int32_t)row_count;
    slice_t* sl = (slice_t*)calloc((size_t)n_threads, sizeof(slice_t));
    pthread_t* th = (pthread_t*)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!sl || !th) { free(sl); free(th); return ARFO_ERR_VALUE; }
    for (int32_t k = 0; k < n_threads; ++k) {
        sl[k].job = j;
        sl[k].t0 = row_begin + row_count * k / n_threads;
        sl[k].t1 = row_begin + row_count * (k + 1) / n_threads;
    }
    int failed = 0;
    for (int32_t k = 1; k < n_threads; ++k)
        if (pthread_create(&th[k], NULL, run_slice, &sl[k]) != 0) { sl[k].failed = 2; }
    run_slice(&sl[0]);
    for (int32_t k = 1; k < n_threads; ++k) {
        if (sl[k].failed == 2) run_slice(&sl[k]);     /* thread did not start: run here */
        else pthread_join(th[k], NULL);
    }
    for (int32_t k = 0; k < n_threads; ++k) failed |= sl[k].failed == 1;
    free(sl);
    free(th);
    return failed ? ARFO_ERR_VALUE : ARFO_OK;
}

static int check_common(const void* partials, int32_t n_shards, int64_t tokens,
                        int32_t hidden, int32_t pdt, int32_t adt, int32_t acc, float eps)
{
    if (!partials) return ARFO_ERR_NULL;
    if (n_shards < 1 || tokens < 0 || hidden < 1) return ARFO_ERR_SHAPE;
    if (adt != ARFO_BF16 && adt != ARFO_F16) return ARFO_ERR_DTYPE;
    if (pdt != ARFO_BF16 && pdt != ARFO_F16 && pdt != ARFO_F32) return ARFO_ERR_DTYPE;
    if (acc != ARFO_ACC_F32 && acc != ARFO_ACC_PARTIAL) return ARFO_ERR_VALUE;
    if (!(eps >= 0.0f) || isinf(eps)) return ARFO_ERR_VALUE;
    return ARFO_OK;
}

/* Resolve a row range against [0, tokens); returns 0 on success. */
static int resolve_rows(int64_t tokens, int64_t begin, int64_t count, int64_t* b, int64_t* c)
{
    if (begin < 0 || begin > tokens) return ARFO_ERR_SHAPE;
    if (count < 0) count = tokens - begin;
    if (count > tokens - begin) return ARFO_ERR_SHAPE;
    *b = begin;
    *c = count;
    return ARFO_OK;
}

int arfo_run(const arfo_args* a)
{
    if (!a) return ARFO_ERR_NULL;
    int rc = check_common(a->partials, a->n_shards, a->tokens, a->hidden, a->partial_dtype,
                          a->act_dtype, a->accumulate, a->eps);
    if (rc) return rc;
    if (!a->residual_in || !a->gamma) return ARFO_ERR_NULL;
    if (a->quant_mode < 0) {
        if (!a->residual_out && !a->norm_out) return ARFO_ERR_NULL;
    } else {
        if (!a->quant_out) return ARFO_ERR_NULL;
        if (a->quant_mode == ARFO_PER_TENSOR) {
            if (!a->scale_in) return ARFO_ERR_NULL;
        } else if (a->quant_mode == ARFO_PER_TOKEN) {
            if (!a->scale_out) return ARFO_ERR_NULL;
        } else if (a->quant_mode == ARFO_MXFP4) {
            if (!a->scale_out) return ARFO_ERR_NULL;
            if (a->hidden % 32 != 0) return ARFO_ERR_SHAPE;
        } else {
            return ARFO_ERR_VALUE;
        }
    }
    int64_t b, c;
    if ((rc = resolve_rows(a->tokens, a->row_begin, a->row_count, &b, &c))) return rc;
    job_t j = {a->partials, a->n_shards, a->tokens, a->hidden, a->partial_dtype, a->act_dtype,
               a->accumulate, NULL, (const uint16_t*)a->residual_in,
               (uint16_t*)a->residual_out, (const uint16_t*)a->gamma, a->eps,
               (uint16_t*)a->norm_out, a->quant_mode < 0 ? NULL : a->quant_out,
               a->quant_mode < 0 ? 0 : a->quant_mode, a->scale_in, a->scale_out};
    return run_job(&j, b, c, a->n_threads);
}

int arfo_reduce_rows(const void* partials, int32_t n_shards, int64_t tokens, int32_t hidden,
                     int32_t partial_dtype, int32_t act_dtype, int32_t accumulate,
                     int64_t row_begin, int64_t row_count, void* sums_out, int32_t n_threads)
{
    int rc = check_common(partials, n_shards, tokens, hidden, partial_dtype, act_dtype,
                          accumulate, 0.0f);
    if (rc) return rc;
    if (!sums_out) return ARFO_ERR_NULL;
    int64_t b, c;
    if ((rc = resolve_rows(tokens, row_begin, row_count, &b, &c))) return rc;
    job_t j = {partials, n_shards, tokens, hidden, partial_dtype, act_dtype, accumulate,
               (uint16_t*)sums_out, NULL, NULL, NULL, 0.0f, NULL, NULL, 0, NULL, NULL};
    return run_job(&j, b, c, n_threads);
}

int arfo_reduce_add_rmsnorm(const void* partials, int32_t n_shards, int64_t tokens,
                            int32_t hidden, int32_t partial_dtype, int32_t act_dtype,
                            const void* residual_in, void* residual_out, const void* gamma,
                            float eps, void* norm_out, int32_t n_threads)
{
    arfo_args a = {partials, n_shards, tokens, hidden, partial_dtype, act_dtype, ARFO_ACC_F32,
                   0, -1, residual_in, residual_out, gamma, eps, norm_out, NULL, -1, NULL,
                   NULL, n_threads};
    return arfo_run(&a);
}

int arfo_reduce_add_rmsnorm_quant(const void* partials, int32_t n_shards, int64_t tokens,
                                  int32_t hidden, int32_t partial_dtype, int32_t act_dtype,
                                  const void* residual_in, void* residual_out,
                                  const void* gamma, float eps, void* norm_out,
                                  uint8_t* quant_out, int32_t mode, const float* scale_in,
                                  float* scale_out, int32_t n_threads)
{
    if (mode != ARFO_PER_TENSOR && mode != ARFO_PER_TOKEN) {
        int rc = check_common(partials, n_shards, tokens, hidden, partial_dtype, act_dtype,
                              ARFO_ACC_F32, eps);
        return rc ? rc : ARFO_ERR_VALUE;
    }
    arfo_args a = {partials, n_shards, tokens, hidden, partial_dtype, act_dtype, ARFO_ACC_F32,
                   0, -1, residual_in, residual_out, gamma, eps, norm_out, quant_out, mode,
                   scale_in, scale_out, n_threads};
    return arfo_run(&a);
}
