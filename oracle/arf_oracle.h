/*
 * arf_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU implementation of the fused "sum the N tensor-parallel
 * partials, add the residual, RMS-normalise, optionally quantise to fp8-e4m3" epilogue.
 * It exists to check the HIP library against; no product code may link, load or call it.
 * It shares no source, header, table or helper with the HIP library.
 *
 * Method source: the TensorRT-LLM page "allReduceFusionKernels.cu" (functions
 * allreduce_sum, add128, rms_norm, fused_op and the oneshot-sync kernel's post-barrier
 * loop), the FlashInfer page for trtllm_create_ipc_workspace_for_all_reduce_fusion
 * (the [N][tokens][hidden] buffer shape and the fp32-partials option), and the OCP
 * 8-bit Floating Point Specification (OFP8) rev 1.0 for the E4M3 encoding.
 *
 * All pointers are HOST pointers owned by the caller. Functions return 0 on success and a
 * positive code on a bad argument (nothing is written in that case).
 */
#ifndef ARF_ORACLE_H
#define ARF_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types, as seen by the oracle. */
enum { ARFO_BF16 = 0, ARFO_F16 = 1, ARFO_F32 = 2 };
/* Accumulation of the shards: fp32 (the page's default), or in the partial type with a
   rounding after every addition (the page's other branch, add128 in DType). */
enum { ARFO_ACC_F32 = 0, ARFO_ACC_PARTIAL = 1 };
/* Quantised-copy modes: fp8-e4m3 with a per-tensor or per-token scale; OCP MXFP4 (E2M1
   elements in blocks of 32 sharing an E8M0 scale). */
enum { ARFO_PER_TENSOR = 0, ARFO_PER_TOKEN = 1, ARFO_MXFP4 = 2 };
/* Error codes. */
enum { ARFO_OK = 0, ARFO_ERR_NULL = 1, ARFO_ERR_SHAPE = 2, ARFO_ERR_DTYPE = 3, ARFO_ERR_VALUE = 4 };

/* Scalar conversions (round to nearest, ties to even). */
uint16_t arfo_f32_to_bf16(float x);   /* overflow -> +-inf, NaN -> quiet NaN          */
float    arfo_bf16_to_f32(uint16_t b);
uint16_t arfo_f32_to_f16(float x);    /* overflow -> +-inf, NaN -> quiet NaN          */
float    arfo_f16_to_f32(uint16_t h);
uint8_t  arfo_f32_to_e4m3(float x);   /* OCP E4M3, saturating to +-448, NaN -> S.1111.111 */
float    arfo_e4m3_to_f32(uint8_t q);
uint8_t  arfo_f32_to_e2m1(float x);   /* OCP MX FP4 E2M1 code (4 bits), saturating to +-6 */
float    arfo_e2m1_to_f32(uint8_t q);
/* OCP MX block scale of a block whose largest magnitude is amax (finite, >= 0): the
   E8M0 code 127 + clamp(floor(log2 amax) - 2, -127, 127); 0 for amax == 0. */
uint8_t  arfo_mx_scale_code(float amax);

/* Bulk conversions (n elements), for tests. */
void arfo_f32_to_bf16_n(const float* x, uint16_t* out, int64_t n);
void arfo_f32_to_f16_n(const float* x, uint16_t* out, int64_t n);
void arfo_f32_to_e4m3_n(const float* x, uint8_t* out, int64_t n);
void arfo_f32_to_e2m1_n(const float* x, uint8_t* out, int64_t n);

/*
 * partials     [n_shards][tokens][hidden] of partial_dtype (ARFO_BF16/F16/F32)
 * residual_in  [tokens][hidden] act_dtype (ARFO_BF16/F16)
 * residual_out [tokens][hidden] act_dtype, may be NULL, may equal residual_in
 * gamma        [hidden] act_dtype
 * norm_out     [tokens][hidden] act_dtype, may be NULL
 * n_threads    rows are split over this many threads (<=0 means 1); results do not
 *              depend on it.
 */
int arfo_reduce_add_rmsnorm(const void* partials, int32_t n_shards, int64_t tokens,
                            int32_t hidden, int32_t partial_dtype, int32_t act_dtype,
                            const void* residual_in, void* residual_out, const void* gamma,
                            float eps, void* norm_out, int32_t n_threads);

/*
 * The same, plus the fp8 copy of the normalised output:
 * quant_out  [tokens][hidden] E4M3 codes (required)
 * mode       ARFO_PER_TENSOR: scale_in[0] is the dequantisation scale (y ~ code * scale)
 *            ARFO_PER_TOKEN:  scale_out[t] = max_i |y[t][i]| / 448 is written per token
 */
int arfo_reduce_add_rmsnorm_quant(const void* partials, int32_t n_shards, int64_t tokens,
                                  int32_t hidden, int32_t partial_dtype, int32_t act_dtype,
                                  const void* residual_in, void* residual_out,
                                  const void* gamma, float eps, void* norm_out,
                                  uint8_t* quant_out, int32_t mode, const float* scale_in,
                                  float* scale_out, int32_t n_threads);

/*
 * General form. Rows [row_begin, row_begin + row_count) of the [tokens] rows are computed
 * (row_count < 0: to the end); every buffer keeps its full [tokens] layout and rows outside
 * the range are neither read nor written. quant_mode < 0: no quantised copy.
 */
typedef struct arfo_args {
    const void* partials;
    int32_t n_shards;
    int64_t tokens;
    int32_t hidden;
    int32_t partial_dtype;
    int32_t act_dtype;
    int32_t accumulate;
    int64_t row_begin;
    int64_t row_count;
    const void* residual_in;
    void* residual_out;
    const void* gamma;
    float eps;
    void* norm_out;
    uint8_t* quant_out;        /* MXFP4: [tokens][hidden/2], element 2k in the low nibble */
    int32_t quant_mode;
    const float* scale_in;
    void* scale_out;           /* per-token: float [tokens]; MXFP4: uint8 [tokens][hidden/32] */
    int32_t n_threads;
} arfo_args;

int arfo_run(const arfo_args* a);

/*
 * Reduce only (one rank's share of the token-slice exchange): sums_out[t][i] = the
 * reduced value cast to act_dtype, for rows t in [row_begin, row_begin + row_count).
 */
int arfo_reduce_rows(const void* partials, int32_t n_shards, int64_t tokens, int32_t hidden,
                     int32_t partial_dtype, int32_t act_dtype, int32_t accumulate,
                     int64_t row_begin, int64_t row_count, void* sums_out, int32_t n_threads);

#ifdef __cplusplus
}
#endif

#endif /* ARF_ORACLE_H */
