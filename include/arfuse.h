/*
 * arfuse.h -- C ABI of libarfuse: the fused epilogue of a tensor-parallel all-reduce on
 * one MI355X (gfx950), at one GPU's share: N per-rank partial hidden states that are
 * already resident in local HBM are summed in rank order, added to the residual,
 * RMS-normalised, and written out (plus an optional OCP fp8-e4m3 copy).
 *
 * The operation is the one defined on the TensorRT-LLM page "allReduceFusionKernels.cu":
 *   - allreduce_sum, fp32-accumulation branch (the default chosen by use_fp32_acc):
 *     acc = float(p[0]); acc += float(p[r]) for r = 1..N-1; s = cast to the activation
 *     type;
 *   - fused_op / add128: r = s + residual_in, formed in the activation type; written
 *     as residual_out;
 *   - rms_norm: inv = 1/sqrt(sum(r^2)/hidden + eps); y = (r * inv) * gamma, cast to the
 *     activation type; written as norm_out;
 *   - the partials buffer is the oneshot-sync kernel's local receive buffer: shard r of
 *     token t at offset (r*tokens + t)*hidden elements (also the FlashInfer page for
 *     trtllm_create_ipc_workspace_for_all_reduce_fusion: tp_size x tokens x hidden
 *     elements, 2-byte or, with use_fp32_lamport, 4-byte).
 * The page's quantised output is a 4-bit format whose definition is not on the pages;
 * this library writes OCP E4M3 codes instead (round to nearest even, saturating to
 * +-448) of q = y * (1/scale), with a per-tensor scale given by the caller or a per-token
 * scale max|y|/448 computed here.
 *
 * Conventions for every entry point below:
 *   - Buffers are DEVICE pointers owned by the caller; the library allocates nothing and
 *     never synchronises. Its only state is a per-device compute-unit count, the test-only
 *     override below, and the row-claim counters of large launches: a file-scope device
 *     array of 256 slots of four 256-byte counters (256 KiB per device, no allocation),
 *     one slot per stream on first use and for the life of the process (a new stream that
 *     gets a destroyed stream's handle gets its slot too: hipStreamDestroy completes the
 *     stream's pending work first on ROCm). A launch with claimed rows leaves its counters
 *     at 0. Calls on one stream run one after another and share its slot; calls on
 *     different streams never share one. A call enqueued under stream capture, on the
 *     per-thread default stream, on a stream of another device, or once every slot
 *     belongs to another stream, takes the same kernel with rows by workgroup index
 *     instead (the same outputs, bit for bit).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). On ARF_OK one kernel
 *     has been enqueued on it (none when tokens == 0; several, in row order, when a
 *     one-row-per-workgroup or one-row-per-wavefront grid would exceed the 2^32 - 1
 *     work-items of one dispatch, which takes tens of millions of rows). Kernel faults
 *     surface at the caller's next synchronisation, as usual in HIP.
 *   - All arguments are validated before any HIP call: on any error status nothing is
 *     enqueued and nothing is written. Sizes, types and eps are checked first; a call
 *     with tokens == 0 is then complete (ARF_OK) and its pointers are not examined.
 *   - Thread-safe and reentrant (arf_set_path_override excepted).
 */
#ifndef ARFUSE_H
#define ARFUSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ARF_VERSION 400 /* 0.4.0 */

/* Element types (arguments typed int32_t take these values). */
#define ARF_BF16 0
#define ARF_F16 1
#define ARF_F32 2

/* Accumulation of the shards (allreduce_sum on the TensorRT-LLM page has both):
   ARF_ACC_F32: fp32 adds in rank order, one cast at the end (the page's default);
   ARF_ACC_PARTIAL: every partial sum is rounded to the partial type (add128 in DType);
   identical to ARF_ACC_F32 for fp32 partials. */
#define ARF_ACC_F32 0
#define ARF_ACC_PARTIAL 1

/* Quantised-copy modes (ARF_QUANT_NONE: no copy, for arf_get_plan_quant only). */
#define ARF_QUANT_NONE (-1)
#define ARF_QUANT_PER_TENSOR 0 /* fp8-e4m3, y ~ code * scale_in[0], scale given by the caller */
#define ARF_QUANT_PER_TOKEN 1  /* fp8-e4m3, scale_out[t] = max_i |y[t][i]| / 448, written    */
#define ARF_QUANT_MXFP4 2      /* OCP MXFP4 (arf_fused_epilogue only): blocks of 32 E2M1
                                  codes sharing an E8M0 scale, see arf_params              */

/* Limits. */
#define ARF_MAX_SHARDS 16
#define ARF_MAX_HIDDEN 65536

typedef enum arf_status {
    ARF_OK = 0,
    ARF_ERR_NULL = 1,      /* a required pointer is NULL                                  */
    ARF_ERR_SHAPE = 2,     /* n_shards not in 1..16, tokens < 0 or > 2^31-1, hidden not a
                              positive multiple of 8 or above ARF_MAX_HIDDEN, or a row
                              range outside [0, tokens)                                    */
    ARF_ERR_DTYPE = 3,     /* act_dtype not BF16/F16, or partial_dtype neither act_dtype
                              nor F32                                                      */
    ARF_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned (scales: 4-byte)      */
    ARF_ERR_ALIAS = 5,     /* an output overlaps another buffer (the only overlap allowed
                              is residual_out == residual_in exactly)                      */
    ARF_ERR_NO_OUTPUT = 6, /* residual_out and norm_out are both NULL (non-quant entry)    */
    ARF_ERR_VALUE = 7,     /* eps negative or not finite; unknown quant or accumulation
                              mode; bad override; wrong struct_size                        */
    ARF_ERR_HIP = 8        /* no usable device, or the kernel launch failed               */
} arf_status;

/*
 * Fused rank-order reduce + residual add + RMSNorm.
 *   partials      [n_shards][tokens][hidden] of partial_dtype, dense (shard stride
 *                 tokens*hidden elements), 16-byte aligned.
 *   n_shards      1..16 (the tensor-parallel degree).
 *   tokens        rows, >= 0; 0 is a valid empty call (ARF_OK, nothing enqueued).
 *   hidden        elements per row, a multiple of 8, at most ARF_MAX_HIDDEN.
 *   partial_dtype ARF_F32 or act_dtype (fp32 partials are the page's fp32-buffer option).
 *   act_dtype     ARF_BF16 or ARF_F16: type of residual_in/out, gamma and norm_out.
 *   residual_in   [tokens][hidden], read.
 *   residual_out  [tokens][hidden], written, nullable; may be equal to residual_in.
 *   gamma         [hidden], read.
 *   eps           >= 0 and finite, added to the mean of squares inside the root.
 *   norm_out      [tokens][hidden], written, nullable.
 * At least one of residual_out and norm_out must be non-NULL.
 */
arf_status arf_reduce_add_rmsnorm(const void* partials, int32_t n_shards, int64_t tokens,
                                  int32_t hidden, int32_t partial_dtype, int32_t act_dtype,
                                  const void* residual_in, void* residual_out,
                                  const void* gamma, float eps, void* norm_out,
                                  void* stream);

/*
 * The same, plus the fp8 copy of the normalised output (the page's quantised-output
 * pattern, with OCP E4M3 in place of its 4-bit format):
 *   residual_out, norm_out  nullable, both may be NULL.
 *   quant_out  [tokens][hidden] uint8 E4M3 codes of y * (1/scale), written, required.
 *   mode       ARF_QUANT_PER_TENSOR: scale_in (device, 1 float) is read; scale_out is
 *              ignored and may be NULL. A scale that is not > 0 gives all-zero codes.
 *              ARF_QUANT_PER_TOKEN: scale_out (device, [tokens] floats) receives
 *              max|y[t]|/448 per token; scale_in is ignored and may be NULL.
 */
arf_status arf_reduce_add_rmsnorm_quant(const void* partials, int32_t n_shards,
                                        int64_t tokens, int32_t hidden,
                                        int32_t partial_dtype, int32_t act_dtype,
                                        const void* residual_in, void* residual_out,
                                        const void* gamma, float eps, void* norm_out,
                                        uint8_t* quant_out, int32_t mode,
                                        const float* scale_in, float* scale_out,
                                        void* stream);

/*
 * General form of the two calls above, mirroring the page's parameter block
 * (AllReduceFusionParams): the same buffers, plus
 *   struct_size  must be sizeof(arf_params) (a newer or older layout is ARF_ERR_VALUE);
 *   row_begin,   rows [row_begin, row_begin + row_count) are computed (row_count < 0:
 *   row_count    through row tokens-1). Every buffer keeps its full [tokens] layout, the
 *                partials their shard stride tokens*hidden; rows outside the range are
 *                neither read nor written. 0 <= row_begin <= tokens.
 *   accumulate   ARF_ACC_F32 or ARF_ACC_PARTIAL.
 *   quant_out    NULL for no quantised copy; else quant_mode, scale_in and scale_out as
 *                in arf_reduce_add_rmsnorm_quant, or quant_mode ARF_QUANT_MXFP4 (OCP
 *                Microscaling Formats v1.0, the 4-bit format that the page's quantised
 *                output stands for here): hidden must be a multiple of 32;
 *                quant_out [tokens][hidden/2] bytes, two E2M1 codes each (element 2k in
 *                the low nibble, 16-byte aligned); scale_out [tokens][hidden/32] uint8
 *                E8M0 codes, X = 2^(code - 127) = 2^(floor(log2 max|y|) - 2) per block of
 *                32 (code 0 for an all-zero block); codes = E2M1(y / X), round to nearest
 *                even, saturating at +-6. E2M1 has no NaN or infinity: NaN and +-inf give
 *                +-6 (code 7 with the sign bit); NaN elements do not enter max|y|.
 */
typedef struct arf_params {
    uint32_t struct_size;
    int32_t n_shards;
    const void* partials;
    int64_t tokens;
    int64_t row_begin;
    int64_t row_count;
    int32_t hidden;
    int32_t partial_dtype;
    int32_t act_dtype;
    int32_t accumulate;
    const void* residual_in;
    void* residual_out;
    const void* gamma;
    float eps;
    void* norm_out;
    uint8_t* quant_out;
    int32_t quant_mode;
    const float* scale_in;
    void* scale_out;
} arf_params;

arf_status arf_fused_epilogue(const arf_params* params, void* stream);

/*
 * Reduce only: one rank's share of the token-slice (twoshot) exchange on the TensorRT-LLM
 * page, where a rank reduces its slice of tokens, all ranks exchange the reduced values,
 * and each then runs the epilogue over all tokens (arf_reduce_add_rmsnorm with
 * n_shards = 1 on the gathered values gives exactly the oneshot result).
 *   sums_out  [tokens][hidden] act_dtype: rows [row_begin, row_begin + row_count) receive
 *             the reduced value cast to act_dtype (the page's slice: tokens/N rows per
 *             rank, the first tokens%N ranks one more). Other arguments as in
 *             arf_fused_epilogue.
 */
arf_status arf_reduce_rows(const void* partials, int32_t n_shards, int64_t tokens,
                           int64_t row_begin, int64_t row_count, int32_t hidden,
                           int32_t partial_dtype, int32_t act_dtype, int32_t accumulate,
                           void* sums_out, void* stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* arf_status_string(int32_t status);

/* ARF_VERSION of the loaded library. */
int32_t arf_version(void);

/*
 * Launch geometry that a call with these sizes and no quantised copy would use, without a
 * device call when num_cus > 0 (then 160 KiB of LDS per workgroup is assumed; num_cus <= 0:
 * the current device's compute-unit count and LDS size are queried, which may return
 * ARF_ERR_HIP). out[0] = path: 1 row per wavefront, 2 row per workgroup, 3 held rows (one
 * workgroup per compute unit reads a batch of rows, keeping each row's rounded residual in
 * LDS, then writes their outputs), 4 row per workgroup with the rows past the first W
 * workgroups per compute unit claimed from 1, 2 or 4 counters in the order the
 * workgroups start (W = 2 workgroups per compute unit, or 4 for rows of less than 96 KiB
 * of traffic; a call that may not claim, see the conventions above, runs path 2 with a
 * grid of one workgroup per row); out[1] = wavefronts per workgroup; out[2] = 16-byte
 * chunks (8 elements) per lane; out[3] = workgroups in the grid (as an unsigned 32-bit
 * value; path 4: the rows plus max(64, rows/16) workgroups that find no row, rounded up
 * so that every counter has as many claimants). Honours arf_set_path_override.
 */
arf_status arf_get_plan(int32_t n_shards, int64_t tokens, int32_t hidden,
                        int32_t partial_dtype, int32_t num_cus, int32_t* out);

/*
 * The same for a call with the quantised copy `quant_mode` (ARF_QUANT_NONE, which gives
 * arf_get_plan's answer, ARF_QUANT_PER_TENSOR, ARF_QUANT_PER_TOKEN or ARF_QUANT_MXFP4; any
 * other value: ARF_ERR_VALUE; MXFP4 with hidden % 32 != 0: ARF_ERR_SHAPE). The plan depends on
 * the copy where the held rows (path 3) are concerned: they take no per-token copy, and a
 * per-tensor or MXFP4 one in most of their range.
 */
arf_status arf_get_plan_quant(int32_t n_shards, int64_t tokens, int32_t hidden,
                              int32_t partial_dtype, int32_t quant_mode, int32_t num_cus,
                              int32_t* out);

/*
 * TEST AND TUNING ONLY; process-wide, not to be changed while other threads call the
 * library. path 0 = automatic (the other two arguments must be 0); 1 = one row per
 * wavefront; 2 = one row per workgroup, rows by workgroup index; 3 = held rows (rows of up
 * to 16384 elements; 4 or 8 wavefronts, 8 only for 16-bit partials, the automatic choice
 * there; arf_reduce_rows keeps its automatic plan);
 * 4 = one row per workgroup with EVERY row claimed from the stream's counters (4 of them
 * for rows of less than 96 KiB of traffic, 2 below 256 KiB, else 1; where a call may
 * claim; a grid beyond one dispatch runs path 2). waves_per_block (paths 2 and 4: 4, 8
 * or 16; path 3: 4 or 8; path 1: 4) and chunks_per_lane (1, 2, 4 or 8) force the geometry when
 * non-zero. A forced geometry that cannot cover a call's hidden size makes that call return
 * ARF_ERR_VALUE. Returns ARF_ERR_VALUE for values outside these sets.
 */
arf_status arf_set_path_override(int32_t path, int32_t waves_per_block,
                                 int32_t chunks_per_lane);

/*
 * The quantiser's conversion alone, for testing it: out[i] = E4M3 code of in[i], round
 * to nearest even, saturating to +-448, NaN -> S.1111.111 (OCP OFP8 E4M3). in and out
 * are device pointers (in 4-byte aligned), n >= 0 elements. One kernel on `stream`.
 */
arf_status arf_e4m3_encode(const float* in, uint8_t* out, int64_t n, void* stream);

/*
 * The MXFP4 copy's element conversion alone, for testing it: out[i] = E2M1 code of in[i] in
 * the low nibble (OCP MX FP4: round to nearest even over 0, 0.5, 1, 1.5, 2, 3, 4, 6,
 * saturating to +-6, infinities and NaN to +-6, sign in bit 3), with no block scale. in and
 * out are device pointers (in 4-byte aligned), n >= 0 elements. One kernel on `stream`.
 */
arf_status arf_e2m1_encode(const float* in, uint8_t* out, int64_t n, void* stream);

/*
 * Streaming copy of `bytes` bytes (a multiple of 16; both pointers 16-byte aligned, the
 * ranges must not overlap) with the same load/store forms as the fused kernel: the
 * measured HBM ceiling and the calibration kernel for the byte counters.
 */
arf_status arf_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);

/*
 * Streaming probe with a chosen read/write mix, for the HBM ceiling of a traffic pattern:
 * reads read_bytes from src and writes write_bytes to dst, with no arithmetic, in `units`
 * work units (one workgroup each). Unit u reads its share of src in order, then writes
 * its share of dst with values derived from what it read, the way a row of the fused
 * kernel reads its inputs before writing its outputs. Byte counts are multiples of 16
 * (either may be 0); pointers 16-byte aligned; the ranges must not overlap; units <= 0
 * picks one unit per 16 KiB of the smaller non-zero side. dst receives unspecified bytes.
 */
arf_status arf_stream_mix(void* dst, int64_t write_bytes, const void* src, int64_t read_bytes,
                          int64_t units, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ARFUSE_H */
