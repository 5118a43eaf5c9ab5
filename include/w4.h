/*
 * w4.h -- C ABI of the int4-weight quantized linear layer for AMD Instinct
 * MI355X (gfx950). Shared library: libw4.so.
 *
 * Sources (cited by page title and symbol):
 *   [inc_w4a8]  vLLM docs page vllm.model_executor.layers.quantization.inc.
 *               schemes.inc_w4a8_linear, class INCXPUW4A8LinearMethod
 *   [ct_w4a8]   vLLM v0.10.1.1 docs page vllm.model_executor.layers.
 *               quantization.compressed_tensors.schemes.compressed_tensors_w4a8_int
 *   [w4afp8]    vLLM docs page vllm.model_executor.layers.quantization.w4afp8
 *   [zentorch]  vLLM docs page vllm.model_executor.kernels.linear.
 *               mixed_precision.zentorch, class ZentorchWNA16LinearKernel
 *   [cpu_int4]  vllm-omni page model_executor/layers/quantization/cpu_int4.py
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers; the caller allocates
 *     and owns every buffer. The library allocates nothing and keeps no state
 *     but the per-thread error message (and, for w4_linear_noalloc only, one
 *     device scratch array per GPU with its looked-up address).
 *   - `stream` is a hipStream_t (NULL: the default stream). Work is enqueued
 *     on it; no entry point synchronizes.
 *   - Arguments are validated before anything is enqueued. On failure the
 *     return value is a negative W4_ERR_* code and w4_last_error() names the
 *     offending argument and sizes; nothing was launched.
 *   - Sizes are element counts; matrices are row-major.
 *   - A weight code q in 0..15 stands for the integer q - 8 ("uint4b8": the
 *     zero point is the constant 8) [w4afp8] _repack_signed_int4_to_uint4b8;
 *     within a packed word the code with the lowest K index is in the lowest
 *     nibble ([cpu_int4] pack_nibbles; [zentorch] int32 words are the same
 *     little-endian byte stream as two codes per byte).
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define W4_OK               0
#define W4_ERR_INVALID     -1  /* null pointer, negative or zero size, bad enum value */
#define W4_ERR_ALIGN       -2  /* K or N not a multiple of 8 ([inc_w4a8] create_weights
                                  requires both GEMM dims to be multiples of 8), or a
                                  pointer / leading dimension not 16-byte aligned */
#define W4_ERR_GROUP       -3  /* group size not accepted (see each entry point) */
#define W4_ERR_DTYPE       -4  /* element type not accepted */
#define W4_ERR_UNSUPPORTED -5  /* shape outside what the kernels handle */
#define W4_ERR_HIP         -6  /* a HIP launch reported an error */

/* Element types. */
#define W4_BF16      1
#define W4_F16       2
#define W4_F32       3
#define W4_I8        4
#define W4_FP8_E4M3  5   /* OCP E4M3FN: bias 7, max 448, no infinities */

/* Source layouts of packed int4 weights accepted by w4_repack. */
#define W4_LAYOUT_GPTQ_KN  1  /* int32 [K/8, N]: 8 codes per word along K; the output
                                 dim is the second ([inc_w4a8] qweight, "NT" layout) */
#define W4_LAYOUT_CT_NK    2  /* int32 [N, K/8]: compressed-tensors weight_packed,
                                 packed along the input dim ([zentorch]) */
#define W4_LAYOUT_S4_NK    3  /* int8 [N, K/2]: signed int4 two per byte (two's
                                 complement nibbles, value = nibble); converted with
                                 XOR 0x88 ([w4afp8] _repack_signed_int4_to_uint4b8) */
#define W4_LAYOUT_I8_NK    4  /* int8 [N, K]: one signed int4 value (-8..7) per byte
                                 ([ct_w4a8] create_weights: weight_packed is int8
                                 [output, input]); values outside -8..7 are
                                 undefined (their low nibble is taken) */

/*
 * Per-token dynamic activation quantization.
 * [inc_w4a8] docstring and apply_weights: activations are quantized per token
 * to symmetric int8 at run time (scale = absmax / 127). [w4afp8]
 * W4AFP8Config: routed-expert activations are quantized per token to 8-bit
 * float, symmetric and dynamic (scale = absmax / 448).
 *
 * For each row m:  a = max_k |x[m,k]| (fp32);  s = a / c  (fp32, correctly
 * rounded; c = 127 for W4_I8, 448 for W4_FP8_E4M3);
 *   W4_I8:       code = clamp(rne(x / s), -127, 127)       (fp32 divide)
 *   W4_FP8_E4M3: code = E4M3(x / s), nearest-even, saturating at +-448
 * An all-zero row gives s = 0 and codes 0. Non-finite inputs: unspecified.
 *
 *   x         device, [M, K] with row stride ldx elements; bf16 or fp16
 *   x_dtype   W4_BF16 or W4_F16
 *   ldx       >= K, a multiple of 8; x must be 16-byte aligned
 *   codes     device, [M, K] contiguous, int8 or E4M3 bytes
 *   code_dtype W4_I8 or W4_FP8_E4M3
 *   scales    device, [M] fp32
 *   group_sums device or NULL, [M, K/group] fp32 (FP8 only): the sum over
 *             each K-group of the decoded FP8 code values of the row, in
 *             fp32. w4a8_grouped_gemm needs it to apply the zero point 8.
 *   group     group size for group_sums (> 0, divides K, multiple of 8);
 *             ignored when group_sums is NULL
 * Errors: INVALID (null, M/K < 0), ALIGN (K % 8, ldx, alignment),
 *         DTYPE, GROUP, HIP.
 */
int w4a8_quantize_act(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                      void* codes, int code_dtype, float* scales,
                      float* group_sums, int64_t group, void* stream);

/*
 * Test hook of the FP8 encode inside w4a8_quantize_act (W4_FP8_E4M3): the
 * fp32 values whose bit patterns are first_bits, first_bits + 1, ...,
 * first_bits + n - 1 are clamped to +-448 and converted to E4M3 (nearest
 * even) exactly as the quantizer converts its quotients x / s. [w4afp8]
 * W4AFP8Config: per-token dynamic 8-bit float activations. It lets a test
 * compare the conversion with a reference on every fp32 input.
 *   n         a multiple of 8, first_bits + n <= 2^32
 *   codes     device, n bytes, 8-byte aligned
 * Non-finite inputs: unspecified codes. Errors: INVALID, ALIGN, HIP.
 */
int w4_fp8_encode_range(uint32_t first_bits, int64_t n, uint8_t* codes, void* stream);

/*
 * The same quantization with a static input scale instead of the per-token
 * one. [ct_w4a8] CompressedTensorsW4A8Int takes is_static_input_scheme: a
 * calibrated, per-tensor activation scale fixed at load time. Every row uses
 *   code = clamp(rne(x / s), -127, 127)  (W4_I8; fp32 divide), or
 *   code = E4M3(x / s) saturating       (W4_FP8_E4M3),
 * so values beyond the calibrated range saturate.
 *   static_scale  device, one fp32 (> 0; 0 gives all-zero codes)
 *   scales        device, [M] fp32 out: static_scale copied to every row, the
 *                 per-row scale array that w4a8_gemm / w4a8_grouped_gemm read
 *   other arguments and errors as w4a8_quantize_act.
 */
int w4a8_quantize_act_static(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             const float* static_scale, void* codes, int code_dtype, float* scales,
                             float* group_sums, int64_t group, void* stream);

/*
 * Per-token asymmetric int8 activation quantization. [ct_w4a8]
 * CompressedTensorsW4A8Int takes an input_symmetric flag and [inc_w4a8]
 * apply_weights hands the per-token quant op's zero output to the int8 GEMM;
 * neither page prints the asymmetric arithmetic. Reading: the min/max grid
 * of [cpu_int4] quantize_groupwise with 256 levels, per row, in fp32:
 *   scale  = (max - min) / 255
 *   code   = clamp(rne((x - min) / scale), 0, 255) - 128   (fp32 divide)
 *   offset = min + 128 * scale          so that x ~ code * scale + offset
 * A constant row gives scale 0, codes -128 and offset = min.
 *   x        device, [M, K] bf16/fp16 with row stride ldx (16-byte aligned)
 *   codes    device, int8 [M, K] (8-byte aligned)
 *   scales, offsets  device, fp32 [M]
 * Rows whose fp32 range (max - min) overflows are outside the reading.
 * Errors: INVALID, ALIGN (K % 8, ldx, alignment), DTYPE, UNSUPPORTED, HIP.
 */
int w4a8_quantize_act_asym(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                           int8_t* codes, float* scales, float* offsets, void* stream);

/*
 * Load-time per-column weight offsets for asymmetric activations:
 *   out[n] = sum_g w_scale[g, n] * sum_{k in g} (q[k, n] - 8)   (fp32)
 * An activation offset z adds z * out[n] to output n, since
 * sum_k z * (q[k, n] - 8) * w_scale[k / group, n] = z * out[n].
 *   w_tiled, w_scale, group, K, N  as w4a8_gemm;  out: device, fp32 [N]
 * Errors: INVALID, ALIGN, GROUP, DTYPE, HIP.
 */
int w4a8_weight_offsets(const void* w_tiled, const void* w_scale, int scale_dtype, int64_t group,
                        int64_t K, int64_t N, float* out, void* stream);

/*
 * W4A8 GEMM with asymmetric per-token activations (codes, scales and
 * offsets from w4a8_quantize_act_asym):
 *   out[m,n] = a_scale[m] * sum_g w_scale[g,n] * P[m,g,n]
 *            + a_offset[m] * w_offsets[n] + bias[n]
 * with P the int32 group sums of w4a8_gemm (the same kernel; the offset
 * term joins the bias in its fp32 epilogue).
 *   a_offset   device, fp32 [M];  w_offsets: device, fp32 [N] from
 *              w4a8_weight_offsets for the same weights, scales and group
 *   other arguments, layouts and errors as w4a8_gemm, except that the
 *   largest K-group (K with group -1) is 131071: asymmetric codes reach
 *   -128, so the int32 sums of 16 * a * (q - 8) need the tighter bound.
 */
int w4a8_gemm_asym(const int8_t* a, const float* a_scale, const float* a_offset, const void* w_tiled,
                   const void* w_scale, int scale_dtype, int64_t group, const float* w_offsets,
                   const void* bias, void* out, int out_dtype, int64_t M, int64_t N, int64_t K,
                   void* stream);

/*
 * Size in bytes of one weight matrix in the kernel-tiled layout produced by
 * w4_repack (tiles of 128 output columns x 128 K, 8 KiB each, ragged edges
 * padded with code 8, i.e. zero weight).
 *   bytes  host pointer receiving the size
 * Errors: INVALID, ALIGN (K or N % 8).
 */
int w4_repack_bytes(int64_t K, int64_t N, size_t* bytes);

/*
 * Load-time repack of `batch` int4 weight matrices [K x N] (batch = number
 * of experts; 1 for a dense layer) from a source layout into the kernel-tiled
 * layout read by w4a8_gemm and w4a8_grouped_gemm. Codes are unchanged
 * (apart from the XOR 0x88 that turns signed int4 into uint4b8 codes for
 * W4_LAYOUT_S4_NK). [inc_w4a8] GPTQ qweight; [zentorch] compressed-tensors
 * weight_packed; [w4afp8] signed-int4 checkpoints.
 *   src     device, batch matrices back to back in `layout`
 *   dst     device, batch * w4_repack_bytes(K, N) bytes, 16-byte aligned
 * Errors: INVALID, ALIGN, HIP.
 */
int w4_repack(const void* src, int layout, int64_t K, int64_t N, int64_t batch,
              void* dst, void* stream);

/*
 * Nibble packing of the byte layout ([cpu_int4] pack_nibbles, unpack_nibbles):
 * [N, K] codes (0..15, one per byte) <-> [N, K/2] bytes with byte j of a row
 * holding code 2j in its low nibble and code 2j+1 in its high nibble, the
 * layout w4a16_repack, w4a16_dequantize and w4_quantize_groupwise use.
 * w4_unpack_nibbles writes the codes as uint8 (the page returns them in an
 * int32 tensor; the values are the same).
 *   codes    device, uint8 [N, K] contiguous; w4_pack_nibbles keeps the low
 *            nibble of each (codes above 15 are outside the definition)
 *   packed   device, uint8 [N, K/2] contiguous
 *   Both buffers 16-byte aligned; the caller owns them.
 * Errors: INVALID (negative size, null pointer), ALIGN (K odd; pointers),
 *         UNSUPPORTED (N*K above 2^40), HIP. N == 0 or K == 0 enqueues nothing.
 */
int w4_pack_nibbles(const uint8_t* codes, int64_t N, int64_t K, uint8_t* packed, void* stream);
int w4_unpack_nibbles(const uint8_t* packed, int64_t N, int64_t K, uint8_t* codes, void* stream);

/*
 * W4A8 GEMM with fused dequantization epilogue.
 * [inc_w4a8] apply_weights: int8 activation codes with per-token scales times
 * int4 weights with fp16 scales per K-group (or per output column), bias
 * fused, result cast to the activation dtype. The GEMM stays on the int8
 * datapath: int32 partial sums per K-group,
 *   P[m,g,n] = sum_{k in g} a[m,k] * (q[k,n] - 8),
 *   out[m,n] = a_scale[m] * sum_g w_scale[g,n] * P[m,g,n] + bias[n].
 *   a         device, int8 [M, K] (codes from w4a8_quantize_act)
 *   a_scale   device, fp32 [M]
 *   w_tiled   device, tiled weights from w4_repack (16-byte aligned)
 *   w_scale   device, [G, N] with G = K/group (1 if group == -1)
 *   scale_dtype must be W4_F16: [inc_w4a8] notes the int8 kernel reads its
 *             scales as fp16 whatever the activation dtype and misreads bf16;
 *             here a bf16 scale is refused instead (W4_ERR_DTYPE)
 *   group     -1 (one group spanning K: per channel, [ct_w4a8] create_weights,
 *             [zentorch] can_implement) or a multiple of 64 dividing K
 *   bias      device or NULL, [N] in out_dtype
 *   out       device, [M, N] in out_dtype (W4_BF16 or W4_F16), 16-byte
 *             aligned (rows are written in 16-byte segments)
 * Errors: INVALID, ALIGN (K or N % 8; w_tiled, out not 16-byte aligned; a
 *         not 8-byte aligned), GROUP, DTYPE, UNSUPPORTED (a K-group, or K
 *         with group -1, above 132096: the int32 sums of 16 * a * (q - 8)
 *         over a group could overflow), HIP. M == 0 or N == 0 enqueues
 *         nothing.
 */
int w4a8_gemm(const int8_t* a, const float* a_scale, const void* w_tiled,
              const void* w_scale, int scale_dtype, int64_t group,
              const void* bias, void* out, int out_dtype,
              int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Test hook of w4a8_gemm: the exact int32 per-group partial sums P[m, g, n]
 * (layout [M, G, N], G = K/group, 1 for group -1). It launches the kernel
 * mode w4a8_gemm launches for the same group (the group-128 and per-channel
 * pipelines included) with a store of each finished group's int32 sum in
 * place of the scaling epilogue. Arguments as w4a8_gemm. Errors as w4a8_gemm.
 */
int w4a8_gemm_partials(const int8_t* a, const void* w_tiled, int64_t group,
                       int32_t* partials, int64_t M, int64_t N, int64_t K,
                       void* stream);

/*
 * W4A16 decode path (M <= 16) on the asymmetric grid w = (q - 8) * scale + zero.
 * [cpu_int4] module docstring: single-stream decode is bandwidth-bound; bf16
 * activations; weights two codes per byte (byte j = w[2j] | w[2j+1] << 4),
 * bf16 scale and zero per (output row, K-group); the weights are repacked
 * once at load time into the layout the kernel streams (as that page does
 * for its own kernel).
 *
 * w4a16_repack_bytes: sizes of the two tiled buffers for a [N, K] matrix.
 * w4a16_repack: load-time repack.
 *   w        device, uint8 [N, K/2] in the byte layout above
 *   scale    device, bf16 [N, K/group];  zero: device bf16 [N, K/group] or
 *            NULL (zero offsets);  sz_dtype must be W4_BF16
 *   group    64, 128, 256 or 512, dividing K
 *   w_tiled  device, w_bytes (16-byte aligned); sz_tiled: device, sz_bytes
 * w4a16_gemm:
 *   out[m,n] = sum_k x[m,k] * ((q[n,k] - 8) * scale[n,k/group] + zero[n,k/group])
 *   x        device, bf16 [M, K] contiguous (16-byte aligned)
 *   w_tiled, sz_tiled  from w4a16_repack with the same K, N, group
 *   out      device, bf16 [M, N]
 * Errors: INVALID, ALIGN (K, N % 8; pointers), GROUP, DTYPE,
 *         UNSUPPORTED (M > 16, N*K >= 2^31), HIP.
 */
int w4a16_repack_bytes(int64_t K, int64_t N, int64_t group, size_t* w_bytes, size_t* sz_bytes);
int w4a16_repack(const uint8_t* w, const void* scale, const void* zero, int sz_dtype, int64_t group,
                 int64_t K, int64_t N, void* w_tiled, void* sz_tiled, void* stream);
int w4a16_gemm(const void* x, const void* w_tiled, const void* sz_tiled, int64_t group, void* out,
               int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Grouped GEMM over routed-expert segments with FP8 activations.
 * [w4afp8] W4AFP8Config: routed experts hold int4 group-128 weights
 * (symmetric, zero point 8) and take per-token dynamic FP8 activations.
 * Routed rows are grouped by expert: rows expert_offsets[e] ..
 * expert_offsets[e+1]-1 belong to expert e and row r carries token
 * row_token[r]:
 *   out[r,n] = a_scale[t] * sum_g w_scale[e,g,n]
 *              * sum_{k in g} dec(a[t,k]) * (q[e,k,n] - 8),   t = row_token[r]
 *   a           device, E4M3 codes [T, K] (from w4a8_quantize_act)
 *   a_scale     device, fp32 [T]
 *   a_group_sums device, fp32 [T, K/group] (from w4a8_quantize_act, same group)
 *   row_token   device, int32 [R], each in [0, T)
 *   expert_offsets device, int32 [E+1], non-decreasing, [0] = 0, [E] = R
 *   w_tiled     device, E tiled matrices (w4_repack with batch = E)
 *   w_scale     device, fp16 [E, G, N]
 *   group       128, 256 or 512, dividing K
 *   out         device, bf16 [R, N], rows in segment order
 *   a, w_tiled and out must be 16-byte aligned.
 * Errors: INVALID, ALIGN, GROUP, DTYPE, UNSUPPORTED (T*K >= 2^31), HIP.
 * Offsets and token ids are read on the device and are not validated;
 * out-of-range values are undefined behaviour.
 */
int w4a8_grouped_gemm(const void* a, int a_dtype, const float* a_scale,
                      const float* a_group_sums, const int32_t* row_token,
                      const int32_t* expert_offsets, int64_t E,
                      const void* w_tiled, const void* w_scale, int scale_dtype,
                      int64_t group, void* out, int out_dtype,
                      int64_t T, int64_t R, int64_t N, int64_t K, void* stream);

/*
 * Weight-only int4 GEMM for few rows on the kernel-tiled weights of w4a8_gemm
 * (the same bytes and the same fp16 scales), activations unquantized.
 * [inc_w4a8] class docstring: the int8 kernel and the weight-only kernel take
 * bit-identical weights; apply_weights: below a token-count threshold the
 * layer calls the weight-only path instead of quantizing the activations.
 *   out[m,n] = sum_g w_scale[g,n] * sum_{k in g} x[m,k] * (q[k,n] - 8) + bias[n]
 *   x         device, [M, K] contiguous, bf16 or fp16 (x_dtype); 8-byte aligned
 *   w_tiled   device, from w4_repack (16-byte aligned)
 *   w_scale   device, fp16 [G, N]; scale_dtype must be W4_F16
 *   group     -1 or a multiple of 64 dividing K (as w4a8_gemm)
 *   bias      device or NULL, [N] in the activation dtype
 *   out       device, [M, N] in the activation dtype
 * Errors: INVALID, ALIGN (K, N % 8; pointers), GROUP, DTYPE,
 *         UNSUPPORTED (M > 16), HIP.
 */
int w4a16_tiled_gemm(const void* x, int x_dtype, const void* w_tiled, const void* w_scale,
                     int scale_dtype, int64_t group, const void* bias, void* out,
                     int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The linear layer with its per-call dispatch ([inc_w4a8] apply_weights and
 * _MIN_TOKENS_FOR_INT8): M >= min_tokens_int8 quantizes the activations per
 * token to int8 (w4a8_quantize_act) and runs w4a8_gemm; fewer rows run the
 * weight-only path (w4a16_tiled_gemm, 16 rows per launch). Both read the same
 * tiled weights and fp16 scales.
 *   min_tokens_int8  threshold; <= 0 selects W4_LINEAR_MIN_TOKENS_INT8, the
 *             crossover measured on MI355X for these kernels (the page's 512
 *             was measured for its own device)
 *   workspace device scratch of at least w4_linear_workspace_bytes(M, N, K,
 *             group, min_tokens_int8) bytes (16-byte aligned; may be NULL
 *             when that is 0): the int8 path's codes and fp32 row scales and,
 *             when the GEMM splits K (group 128 with too few tiles to fill
 *             the chip: few rows), its fp32 partial tiles, summed by a second
 *             kernel (the sum order is fixed: results are reproducible). The
 *             caller owns it; calls sharing one workspace must not overlap.
 *   x, out    device, 16-byte aligned; out [M, N] in the activation dtype
 *   other arguments as w4a16_tiled_gemm.
 * Errors: those of the path taken (UNSUPPORTED for a K-group above 132096,
 *         as w4a8_gemm, whatever M), and INVALID when the workspace is too small.
 */
#define W4_LINEAR_MIN_TOKENS_INT8 33
int w4_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t group, int64_t min_tokens_int8,
                              size_t* bytes);
int w4_linear(const void* x, int x_dtype, const void* w_tiled, const void* w_scale, int scale_dtype,
              int64_t group, const void* bias, void* out, int64_t M, int64_t N, int64_t K,
              int64_t min_tokens_int8, void* workspace, size_t workspace_bytes, void* stream);

/*
 * w4_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same dispatch and kernels, with the workspace taken from a device array
 * inside the library instead of an argument.
 *   - The array holds W4_LINEAR_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU
 *     the entry point runs on, from its first call there until the process
 *     ends. A call whose workspace (w4_linear_workspace_bytes) exceeds it
 *     returns W4_ERR_UNSUPPORTED before anything is enqueued; the weight-only
 *     side (M below the threshold) needs none.
 *   - Call it with the stream's device current. Its first call on a device
 *     looks up the array's address there (hipGetSymbolAddress); no call
 *     allocates (no hipMalloc, hipFree or allocating library routine).
 *   - Every call on one GPU shares that GPU's array, and the array keeps the
 *     last call's contents: calls that overlap on one GPU (other streams,
 *     other threads) race and give undefined results. Nothing in it needs to
 *     start at zero (each call writes all of the scratch it reads).
 * Arguments, results and other errors as w4_linear without the workspace.
 */
#define W4_LINEAR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int w4_linear_noalloc(const void* x, int x_dtype, const void* w_tiled, const void* w_scale, int scale_dtype,
                      int64_t group, const void* bias, void* out, int64_t M, int64_t N, int64_t K,
                      int64_t min_tokens_int8, void* stream);

/*
 * Prefill path of the W4A16 layer: the weight unpacked to bf16 once per call
 * for an ordinary bf16 GEMM. [cpu_int4] module docstring: large batches
 * unpack the weight to bf16 once per call and hand it to the ordinary GEMM
 * (one extra pass over the weights, reading a row-major copy); dequantize:
 * w = (q - 8) * scale + zero.
 *   w        device, uint8 [N, K/2], byte j = q[2j] | q[2j+1] << 4 (8-byte aligned)
 *   scale    device, bf16 [N, K/group]; zero: device bf16 [N, K/group] or NULL
 *   group    64, 128, 256 or 512, dividing K
 *   out      device, bf16 [N, K] row-major (16-byte aligned): computed in
 *            fp32 as fma(q - 8, scale, zero), rounded to nearest even
 * The GEMM on it is w4a16_prefill_gemm (w4a16_prefill runs both).
 * Errors: INVALID, ALIGN, GROUP, DTYPE, UNSUPPORTED (N*K >= 2^31), HIP.
 */
int w4a16_dequantize(const uint8_t* w, const void* scale, const void* zero, int sz_dtype, int64_t group,
                     int64_t K, int64_t N, void* out, void* stream);

/*
 * The prefill path's GEMM and the whole path ([cpu_int4] _cpu_int4_linear:
 * batches at or above the threshold take the dequantized bf16 weight through
 * an ordinary GEMM, y = x @ w^T).
 * w4a16_prefill_gemm: hand-written bf16 matrix-core GEMM, fp32 sums, output
 *   rounded to bf16 (nearest even):
 *     out[m, n] = sum_k x[m, k] * w[n, k]
 *   x      device, bf16 [M, K] row-major
 *   w      device, bf16 [N, K] row-major (e.g. from w4a16_dequantize)
 *   out    device, bf16 [M, N] row-major
 *   All three 16-byte aligned; K a multiple of 64, N of 8.
 * w4a16_prefill_workspace_bytes: N * K * 2, the bf16 weight's size.
 * w4a16_prefill: w4a16_dequantize into the workspace, then
 *   w4a16_prefill_gemm, on one stream.
 *   w, scale, zero, group as w4a16_dequantize; x, out as w4a16_prefill_gemm
 *   workspace  device, >= w4a16_prefill_workspace_bytes(N, K), 16-byte
 *              aligned, owned by the caller; calls sharing it must not overlap
 * Errors: INVALID (null, negative sizes, workspace too small), ALIGN (K % 64,
 *         N % 8, pointers), GROUP, DTYPE (scale/zero not bf16), UNSUPPORTED
 *         (sizes; N*K >= 2^31 for w4a16_prefill), HIP. M == 0 or N == 0
 *         enqueues nothing.
 */
int w4a16_prefill_gemm(const void* x, const void* w, void* out, int64_t M, int64_t N, int64_t K, void* stream);
int w4a16_prefill_workspace_bytes(int64_t N, int64_t K, size_t* bytes);
int w4a16_prefill(const void* x, const uint8_t* w, const void* scale, const void* zero, int sz_dtype, int64_t group,
                  void* out, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Groupwise min/max int4 quantization of a weight matrix, on the device.
 * [cpu_int4] quantize_groupwise: per row n and group g of `group` columns, in
 * fp32: scale = max(max - min, 1e-9) / 15, zero = min + 8 * scale,
 * q = clamp(rne((w - min) / scale), 0, 15), so that (q - 8) * scale + zero
 * reproduces the group's min and max; codes two per byte, low nibble first
 * ([cpu_int4] pack_nibbles), the byte layout that w4a16_repack reads.
 *   w        device, [N, K] contiguous, bf16, fp16 or fp32 (w_dtype);
 *            16-byte aligned
 *   group    64, 128, 256 or 512, dividing K
 *   packed   device, uint8 [N, K/2], 4-byte aligned
 *   scale, zero  device, [N, K/group] each, fp32 or bf16 (sz_dtype; bf16 is
 *            the fp32 value rounded to nearest even)
 * Errors: INVALID, ALIGN (pointers), GROUP, DTYPE, HIP. Any N (rows are
 *         independent); w4a16_repack then needs N % 8 == 0.
 */
int w4_quantize_groupwise(const void* w, int w_dtype, int64_t N, int64_t K, int64_t group,
                          uint8_t* packed, void* scale, void* zero, int sz_dtype, void* stream);

/*
 * Int4 embedding gather. [cpu_int4] CPUInt4EmbeddingMethod.embedding: the rows
 * of the vocab table picked by the token ids, dequantized as
 * (q - 8) * scale + zero in fp32 and cast to bf16. The table is read in the
 * W4A16 tiled layout, so the same w_tiled / sz_tiled serve the tied output
 * head (w4a16_gemm) ([cpu_int4] tie_weights shares every quantized tensor).
 *   ids      device, int32 [T]; an id outside [0, V) yields a zero row
 *   w_tiled, sz_tiled  from w4a16_repack of the [V, K] table with this group
 *   out      device, bf16 [T, K], 16-byte aligned
 * Errors: INVALID, ALIGN, GROUP, UNSUPPORTED (V*K >= 2^31), HIP.
 */
int w4a16_embedding(const int32_t* ids, int64_t T, const void* w_tiled, const void* sz_tiled,
                    int64_t group, int64_t V, int64_t K, void* out, void* stream);

/*
 * Measurement support: the matrix core's measured peak on this GPU. Pure
 * MFMA loops with no memory traffic (1024 blocks of 256 threads, eight
 * independent accumulator chains per wave, iters iterations), kind 0:
 * v_mfma_i32_16x16x64_i8, 1: v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3), 2:
 * v_mfma_f32_16x16x32_bf16. The rates the GEMMs reach are reported against
 * it beside the nominal peaks.
 *   iters       1 .. 2^24
 *   sink        device int32 [sink_elems], sink_elems >= 1024 * 256; receives
 *               a value per thread that depends on every chain
 *   ops         host: set to the operations one launch performs
 *               (2 * 16 * 16 * K per MFMA, K = 64, 128 or 32)
 * Errors: INVALID, ALIGN, HIP.
 */
int w4_probe_mfma(int kind, int64_t iters, int32_t* sink, int64_t sink_elems, double* ops, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* w4_last_error(void);

/* ABI version (major * 100 + minor). */
int w4_version(void);

#ifdef __cplusplus
}
#endif
#endif /* W4_H */
