/*
 * nvfp4.h -- C ABI of libnvfp4.so: NVFP4 block-scaled quantize / dequantize /
 * quantize-dequantize and the qmv, qqmm and gather_qmm contractions on one
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited:
 *   "mlx 0.30.7.2 -> 0.30.7.6" source diff, page 8 (my.diffend.io): ops.cpp
 *       hunks validate_global_scale, validate_qqmm_inputs, qqmm, fp_quantize,
 *       quantize, fp_dequantize, dequantize; ops.h declarations.
 *   same diff, page 7: fp_quantize.cu (fp_quantize_dequantize,
 *       fp_quantize_rowwise, fp_dequantize and their host wrappers), qqmm.cpp
 *       (QQMatmul::eval_gpu).
 *   "[Metal] global scale for qmm", ml-explore/mlx pull request 4458:
 *       statement and "Example"; gather_qmm test loops in the review.
 *   osaurus-ai/mlx pull request 31: "What fails", "The test", "The fix".
 *
 * Number format (NVFP4): every 16 consecutive elements of a row share one
 * e4m3 block scale; each element is a 4-bit e2m1 code.  An optional float32
 * per-tensor global scale g (the tensor's absolute maximum) sets the encode
 * factor 2688/g and the decode factor g/2688, 2688 = 448 * 6.  Decoding is
 *     w = e2m1(q) * (e4m3(s) * g/2688)
 * with the global factor on the block scale, never on the output.
 *
 * Layout of a quantized [rows, k] tensor (k a multiple of 16), all row-major,
 * contiguous, no padding:
 *   codes   uint8 [rows, k/2]   element 2j in the low nibble of byte j
 *   scales  uint8 [rows, k/16]  e4m3 bytes
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers to caller-owned memory.  The
 *     library never allocates, frees or keeps them, and keeps no state
 *     between calls except a per-thread error message and a per-device
 *     "architecture checked" flag.
 *   - Every call enqueues work on `stream` and returns without waiting.
 *   - A global scale is a device pointer to one float32 (per expert: e
 *     floats), or NULL for "no global scale" (factors 1).  Its value must be
 *     finite and > 0 (not checked: it lives on the device).
 *   - Returns NVFP4_OK, or an error code with nothing enqueued; the message
 *     is then available from nvfp4_last_error() on the same thread.  Argument
 *     errors are detected on the host before any HIP call.
 *   - Element types: NVFP4_F32, NVFP4_F16, NVFP4_BF16 (float64 is rejected
 *     as in the pages' dispatch).
 *   - The device behind `stream` (the current device for the null stream)
 *     must be gfx950; otherwise NVFP4_ERR_UNSUPPORTED.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARGUMENT = 1, /* bad shape, pointer, dtype or combination     */
  NVFP4_ERR_UNSUPPORTED = 2,      /* device is not gfx950, or size above a limit  */
  NVFP4_ERR_DEVICE = 3            /* a HIP call failed (message has HIP's text)   */
} nvfp4_status;

typedef enum { NVFP4_F32 = 0, NVFP4_F16 = 1, NVFP4_BF16 = 2 } nvfp4_dtype;

/* Message of the last failed call on this thread ("[op] ..."), or "". */
const char* nvfp4_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int nvfp4_version(void);

/*
 * nvfp4_tensor_amax -- amax_out[0] = max |x[i]| over i < n, as float32.
 * This is the per-tensor global scale g the configurations use (the
 * cotangent amax of QQMatmul::vjp, diff page 8, is the same reduction).
 *   x         device, n elements of type dt
 *   amax_out  device, 1 float; written (n == 0 gives 0)
 * One kernel launch; its workgroups reduce through one of 64 library-owned
 * device words, taken in turn per call, so up to 64 calls may be in flight at
 * once on different streams (a captured graph keeps its word: do not replay
 * one graph on two streams at once).
 * Errors: NULL pointer, n < 0, bad dtype.
 */
nvfp4_status nvfp4_tensor_amax(const void* x, nvfp4_dtype dt, int64_t n, float* amax_out,
                               hipStream_t stream);

/*
 * nvfp4_quantize -- NVFP4 encode of x [rows, k] (diff page 7,
 * fp_quantize_rowwise; diff page 8, fp_quantize and quantize).  Per group of
 * 16: sd = (amax/6) * (2688/g) in float32, s = e4m3(sd) (nearest-even,
 * saturating), q_i = e2m1(x_i * ((2688/g) / e4m3value(s))); a block whose
 * scale is 0 gets all-zero codes (sign kept).
 *   x             device [rows, k] of type dt, row-major
 *   global_scale  device float or NULL
 *   codes         device uint8 [rows, k/2], written
 *   scales        device uint8 [rows, k/16], written
 * Errors: NULL pointer, rows < 0, k <= 0 or k % 16 != 0, bad dtype.
 */
nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t k,
                            const float* global_scale, uint8_t* codes, uint8_t* scales,
                            hipStream_t stream);

/*
 * nvfp4_dequantize -- out = T(e2m1(q) * (e4m3(s) * g/2688)) (diff page 7,
 * fp_dequantize; diff page 8, fp_dequantize and dequantize).
 *   codes, scales  device, layout above, [rows, k]
 *   global_scale   device float or NULL
 *   out            device [rows, k] of type out_dt, written
 * Errors: NULL pointer, rows < 0, k <= 0 or k % 16 != 0, bad dtype.
 */
nvfp4_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                              int64_t k, const float* global_scale, void* out,
                              nvfp4_dtype out_dt, hipStream_t stream);

/*
 * nvfp4_quant_dequant -- x_hat = dequantize(quantize(x, g), g) in x's type
 * (diff page 7, fp_quantize_dequantize; osaurus-ai/mlx PR 31, "The fix").
 *   x      device [rows, k] of type dt
 *   x_hat  device [rows, k] of type dt, written (may equal x)
 * Errors: as nvfp4_quantize.
 */
nvfp4_status nvfp4_quant_dequant(const void* x, nvfp4_dtype dt, int64_t rows, int64_t k,
                                 const float* global_scale, void* x_hat, hipStream_t stream);

/*
 * nvfp4_qmv -- out[n] = T( sum_k x_hat[k] * w[n, k] ), M = 1 (diff page 7,
 * QQMatmul::eval_gpu, M == 1 branch): x goes through the NVFP4 round trip with
 * global_scale_x inside the kernel, w is decoded with global_scale_w on each
 * block scale ("[Metal] global scale for qmm" PR 4458, statement), float32
 * accumulation.
 *   x               device [k] of type dt
 *   global_scale_x  device float or NULL
 *   w_codes         device uint8 [n, k/2];  w_scales device uint8 [n, k/16]
 *   global_scale_w  device float or NULL; both or neither of the two global
 *                   scales (diff page 8, validate_qqmm_inputs)
 *   out             device [n] of type dt, written
 * Errors: NULL pointer, n <= 0, k <= 0 or k % 16 != 0, exactly one global
 * scale, bad dtype, k above 32768 (UNSUPPORTED).
 */
nvfp4_status nvfp4_qmv(const void* x, nvfp4_dtype dt, const float* global_scale_x,
                       const uint8_t* w_codes, const uint8_t* w_scales,
                       const float* global_scale_w, int64_t n, int64_t k, void* out,
                       hipStream_t stream);

/*
 * nvfp4_qqmm_workspace_size -- bytes of device workspace nvfp4_qqmm needs for
 * these sizes (0 when m == 1).  The workspace holds x_hat [m, k] of type dt.
 */
size_t nvfp4_qqmm_workspace_size(int64_t m, int64_t n, int64_t k, nvfp4_dtype dt);

/*
 * nvfp4_qqmm -- out = T( x_hat @ w^T ), x [m, k] and w NVFP4 [n, k] (diff
 * page 8, qqmm; diff page 7, QQMatmul::eval_gpu): x_hat is x after the NVFP4
 * round trip with global_scale_x, w is decoded with global_scale_w on the
 * block scale; float32 accumulation.  m == 1 runs the qmv kernel; 2 <= m
 * <= 16 with 16-bit x, k % 128 == 0 and m (k + 8) 2 + 7168 <= 163840 runs
 * the small-batch kernel, which does the x round trip itself (the workspace
 * is then not touched); larger m go through the workspace and the
 * matrix-core kernels.  The paths other than qmv round each decoded weight
 * e2m1(q) * fp32(e4m3(s) * g_w/2688) to dt before the products.
 *   x               device [m, k] of type dt
 *   w_codes/scales  device [n, k/2] / [n, k/16]
 *   out             device [m, n] of type dt, written
 *   workspace       device, at least nvfp4_qqmm_workspace_size() bytes,
 *                   256-byte aligned; may be NULL when that size is 0
 * Errors: NULL pointer, m, n <= 0, k <= 0 or k % 16 != 0, exactly one global
 * scale, workspace too small or misaligned, bad dtype; UNSUPPORTED when m > 1
 * and x (m * k elements) or the weight's codes (n * k / 2 bytes) reach 2 GB
 * (the matrix-core kernels address them with 32-bit offsets).
 */
nvfp4_status nvfp4_qqmm(const void* x, nvfp4_dtype dt, const float* global_scale_x,
                        const uint8_t* w_codes, const uint8_t* w_scales,
                        const float* global_scale_w, int64_t m, int64_t n, int64_t k, void* out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_qmm -- out = T( x @ w^T ) with x used as given (not quantized) and w
 * NVFP4 decoded with global_scale_w on the block scale: the pages'
 * quantized_matmul (diff page 8, ops.cpp quantized_matmul; "mlx 0.30.7" diff
 * page 71, QuantizedMatmul::eval_gpu), i.e. the contraction of nvfp4_qqmm
 * without the activation round trip.  No workspace.  1 <= m <= 16 runs the
 * small-batch kernel under the conditions given for nvfp4_qqmm.
 *   x               device [m, k] of type dt, 16-byte aligned
 *   w_codes/scales  device [n, k/2] / [n, k/16]
 *   global_scale_w  device float or NULL
 *   out             device [m, n] of type dt, written
 * Errors: NULL pointer, m, n <= 0, k <= 0 or k % 16 != 0, bad dtype; the 2 GB
 * limits of nvfp4_qqmm for m > 1.
 */
nvfp4_status nvfp4_qmm(const void* x, nvfp4_dtype dt, const uint8_t* w_codes,
                       const uint8_t* w_scales, const float* global_scale_w, int64_t m, int64_t n,
                       int64_t k, void* out, hipStream_t stream);

/* ---------------------------------------------------------------- backward
 *
 * nvfp4_quantize_columnwise -- quantize x [rows, cols] (row-major) along its
 * first axis, i.e. encode the transpose x^T [cols, rows] row by row: the
 * pages' columnwise quantize of an M-major tensor ("mlx 0.30.7.2 ->
 * 0.30.7.6" diff page 7, fp_quantize_columnwise), with the same per-group
 * arithmetic as nvfp4_quantize.
 *   x            device [rows, cols] of type dt, 16-byte aligned
 *   codes        device uint8 [cols, rows/2], 8-byte aligned, written
 *   scales       device uint8 [cols, rows/16], written
 * Errors: rows not a multiple of 16, cols not a multiple of 8 (16-bit) or 4
 * (float32), NULL pointer, misalignment, bad dtype.
 */
nvfp4_status nvfp4_quantize_columnwise(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                       const float* global_scale, uint8_t* codes, uint8_t* scales,
                                       hipStream_t stream);

/*
 * nvfp4_quant_dequant_columnwise -- the NVFP4 round trip of x^T: writes
 * xhat_t [cols, rows] of type dt, the dequantized nvfp4_quantize_columnwise
 * (what nvfp4_quant_dequant gives for the transpose).  xhat_t 16-byte
 * aligned; errors as nvfp4_quantize_columnwise.
 */
nvfp4_status nvfp4_quant_dequant_columnwise(const void* x, nvfp4_dtype dt, int64_t rows,
                                            int64_t cols, const float* global_scale, void* xhat_t,
                                            hipStream_t stream);

/*
 * nvfp4_qqmm_vjp -- gradients of y = qqmm(x, w) for the cotangent dy
 * ("mlx 0.30.7.2 -> 0.30.7.6" diff page 8, primitives.cpp QQMatmul::vjp):
 *   g_dy = float32(max |dy|) when the global scales are given (none otherwise)
 *   dx [m, k] = qqmm(dy, w^T): dy round-tripped under g_dy, w^T [k, n]
 *               quantized along n under g_w;
 *   dw [n, k] = qqmm(dy^T, x^T): dy^T round-tripped along m under g_dy, x^T
 *               [k, m] quantized along m under g_x;
 * float32 accumulation, outputs of type dt (the gradients of the global
 * scales are zero and not produced).  Every step runs on the matrix-core or
 * small-batch contraction kernels of nvfp4_qqmm / nvfp4_qmm.
 *   x [m, k], w [n, k], dy [m, n]   device, type dt, 16-byte aligned
 *   global_scale_x, global_scale_w  device floats, both or neither
 *   dx, dw          device outputs; either may be NULL (not computed), not both
 *   dy_amax         device float written with g_dy, or NULL
 *   workspace       device, nvfp4_qqmm_vjp_workspace_size() bytes, 256-byte
 *                   aligned; its contents afterwards are scratch
 * Errors: m, n or k not a positive multiple of 16 (each is the quantized
 * dimension of an operand), exactly one global scale, NULL or misaligned
 * pointers, workspace too small, bad dtype.
 */
size_t nvfp4_qqmm_vjp_workspace_size(int64_t m, int64_t n, int64_t k, nvfp4_dtype dt);
nvfp4_status nvfp4_qqmm_vjp(const void* x, const void* w, const void* dy, nvfp4_dtype dt,
                            const float* global_scale_x, const float* global_scale_w, int64_t m,
                            int64_t n, int64_t k, void* dx, void* dw, float* dy_amax,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_gather_qmm_workspace_size -- bytes of device workspace
 * nvfp4_gather_qmm (and nvfp4_gather_qmm_packed, nvfp4_mx_gather_qmm) needs:
 * the routing tables (expert offsets, the pair order) and the routing's
 * per-chunk counts.
 * 0 for non-positive sizes or t * top_k >= 2^31.
 */
size_t nvfp4_gather_qmm_workspace_size(int64_t t, int64_t top_k, int64_t e, int64_t n,
                                       int64_t k);

/*
 * nvfp4_gather_qmm -- mixture-of-experts product with per-expert NVFP4
 * weights ("[Metal] global scale for qmm" PR 4458: x @ dequant(W) with the
 * per-expert global scale, shape [E, 1, 1], inside the dequantization):
 *     out[t, j, :] = T( x[t, :] @ w[idx[t, j]]^T )
 * x is used as given (not quantized).  The pairs (t, j) are first grouped by
 * expert in a stable order (ascending t, then j), then each expert's rows
 * are multiplied by its decoded weights.
 *   x               device [t, k] of type dt
 *   w_codes         device uint8 [e, n, k/2];  w_scales uint8 [e, n, k/16]
 *   global_scale_w  device float [e] or NULL
 *   expert_idx      device int32 [t, top_k]; a pair whose index lies
 *                   outside [0, e) multiplies no expert and its output row
 *                   out[t, j, :] is written with zeros
 *   out             device [t, top_k, n] of type dt, written
 *   workspace       device, at least nvfp4_gather_qmm_workspace_size() bytes,
 *                   256-byte aligned
 * Errors: NULL pointer, t, top_k, e, n <= 0, k <= 0 or k % 16 != 0, workspace
 * too small, bad dtype; UNSUPPORTED for more than 1024 experts, t * top_k >=
 * 2^31, or x (t * k elements) or one expert's codes (n * k / 2 bytes) of 2 GB
 * or more.
 */
nvfp4_status nvfp4_gather_qmm(const void* x, nvfp4_dtype dt, const uint8_t* w_codes,
                              const uint8_t* w_scales, const float* global_scale_w,
                              const int32_t* expert_idx, int64_t t, int64_t top_k, int64_t e,
                              int64_t n, int64_t k, void* out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_gather_qmm_noalloc -- nvfp4_gather_qmm for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same arguments without the
 * workspace, the same kernels and results.  The routing tables live in a
 * fixed 5 MiB device array of the library (one per GPU, held until the
 * process ends), so the call allocates nothing.  Its contents are whatever
 * the last call on that GPU left; every table the call reads it writes
 * first.  Calls that overlap on one GPU (on different streams, or graph
 * replays in flight together) share that array and race: serialize them.
 * Limit: the tables (e + 1 + t * top_k ints plus the routing's per-chunk
 * counts, each part rounded up to 256 bytes) must fit in 5 MiB -- e.g.
 * t * top_k = 1,048,576 pairs with up to 256 experts; larger calls return
 * NVFP4_ERR_UNSUPPORTED with a message naming the sizes.  Other errors as
 * nvfp4_gather_qmm.
 */
nvfp4_status nvfp4_gather_qmm_noalloc(const void* x, nvfp4_dtype dt, const uint8_t* w_codes,
                                      const uint8_t* w_scales, const float* global_scale_w,
                                      const int32_t* expert_idx, int64_t t, int64_t top_k,
                                      int64_t e, int64_t n, int64_t k, void* out,
                                      hipStream_t stream);

/*
 * nvfp4_moe_route -- the routing step of nvfp4_gather_qmm on its own:
 * offsets[0..e] = exclusive prefix sum of the per-expert pair counts,
 * perm[offsets[x] .. offsets[x+1]) = the flat pair ids t*top_k + j routed to
 * expert x, ascending; perm[offsets[e] .. t*top_k) = the pairs whose index
 * lies outside [0, e), ascending.
 *   expert_idx  device int32 [t, top_k]
 *   offsets     device int32 [e + 1], written
 *   perm        device int32 [t * top_k], written
 *   workspace   device, nvfp4_moe_route_workspace_size() bytes (the
 *               counting sort's per-chunk counts), 256-byte aligned
 * Errors: NULL pointer, t, top_k, e <= 0, workspace too small or misaligned;
 * UNSUPPORTED for t * top_k >= 2^31 or more than 1024 experts.
 */
size_t nvfp4_moe_route_workspace_size(int64_t t, int64_t top_k, int64_t e);
nvfp4_status nvfp4_moe_route(const int32_t* expert_idx, int64_t t, int64_t top_k, int64_t e,
                             int32_t* offsets, int32_t* perm, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Packed weights for the matrix-core contractions.
 *
 * The row-major layout above is the exchange format (quantize, dequantize,
 * qmv and the contractions all accept it).  A weight that will be multiplied
 * many times can also be repacked once into the order the gfx950 matrix-core
 * kernel reads it in, the analogue of the pages' one-time scale swizzle into
 * the block-scaled GEMM's tile layout ("mlx 0.30.7.2 -> 0.30.7.6" diff page
 * 7, qqmm_utils / QQMatmul::eval_gpu).  The values are the same bytes; only
 * their order changes.  For 32-row tile T and 64-wide k-step s:
 *   packed codes   1 KB block (T, s); bytes 16 l .. 16 l + 15 are row-major
 *                  code bytes 32 s + 16 (l / 32) .. + 15 of row 32 T + l % 32
 *   packed scales  128-byte block (T, s); bytes 4 c .. 4 c + 3 are row-major
 *                  scale bytes 4 s .. 4 s + 3 of row 32 T + c
 * blocks in (T, s) order, rows past `rows` zero.  k must be a multiple of 64.
 * Experts stack as consecutive row ranges, so a stacked [e, n, k] weight is
 * packed as rows = e * n (n a multiple of 32 for gather_qmm_packed).
 */

/*
 * nvfp4_mfma_pack_size -- bytes of the packed codes and scales of a
 * [rows, k] NVFP4 weight.
 * Errors: NULL pointer, rows <= 0, k not a positive multiple of 64 (the
 * outputs are then 0).
 */
nvfp4_status nvfp4_mfma_pack_size(int64_t rows, int64_t k, size_t* codes_bytes,
                                  size_t* scales_bytes);

/*
 * nvfp4_mfma_pack -- write the packed copy of a row-major NVFP4 weight.
 *   codes, scales                device [rows, k/2] / [rows, k/16], row-major
 *   packed_codes, packed_scales  device, sizes from nvfp4_mfma_pack_size,
 *                                written
 * Errors: as nvfp4_mfma_pack_size; NULL pointer; codes / packed_codes not
 * 16-byte or scales / packed_scales not 4-byte aligned.
 */
nvfp4_status nvfp4_mfma_pack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                             uint8_t* packed_codes, uint8_t* packed_scales, hipStream_t stream);

/*
 * nvfp4_qqmm_packed, nvfp4_qmm_packed, nvfp4_gather_qmm_packed -- nvfp4_qqmm,
 * nvfp4_qmm and nvfp4_gather_qmm with the weight given as its packed copy.
 * They run the matrix-core path only: x float16 or bfloat16, k a multiple of
 * 64, n a multiple of 4 (gather: of 32).  The remaining arguments,
 * workspaces and errors are those of the row-major calls; any m >= 1 runs a
 * matrix-core kernel.  Above 16 rows (or outside the small-batch conditions
 * of nvfp4_qqmm) the results equal the row-major calls' bit for bit; with
 * 1 <= m <= 16 the packed small-batch kernel sums in another order than the
 * row-major one (32-row instead of 16-row tiles), so the two agree to
 * rounding, not bitwise.  nvfp4_qqmm_packed with 1 <= m <= 4 rows of
 * bfloat16 x and 512 <= k <= 8192 runs the fp4 matrix-core kernel, which
 * feeds the stored weight codes to the matrix cores and x_hat as two e2m1
 * vectors per block times per-block coefficients; that split is x_hat itself
 * while x_hat stays out of bfloat16's subnormal range, i.e. for g_x >= 2688 *
 * 2^-116 (about 3.2e-32) or without global scales.  Below that bound x_hat
 * elements that are bfloat16 subnormals may differ by one subnormal step.
 */
nvfp4_status nvfp4_qqmm_packed(const void* x, nvfp4_dtype dt, const float* global_scale_x,
                               const uint8_t* packed_codes, const uint8_t* packed_scales,
                               const float* global_scale_w, int64_t m, int64_t n, int64_t k,
                               void* out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);
nvfp4_status nvfp4_qmm_packed(const void* x, nvfp4_dtype dt, const uint8_t* packed_codes,
                              const uint8_t* packed_scales, const float* global_scale_w, int64_t m,
                              int64_t n, int64_t k, void* out, hipStream_t stream);
nvfp4_status nvfp4_gather_qmm_packed(const void* x, nvfp4_dtype dt, const uint8_t* packed_codes,
                                     const uint8_t* packed_scales, const float* global_scale_w,
                                     const int32_t* expert_idx, int64_t t, int64_t top_k,
                                     int64_t e, int64_t n, int64_t k, void* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * gather_qmm in its indexed form -- the cells of the pages' gather_qmm test
 * loops ("[Metal] global scale for qmm" (ml-explore/mlx PR 4458): float32,
 * float16 and bfloat16; transpose True and False; per-expert global scales
 * [E, 1, 1]) and the op's lhs_indices, rhs_indices and sorted_indices.
 *   x            device [entries, rows_per_entry, k] of type dt, 16-byte aligned
 *   w_codes      transpose = 1: [e, n, k/2] with scales [e, n, k/16] (each
 *                expert's [n, k] weight quantized along k, out = x @ w^T);
 *                transpose = 0: [e, k, n/2] with scales [e, k, n/16] (each
 *                expert's [k, n] weight quantized along n, out = x @ w)
 *   global_scale_w  device float32 [e] or NULL
 *   lhs_indices  device int32 [pairs] in [0, entries), or NULL: pair p uses
 *                x entry p (then pairs <= entries)
 *   rhs_indices  device int32 [pairs], the expert of each pair
 *   out          device [pairs, rows_per_entry, n] of type dt: rows
 *                p * rows_per_entry + r = x[lhs[p], r] times expert rhs[p]
 *   sorted_indices  1 asserts that rhs_indices is non-decreasing: the pairs
 *                are then grouped by binary search instead of the routing
 *                sort (same results; an unsorted array gives undefined values)
 *   workspace    nvfp4_gather_qmm_indexed_workspace_size(pairs,
 *                rows_per_entry, e, lhs_indices != NULL) bytes, 256-byte aligned
 * x is used as given; the global scale multiplies the block scale.  The
 * rows of a pair whose expert lies outside [0, e) are written with zeros (with
 * sorted_indices such pairs can only sit at the two ends); an lhs index
 * outside [0, entries) is a precondition violation.
 * transpose = 1 runs the matrix-core kernels of nvfp4_gather_qmm (float16 /
 * bfloat16) or the float32 kernel; transpose = 0 a matrix-core kernel that
 * decodes each weight tile into LDS (float32: the float32 kernel).
 * Errors: bad dtype, non-positive sizes, k (transpose = 1) or n (transpose =
 * 0) not a multiple of 16, k % 8 != 0 with transpose = 0, pairs > entries
 * without lhs_indices, NULL or misaligned pointers, workspace too small,
 * sizes too large, e > 1024.
 */
size_t nvfp4_gather_qmm_indexed_workspace_size(int64_t pairs, int64_t rows_per_entry, int64_t e,
                                               int with_lhs);
nvfp4_status nvfp4_gather_qmm_indexed(const void* x, nvfp4_dtype dt, int64_t entries,
                                      int64_t rows_per_entry, const uint8_t* w_codes,
                                      const uint8_t* w_scales, const float* global_scale_w,
                                      const int32_t* lhs_indices, const int32_t* rhs_indices,
                                      int64_t pairs, int64_t e, int64_t n, int64_t k, int transpose,
                                      int sorted_indices, void* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * The mx modes: mxfp4 and mxfp8 ("mlx 0.30.7.2 -> 0.30.7.6" diff, page 8,
 * fp_quantize / fp_dequantize: group size 32 outside nvfp4, 8 bits for mxfp8
 * and 4 otherwise, scales converted to E8M0 and decoded as 2^(s - 127);
 * validate_global_scale: no global scale outside nvfp4).
 *
 * Format of a quantized tensor [rows, k], k a multiple of 32:
 *   codes   mxfp4: [rows, k/2], e2m1, element 2j in the low nibble of byte j;
 *           mxfp8: [rows, k], one e4m3 byte per element
 *   scales  [rows, k/32], one E8M0 byte per 32 consecutive elements of a row
 * Encode per group of 32 (page 7, fp_quantize_rowwise with use_mx_scale):
 * the group amax, s = the smallest power of two >= amax / maxval (maxval 6 or
 * 448; the float32 quotient rounded UP, clamped to 2^-127 .. 2^127 -- the pull
 * request referenced from the "[Metal] global scale for qmm" page, "mxfp8
 * block scales round up", section "Why"), then each code the nearest value
 * (ties to even, saturating) of x * 2^-s.  Decode T(value(code) * 2^s),
 * exact in float32 before the rounding to T.
 */
typedef enum { NVFP4_MXFP4 = 4, NVFP4_MXFP8 = 8 } nvfp4_mx_mode;

/*
 * nvfp4_mx_quantize -- codes and scales of x [rows, k] in an mx mode.
 *   x        device [rows, k] of type dt, 16-byte aligned
 *   codes    device, written, 16-byte aligned; scales device, written
 * Errors: bad dtype or mode, rows < 0, k not a positive multiple of 32, NULL
 * or misaligned pointer (rows > 0).
 */
nvfp4_status nvfp4_mx_quantize(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode, int64_t rows,
                               int64_t k, uint8_t* codes, uint8_t* scales, hipStream_t stream);

/*
 * nvfp4_mx_dequantize -- T(value(code) * 2^(s - 127)) as [rows, k] of out_dt
 * (16-byte aligned); the codes 16-byte aligned.  Errors as nvfp4_mx_quantize.
 */
nvfp4_status nvfp4_mx_dequantize(const uint8_t* codes, const uint8_t* scales, nvfp4_mx_mode mode,
                                 int64_t rows, int64_t k, void* out, nvfp4_dtype out_dt,
                                 hipStream_t stream);

/*
 * nvfp4_mx_quant_dequant -- the round trip of x in x's type (page 7,
 * fp_quantize_dequantize with use_mx_scale); x_hat 16-byte aligned.
 */
nvfp4_status nvfp4_mx_quant_dequant(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                                    int64_t rows, int64_t k, void* x_hat, hipStream_t stream);

/*
 * Packed mx operands for the block-scaled matrix-core product (gfx950's
 * v_mfma_scale_f32_32x32x64_f8f6f4 consumes the codes and E8M0 scales
 * directly).  Rows in tiles of 32; k in steps of 64, the step count padded to
 * a multiple of 4.  For tile T and step s, P = 2 (mxfp4) or 4 (mxfp8) blocks
 * of 512 bytes; block p holds bytes 16p .. 16p + 15 of the step's row-major
 * codes of rows 32T .. 32T + 31, in row order.  For tile T and quad q of
 * steps, a 256-byte scale block whose byte 4l + j is the scale of row
 * 32T + l % 32, group 2 (4q + j) + l / 32.  Blocks in (T, s) / (T, q) order;
 * padding rows and steps are zero.
 */

/*
 * nvfp4_mx_pack_size -- bytes of the packed codes and scales of a [rows, k]
 * mx operand.  Errors: NULL pointer, bad mode, rows <= 0, k not a positive
 * multiple of 32 (the outputs are then 0).
 */
nvfp4_status nvfp4_mx_pack_size(nvfp4_mx_mode mode, int64_t rows, int64_t k, size_t* codes_bytes,
                                size_t* scales_bytes);

/*
 * nvfp4_mx_pack -- write the packed copy of row-major mx codes and scales.
 * codes and packed_codes 16-byte aligned.  Errors as nvfp4_mx_pack_size, NULL
 * or misaligned pointers.
 */
nvfp4_status nvfp4_mx_pack(const uint8_t* codes, const uint8_t* scales, nvfp4_mx_mode mode,
                           int64_t rows, int64_t k, uint8_t* packed_codes, uint8_t* packed_scales,
                           hipStream_t stream);

/*
 * nvfp4_mx_quantize_packed -- quantize x [rows, k] (type dt, 16-byte aligned)
 * in an mx mode straight into the packed layout (the same bytes as
 * nvfp4_mx_quantize followed by nvfp4_mx_pack); packed_codes 16-byte aligned,
 * sizes from nvfp4_mx_pack_size.  Errors as nvfp4_mx_quantize, rows <= 0.
 */
nvfp4_status nvfp4_mx_quantize_packed(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                                      int64_t rows, int64_t k, uint8_t* packed_codes,
                                      uint8_t* packed_scales, hipStream_t stream);

/*
 * nvfp4_mx_mm_packed -- out [m, n] (type out_dt, 16-byte aligned) = the
 * block-scaled product of two packed mx operands, x [m, k] and w [n, k] in
 * the same mode: out = T( sum_k x_hat[m, k] * w_hat[n, k] ), the products of
 * the decodes exact in float32, summed in float32.  nvfp4_mx_qqmm_packed is
 * nvfp4_mx_quantize_packed of x followed by this call.
 * Errors: bad mode or dtype, m, n <= 0, k not a positive multiple of 32, NULL
 * or misaligned pointer, a packed operand of 2 GB or more.
 */
nvfp4_status nvfp4_mx_mm_packed(const uint8_t* x_packed_codes, const uint8_t* x_packed_scales,
                                const uint8_t* w_packed_codes, const uint8_t* w_packed_scales,
                                nvfp4_mx_mode mode, int64_t m, int64_t n, int64_t k, void* out,
                                nvfp4_dtype out_dt, hipStream_t stream);

/*
 * nvfp4_mx_qqmm_workspace_size -- bytes of workspace nvfp4_mx_qqmm (packed_w
 * = 0) or nvfp4_mx_qqmm_packed (packed_w = 1) needs: x's packed codes and
 * scales, and for a row-major weight its packed copy, each 256-byte aligned.
 * 0 for invalid sizes, and 0 for nvfp4_mx_qqmm with m = 1 and at most 8 KB
 * of codes per row (the matrix-vector kernel uses none).
 */
size_t nvfp4_mx_qqmm_workspace_size(nvfp4_mx_mode mode, int64_t m, int64_t n, int64_t k,
                                    int packed_w);

/*
 * nvfp4_mx_qqmm -- out [m, n] = T( sum_k x_hat[m, k] * w_hat[n, k] ) in an mx
 * mode: x [m, k] of type dt (float32, float16, bfloat16) is quantized in the
 * same mode (page 8, qqmm: the mode selects both operands' group size and
 * scale type), w is given quantized [n, k]; the products of the two decodes
 * are exact in float32 and summed in float32 by the matrix cores; out of
 * type dt.  nvfp4_mx_qqmm_packed takes the weight as its packed copy.  With
 * one row of x (m = 1) and a row of at most 8 KB of codes (k <= 16384 for
 * mxfp4, 8192 for mxfp8), nvfp4_mx_qqmm runs a matrix-vector kernel on the
 * row-major weight instead: per group of 32 the code values' dot product
 * (exact products, float32 sums) times both groups' scales.
 *   x        device, 16-byte aligned
 *   w_codes  device, 16-byte aligned (row-major) / packed copy
 *   out      device [m, n], 16-byte aligned
 *   workspace  device, nvfp4_mx_qqmm_workspace_size() bytes, 256-byte aligned
 *            (may be NULL when that size is 0)
 * Errors: bad dtype or mode, m, n <= 0, k not a positive multiple of 32, NULL
 * or misaligned pointer, workspace too small, operands too large (a packed
 * operand of 2 GB or more).
 */
nvfp4_status nvfp4_mx_qqmm(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                           const uint8_t* w_codes, const uint8_t* w_scales, int64_t m, int64_t n,
                           int64_t k, void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);
nvfp4_status nvfp4_mx_qqmm_packed(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                                  const uint8_t* packed_codes, const uint8_t* packed_scales,
                                  int64_t m, int64_t n, int64_t k, void* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_mx_gather_qmm -- nvfp4_gather_qmm with per-expert weights in an mx
 * mode (the gather_qmm op takes the same mode argument as the other
 * quantized products, "mlx 0.30.7.2 -> 0.30.7.6" diff page 8; the mx decode
 * of fp_dequantize there, no global scale):
 *     out[t, j, :] = T( x[t, :] @ w_hat[idx[t, j]]^T ),
 * w_hat = code value * 2^(s - 127), exact in float32; x used as given.  The
 * pairs are grouped by expert as in nvfp4_gather_qmm; for float16 and
 * bfloat16 x the decoded weights are rounded to T for the matrix cores
 * (exact unless a block scale puts them outside T's normal range), float32
 * x runs a float32 kernel; float32 accumulation.
 *   x           device [t, k] of type dt, 16-byte aligned
 *   w_codes     device uint8 [e, n, k/2] (mxfp4, element 2j in the low
 *               nibble of byte j) or [e, n, k] (mxfp8), 16-byte aligned
 *   w_scales    device uint8 [e, n, k/32], E8M0
 *   expert_idx  device int32 [t, top_k]; a pair whose index lies outside
 *               [0, e) multiplies no expert and its output row is zeros
 *   out         device [t, top_k, n] of type dt, written
 *   workspace   device, nvfp4_gather_qmm_workspace_size(t, top_k, e, n, k)
 *               bytes, 256-byte aligned (the routing tables)
 * Errors: bad dtype or mode, NULL or misaligned pointer, t, top_k, e, n <= 0,
 * k not a positive multiple of 32, workspace too small; UNSUPPORTED for more
 * than 1024 experts, t * top_k >= 2^31, or x or one expert's codes of 2 GB
 * or more.
 */
nvfp4_status nvfp4_mx_gather_qmm(const void* x, nvfp4_dtype dt, nvfp4_mx_mode mode,
                                 const uint8_t* w_codes, const uint8_t* w_scales,
                                 const int32_t* expert_idx, int64_t t, int64_t top_k, int64_t e,
                                 int64_t n, int64_t k, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Test hook: treat every device as having this gcnArchName (NULL restores the
 * real query).  Lets host-only tests reach the unsupported-device error.
 */
void nvfp4_debug_set_arch_override(const char* arch);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
