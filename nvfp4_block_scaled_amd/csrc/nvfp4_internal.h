// nvfp4_internal.h -- host-side launchers shared between the C ABI layer and
// the kernel translation units.  Each launcher enqueues on `s` and returns the
// HIP status of the launch; argument validation happens in capi.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

// codec.hip
hipError_t launch_tensor_amax(const void* x, int dt, int64_t n, float* out, hipStream_t s);
hipError_t launch_quantize(const void* x, int dt, int64_t rows, int64_t k, const float* g,
                           uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_quant_dequant(const void* x, int dt, int64_t rows, int64_t k, const float* g,
                                void* xhat, hipStream_t s);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                             const float* g, void* out, int dt, hipStream_t s);
// quantize x [rows, cols] along rows (the transpose's encode): codes
// [cols, rows/2] and scales [cols, rows/16], or x_hat of the transpose
// [cols, rows]; rows % 16 == 0, cols % 8 == 0 (16-bit) / % 4 == 0 (float32)
hipError_t launch_quantize_colwise(const void* x, int dt, int64_t rows, int64_t cols, const float* g,
                                   uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_quant_dequant_colwise(const void* x, int dt, int64_t rows, int64_t cols,
                                        const float* g, void* xhat_t, hipStream_t s);

// qmv.hip
constexpr int64_t kQmvMaxK = 32768;
hipError_t launch_qmv(const void* x, int dt, const float* gx, const uint8_t* wc,
                      const uint8_t* ws, const float* gw, int64_t n, int64_t k, void* out,
                      hipStream_t s);
// 1 <= m <= 2 rows of 16-bit x, k = 4096, row-major weight: x_hat [m, k] @ w^T
// with x_hat x's round trip under gx (quantize_x) or x as given
bool qmv_rows_ok(int dt, int64_t m, int64_t n, int64_t k);
hipError_t launch_qmv_rows(const void* x, int dt, int64_t m, bool quantize_x, const float* gx,
                           const uint8_t* wc, const uint8_t* ws, const float* gw, int64_t n,
                           void* out, hipStream_t s);

// qmv_packed.hip: qqmm with 1 <= m <= 4 rows of bfloat16 x against the packed
// weight, 512 <= k <= 8192 (k % 64 == 0), on the fp4 matrix cores
bool qmv_packed_ok(int dt, int64_t m, int64_t k);
hipError_t launch_qmv_packed(const void* x, int dt, int64_t m, const float* gx, const uint8_t* pc,
                             const uint8_t* ps, const float* gw, int64_t n, int64_t k, void* out,
                             hipStream_t s);

// gemm.hip
hipError_t launch_qqmm_gemm(const void* xhat, int dt, const uint8_t* wc, const uint8_t* ws,
                            const float* gw, int64_t m, int64_t n, int64_t k, void* out,
                            hipStream_t s);
// routing: row q (of entries * rows_per_entry) goes to expert idx[q / rows_per_entry];
// offsets [e + 1], perm [rows] (rows with an expert outside [0, e) at
// perm[offsets[e] ..]); scratch of route_scratch_bytes(rows, e); with zero_out,
// zeros to row q (row_bytes bytes) of zero_out for every such row
size_t route_scratch_bytes(int64_t rows, int64_t e);
hipError_t launch_moe_route(const int32_t* idx, int64_t entries, int64_t rows_per_entry, int64_t e,
                            int32_t* offsets, int32_t* perm, int32_t* scratch, void* zero_out,
                            int64_t row_bytes, hipStream_t s);
// gather contraction over `rows` routed rows: the A row of routed row s is
// amap[s] when amap is given, else perm[s] / top_k; its output row perm[s];
// x holds x_rows rows
hipError_t launch_gather_gemm(const void* x, int dt, const uint8_t* wc, const uint8_t* ws,
                              const float* gw, const int32_t* offsets, const int32_t* perm,
                              int64_t x_rows, int64_t rows, int64_t top_k, const int32_t* amap,
                              int64_t e, int64_t n, int64_t k, void* out, hipStream_t s);
hipError_t launch_gather_gemm_t_f32(const float* x, const uint8_t* wc, const uint8_t* ws,
                                   const float* gw, const int32_t* offsets, const int32_t* perm,
                                   int64_t rows, int64_t top_k, const int32_t* amap, int64_t e,
                                   int64_t n, int64_t k, float* out, hipStream_t s);
// the same contraction (no x-row map) on row-major mx weights: mode 4 (mxfp4
// codes [e, n, k/2]) or 8 (mxfp8 codes [e, n, k]), E8M0 scales [e, n, k/32],
// k % 32 == 0
hipError_t launch_mx_gather_gemm(const void* x, int dt, int mode, const uint8_t* wc, const uint8_t* ws,
                                 const int32_t* offsets, const int32_t* perm, int64_t x_rows,
                                 int64_t rows, int64_t top_k, int64_t e, int64_t n, int64_t k,
                                 void* out, hipStream_t s);
// the packed weight layout of the matrix-core path (gemm.hip, mfma_pack_kernel)
constexpr int64_t kPackK = 64;             // k must be a multiple of this
constexpr int64_t kPackCodeBytes = 1024;   // per 32-row tile and 64-wide k-step
constexpr int64_t kPackScaleBytes = 128;
hipError_t launch_mfma_pack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                            uint8_t* pc, uint8_t* ps, hipStream_t s);
hipError_t launch_qqmm_gemm_packed(const void* xhat, int dt, const uint8_t* pc, const uint8_t* ps,
                                   const float* gw, int64_t m, int64_t n, int64_t k, void* out,
                                   hipStream_t s);
hipError_t launch_gather_gemm_packed(const void* x, int dt, const uint8_t* pc, const uint8_t* ps,
                                     const float* gw, const int32_t* offsets, const int32_t* perm,
                                     int64_t x_rows, int64_t rows, int64_t top_k, const int32_t* amap,
                                     int64_t e, int64_t n, int64_t k, void* out, hipStream_t s);

// gather_ex.hip: routing of sorted expert indices (offsets by binary search,
// identity permutation), the x-row map of lhs indices, and the contraction
// with weights [e, K, N] quantized along N (transpose = False; K % 8 == 0)
hipError_t launch_sorted_route(const int32_t* rhs, int64_t pairs, int64_t mr, int64_t e,
                               int32_t* offsets, int32_t* perm, void* zero_out, int64_t row_bytes,
                               hipStream_t s);
hipError_t launch_amap(const int32_t* perm, const int32_t* lhs, int64_t rows, int64_t mr, int32_t* amap,
                       hipStream_t s);
hipError_t launch_gather_gemm_t(const void* x, int dt, const uint8_t* wc, const uint8_t* ws,
                                const float* gw, const int32_t* offsets, const int32_t* perm,
                                int64_t x_rows, int64_t rows, int64_t top_k, const int32_t* amap,
                                int64_t e, int64_t n, int64_t k, void* out, hipStream_t s);

// compute units of the current device (cached per device)
int device_cu_count();

// smallm.hip: 1 <= m <= kSmallMaxM rows of x, 16-bit x, k % 128 == 0, with x
// and its padding in LDS (m (k + 8) 2 bytes plus 7 KB within kSmallMaxLds)
// and the weight's codes below 2 GB
constexpr int64_t kSmallMaxM = 16;
constexpr size_t kSmallMaxLds = 160 * 1024;
bool small_m_ok(int dt, bool packed, int64_t m, int64_t n, int64_t k);
hipError_t launch_small_m(const void* x, int dt, bool quantize_x, const float* gx,
                          const uint8_t* wc, const uint8_t* ws, bool packed, const float* gw,
                          int64_t m, int64_t n, int64_t k, void* out, hipStream_t s);

// mx_codec.hip / mx_gemm.hip: the mx modes (bits 4 = mxfp4, 8 = mxfp8), k % 32
// == 0.  Packed operand layout: rows padded to tiles of 32, k to quads of
// four 64-wide steps (mx_packed_quads quads).
int64_t mx_packed_quads(int64_t k);
size_t mx_packed_code_bytes(int64_t rows, int64_t k, int bits);
size_t mx_packed_scale_bytes(int64_t rows, int64_t k);
hipError_t launch_mx_quantize(const void* x, int dt, int bits, int64_t rows, int64_t k,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_mx_quant_dequant(const void* x, int dt, int bits, int64_t rows, int64_t k,
                                   void* xhat, hipStream_t s);
hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int bits, int64_t rows,
                                int64_t k, void* out, int dt, hipStream_t s);
hipError_t launch_mx_quantize_packed(const void* x, int dt, int bits, int64_t rows, int64_t k,
                                     uint8_t* pc, uint8_t* ps, hipStream_t s);
hipError_t launch_mx_pack(const uint8_t* codes, const uint8_t* scales, int bits, int64_t rows,
                          int64_t k, uint8_t* pc, uint8_t* ps, hipStream_t s);
// y [m, n] of type dt from the packed x (m rows) and w (n rows); the packed
// mx_qmv.hip: qqmm in an mx mode (4 or 8) with one row of x, k % 32 == 0 and
// at most 8 KB of codes per row, row-major weight codes [n, k * mode / 8] and
// scales [n, k / 32]
bool mx_qmv_ok(int mode, int64_t m, int64_t n, int64_t k);
hipError_t launch_mx_qmv(const void* x, int dt, int mode, const uint8_t* wc, const uint8_t* ws,
                         int64_t n, int64_t k, void* out, hipStream_t s);
// operands must be below kMxMaxPackedBytes
constexpr size_t kMxMaxPackedBytes = 0x7F000000u;
hipError_t launch_mx_gemm(const uint8_t* xpc, const uint8_t* xps, const uint8_t* wpc,
                          const uint8_t* wps, int bits, int64_t m, int64_t n, int64_t k, void* out,
                          int dt, hipStream_t s);

}  // namespace nvfp4
