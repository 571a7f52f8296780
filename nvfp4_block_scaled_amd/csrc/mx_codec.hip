// mx_codec.hip -- quantize, dequantize and quantize-dequantize of the mx
// modes (mxfp4, mxfp8) for gfx950, and the packed operand layout of the
// block-scaled matrix-core product (mx_gemm.hip).
//
// The modes ("mlx 0.30.7.2 -> 0.30.7.6" diff, page 8, fp_quantize and
// fp_dequantize; page 7, fp_quantize_rowwise / fp_quantize_dequantize with
// use_mx_scale): groups of 32 consecutive elements of a row, one E8M0 scale
// byte per group, e2m1 codes (mxfp4, element 2j in the low nibble of byte j)
// or e4m3 codes (mxfp8, one byte per element), no global scale.  Per group:
// the amax, the scale s = E8M0 round-up of amax / maxval (maxval 6 or 448, a
// float32 division), enc_b = 2^(127 - s), each code that of x * enc_b; the
// decode is T(value(code) * 2^(s - 127)), whose product is exact in float32.
//
// Row-major layout: codes [rows, k/2] (mxfp4) or [rows, k] (mxfp8), scales
// [rows, k/32].  Kernels on it walk the tensor in 8-element pieces, one lane
// each and four lanes per group (the group amax over the four with two lane
// swaps), so every load and store instruction of a wave is contiguous.
//
// Packed layout, the operand format of the block-scaled product: rows in
// tiles of 32, k in steps of 64, the steps padded to a multiple of 4.  Per
// tile and step, P = 2 (mxfp4) or 4 (mxfp8) blocks of 512 bytes; block p
// holds piece p (row-major code bytes 16p .. 16p + 15 of the step) of the 32
// rows in row order.  Per tile and quad of 4 steps, a 256-byte scale block
// whose dword l holds in byte j the scale of row l % 32, group 2 (4q + j) +
// l / 32.  Padding rows and steps hold zero codes and zero scale bytes, which
// decode to zero.
#include "mx_device.h"
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ row-major quantize

// Lane h covers elements 8h .. 8h + 7 of the flat tensor (group h / 4).
// MODE 0 writes codes and scales, MODE 1 the round trip x_hat in the input
// type.  The four lanes of a group always run the same iterations: the
// stride is a multiple of 4 and so is the piece count.
template <int DT, int BITS, int MODE>
__device__ __forceinline__ void mx_quantize_piece(const float (&v)[8], int64_t h,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales,
                                                  void* __restrict__ xhat) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
  a = fmaxf(a, __shfl_xor(a, 1, 64));
  a = fmaxf(a, __shfl_xor(a, 2, 64));
  float enc_b;
  const uint32_t s = mx_scale<BITS>(a, enc_b);
  float o[8];
  if constexpr (BITS == 4) {
    const uint32_t w = mx_codes4(v, enc_b);
    if constexpr (MODE == 0)
      reinterpret_cast<uint32_t*>(codes)[h] = w;
    else
      mx_values4(w, e8m0_value(s), o);
  } else {
    const u32x2 w = mx_codes8(v, enc_b);
    if constexpr (MODE == 0)
      reinterpret_cast<u32x2*>(codes)[h] = w;
    else
      mx_values8(w, e8m0_value(s), o);
  }
  if constexpr (MODE == 0) {
    if ((h & 3) == 0) scales[h >> 2] = (uint8_t)s;
  } else {
    store8<DT>(xhat, h, o);
  }
}

template <int DT, int BITS, int MODE>
__global__ void __launch_bounds__(kThreads)
mx_quantize_kernel(const void* __restrict__ x, int64_t pieces, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ scales, void* __restrict__ xhat) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; h + stride < pieces; h += 2 * stride) {
    float v[8], u[8];
    load8<DT>(x, h, v);
    load8<DT>(x, h + stride, u);
    mx_quantize_piece<DT, BITS, MODE>(v, h, codes, scales, xhat);
    mx_quantize_piece<DT, BITS, MODE>(u, h + stride, codes, scales, xhat);
  }
  if (h < pieces) {
    float v[8];
    load8<DT>(x, h, v);
    mx_quantize_piece<DT, BITS, MODE>(v, h, codes, scales, xhat);
  }
}

// ------------------------------------------------------------------ row-major dequantize

template <int DT, int BITS>
__global__ void __launch_bounds__(kThreads)
mx_dequantize_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                     int64_t pieces, void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t h = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; h < pieces; h += stride) {
    const float sc = e8m0_value(scales[h >> 2]);
    float o[8];
    if constexpr (BITS == 4)
      mx_values4(reinterpret_cast<const uint32_t*>(codes)[h], sc, o);
    else
      mx_values8(reinterpret_cast<const u32x2*>(codes)[h], sc, o);
    store8<DT>(out, h, o);
  }
}

// ------------------------------------------------------------------ packed layout

// One thread per (row, group) of the padded operand: 32 consecutive threads
// take the 32 rows of a tile at one group, so each 16-byte piece store of a
// wave half fills a whole 512-byte block.
struct PackedIndex {
  int64_t row;
  int64_t group;  // group index along k (0 .. 8 KQ - 1)
  int64_t code_off;  // byte offset of the group's first 16-byte piece
  int64_t scale_off;
};

template <int BITS>
__device__ __forceinline__ PackedIndex packed_index(int64_t t, int KQ) {
  const int64_t gp = 8 * (int64_t)KQ;  // padded groups per row
  const int64_t rt = t / (32 * gp), rem = t % (32 * gp);
  const int64_t g = rem / 32, i = rem % 32;
  const int64_t ks = g / 2, half = g % 2;
  PackedIndex p;
  p.row = 32 * rt + i;
  p.group = g;
  // mxfp4: piece `half` of the step; mxfp8: pieces 2 half and 2 half + 1
  p.code_off = ((rt * 4 * KQ + ks) * MxFormat<BITS>::kPieces + (BITS == 4 ? half : 2 * half)) * 512 +
               16 * i;
  p.scale_off = (rt * KQ + ks / 4) * 256 + 4 * (i + 32 * half) + ks % 4;
  return p;
}

// Quantize x [rows, k] straight into the packed layout (the activation
// operand of the block-scaled product).
template <int DT, int BITS>
__global__ void __launch_bounds__(kThreads)
mx_quantize_packed_kernel(const void* __restrict__ x, int64_t rows, int64_t k, int KQ,
                          int64_t threads, uint8_t* __restrict__ pc, uint8_t* __restrict__ ps) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= threads) return;
  const PackedIndex p = packed_index<BITS>(t, KQ);
  float v[4][8];
  if (p.row < rows && p.group < k / 32) {
    const int64_t first = (p.row * k + 32 * p.group) / 8;  // 8-element piece index
#pragma unroll
    for (int j = 0; j < 4; ++j) load8<DT>(x, first + j, v[j]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[j][e] = 0.0f;
  }
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, __builtin_fabsf(v[j][e]));
  float enc_b;
  const uint32_t s = mx_scale<BITS>(a, enc_b);
  if constexpr (BITS == 4) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = mx_codes4(v[j], enc_b);
    *reinterpret_cast<u32x4*>(pc + p.code_off) = w;
  } else {
    u32x4 w0, w1;
    {
      const u32x2 a0 = mx_codes8(v[0], enc_b), a1 = mx_codes8(v[1], enc_b);
      const u32x2 a2 = mx_codes8(v[2], enc_b), a3 = mx_codes8(v[3], enc_b);
      w0 = u32x4{a0.x, a0.y, a1.x, a1.y};
      w1 = u32x4{a2.x, a2.y, a3.x, a3.y};
    }
    *reinterpret_cast<u32x4*>(pc + p.code_off) = w0;
    *reinterpret_cast<u32x4*>(pc + p.code_off + 512) = w1;
  }
  ps[p.scale_off] = (uint8_t)s;
}

// Row-major codes and scales -> the packed layout (the weight operand).
template <int BITS>
__global__ void __launch_bounds__(kThreads)
mx_pack_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t rows,
               int64_t k, int KQ, int64_t threads, uint8_t* __restrict__ pc,
               uint8_t* __restrict__ ps) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= threads) return;
  const PackedIndex p = packed_index<BITS>(t, KQ);
  constexpr int kBytes = BITS == 4 ? 16 : 32;  // code bytes per group
  u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
  uint8_t sb = 0;
  if (p.row < rows && p.group < k / 32) {
    const uint8_t* src = codes + (p.row * (k / 32) + p.group) * kBytes;
    lo = *reinterpret_cast<const u32x4*>(src);
    if constexpr (BITS == 8) hi = *reinterpret_cast<const u32x4*>(src + 16);
    sb = scales[p.row * (k / 32) + p.group];
  }
  *reinterpret_cast<u32x4*>(pc + p.code_off) = lo;
  if constexpr (BITS == 8) *reinterpret_cast<u32x4*>(pc + p.code_off + 512) = hi;
  ps[p.scale_off] = sb;
}

int blocks_for(int64_t units) {
  const int64_t b = (units + kThreads - 1) / kThreads;
  return (int)(b < 1024 * 16 ? b : 1024 * 16);
}

}  // namespace

// ------------------------------------------------------------------ launchers

int64_t mx_packed_quads(int64_t k) { return (k + 255) / 256; }

size_t mx_packed_code_bytes(int64_t rows, int64_t k, int bits) {
  return (size_t)((rows + 31) / 32) * (size_t)(4 * mx_packed_quads(k)) * (bits == 4 ? 2 : 4) * 512;
}

size_t mx_packed_scale_bytes(int64_t rows, int64_t k) {
  return (size_t)((rows + 31) / 32) * (size_t)mx_packed_quads(k) * 256;
}

#define MX_DISPATCH(DT, BITS, CALL)                     \
  do {                                                  \
    if (BITS == 4) {                                    \
      if (DT == kF32) CALL(kF32, 4);                    \
      else if (DT == kF16) CALL(kF16, 4);               \
      else CALL(kBF16, 4);                              \
    } else {                                            \
      if (DT == kF32) CALL(kF32, 8);                    \
      else if (DT == kF16) CALL(kF16, 8);               \
      else CALL(kBF16, 8);                              \
    }                                                   \
  } while (0)

hipError_t launch_mx_quantize(const void* x, int dt, int bits, int64_t rows, int64_t k,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t pieces = rows * k / 8;
  if (pieces == 0) return hipSuccess;
  const int blocks = blocks_for(pieces / 2 > 0 ? pieces / 2 : 1);
#define MX_Q(D, B) mx_quantize_kernel<D, B, 0><<<blocks, kThreads, 0, s>>>(x, pieces, codes, scales, nullptr)
  MX_DISPATCH(dt, bits, MX_Q);
#undef MX_Q
  return hipGetLastError();
}

hipError_t launch_mx_quant_dequant(const void* x, int dt, int bits, int64_t rows, int64_t k,
                                   void* xhat, hipStream_t s) {
  const int64_t pieces = rows * k / 8;
  if (pieces == 0) return hipSuccess;
  const int blocks = blocks_for(pieces / 2 > 0 ? pieces / 2 : 1);
#define MX_QD(D, B) mx_quantize_kernel<D, B, 1><<<blocks, kThreads, 0, s>>>(x, pieces, nullptr, nullptr, xhat)
  MX_DISPATCH(dt, bits, MX_QD);
#undef MX_QD
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int bits, int64_t rows,
                                int64_t k, void* out, int dt, hipStream_t s) {
  const int64_t pieces = rows * k / 8;
  if (pieces == 0) return hipSuccess;
  const int blocks = blocks_for(pieces);
#define MX_DQ(D, B) mx_dequantize_kernel<D, B><<<blocks, kThreads, 0, s>>>(codes, scales, pieces, out)
  MX_DISPATCH(dt, bits, MX_DQ);
#undef MX_DQ
  return hipGetLastError();
}

hipError_t launch_mx_quantize_packed(const void* x, int dt, int bits, int64_t rows, int64_t k,
                                     uint8_t* pc, uint8_t* ps, hipStream_t s) {
  const int KQ = (int)mx_packed_quads(k);
  const int64_t threads = ((rows + 31) / 32) * 32 * 8 * (int64_t)KQ;
  if (threads == 0) return hipSuccess;
  const int blocks = (int)((threads + kThreads - 1) / kThreads);
#define MX_QP(D, B) \
  mx_quantize_packed_kernel<D, B><<<blocks, kThreads, 0, s>>>(x, rows, k, KQ, threads, pc, ps)
  MX_DISPATCH(dt, bits, MX_QP);
#undef MX_QP
  return hipGetLastError();
}

hipError_t launch_mx_pack(const uint8_t* codes, const uint8_t* scales, int bits, int64_t rows,
                          int64_t k, uint8_t* pc, uint8_t* ps, hipStream_t s) {
  const int KQ = (int)mx_packed_quads(k);
  const int64_t threads = ((rows + 31) / 32) * 32 * 8 * (int64_t)KQ;
  if (threads == 0) return hipSuccess;
  const int blocks = (int)((threads + kThreads - 1) / kThreads);
  if (bits == 4)
    mx_pack_kernel<4><<<blocks, kThreads, 0, s>>>(codes, scales, rows, k, KQ, threads, pc, ps);
  else
    mx_pack_kernel<8><<<blocks, kThreads, 0, s>>>(codes, scales, rows, k, KQ, threads, pc, ps);
  return hipGetLastError();
}

}  // namespace nvfp4
