// nvfp4_device.h -- device-side building blocks of the NVFP4 kernels (gfx950).
//
// Formats (the pages fix them through their constants F4E2M1_MAX = 6 and
// F8E4M3_MAX = 448, "mlx 0.30.7.2 -> 0.30.7.6" diff, page 7, fp_quantize.cu):
//   e2m1  4-bit code s.ee.m, exponent bias 1, exponent 0 subnormal (step 0.5);
//         magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
//   e4m3  8-bit s.eeee.mmm, bias 7, exponent 0 subnormal (m * 2^-9), largest
//         finite 448 (0x7E), 0x7F / 0xFF NaN.
// Both encoders round to nearest, ties to even, and saturate; a value that
// rounds to zero keeps its sign (e2m1 code 0x8).
//
// Layout of a quantized tensor [rows, k] (k a multiple of 16): codes
// [rows, k/2] bytes with element 2j in the low nibble of byte j, scales
// [rows, k/16] e4m3 bytes, one per 16 consecutive elements of a row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;
constexpr int kGroup = 16;

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// ----------------------------------------------------------------- element types

template <int DT> struct Elem;
template <> struct Elem<kF32> { using T = float; };
template <> struct Elem<kF16> { using T = _Float16; };
template <> struct Elem<kBF16> { using T = __bf16; };

// Round-to-nearest-even conversion of float to the element type (gfx950
// v_cvt_pk_bf16_f32 / v_cvt_f16_f32 under the default round mode).  For
// float16 the value first passes an empty asm: left alone, the compiler
// merges a float32 multiply and the conversion that follows into one
// v_fma_mix (one rounding, straight to float16), whatever the contraction
// setting of the multiply.  The pages round to float32 first and then to
// the element type; where the float32 product lands on a float16 midpoint
// the two differ (seen: 77 of 2048 elements of an x round trip under one
// g_x, every element sharing the offending block scale and code).
template <int DT>
__device__ __forceinline__ typename Elem<DT>::T from_f32(float v) {
  if constexpr (DT == kF16) asm("" : "+v"(v));
  return static_cast<typename Elem<DT>::T>(v);
}
template <int DT>
__device__ __forceinline__ float to_f32(typename Elem<DT>::T v) {
  return static_cast<float>(v);
}

// ----------------------------------------------------------------- global scale

// Global encode factor 2688/g and decode factor g/2688, each one correctly
// rounded float32 division; 1 without a global scale ("mlx 0.30.7.2 ->
// 0.30.7.6" diff page 7, fp_quantize_rowwise and fp_dequantize; page 8,
// fp_dequantize fallback).
__device__ __forceinline__ float global_encode(const float* g) {
#pragma clang fp contract(off)
  return g ? (kE4M3Max * kE2M1Max) / *g : 1.0f;
}
__device__ __forceinline__ float global_decode(const float* g) {
#pragma clang fp contract(off)
  return g ? *g / (kE4M3Max * kE2M1Max) : 1.0f;
}

// ----------------------------------------------------------------- e4m3

// Decode an e4m3 byte (the low byte of b; v_cvt_f32_fp8 decodes gfx950's
// OCP E4M3 exactly, including the subnormals m * 2^-9 and NaN for 0x7F/0xFF).
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}
// Decode byte B of a dword of scales.
template <int B>
__device__ __forceinline__ float e4m3_decode_byte(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, B);
}

// Encode v >= 0 to e4m3: nearest, ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float v) {
  if (!(v < kE4M3Max)) return 0x7Eu;
  if (v < 0.015625f) {  // below 2^-6: the subnormal grid has step 2^-9
    return (uint32_t)__builtin_rintf(v * 512.0f);
  }
  uint32_t u = __float_as_uint(v);
  uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;  // keep 3 fraction bits
  return r - (120u << 3);                                   // rebias 127 -> 7
}

// ----------------------------------------------------------------- e2m1

// Encode y to an e2m1 code: nearest grid value, ties to the even code,
// |y| > 6 saturates to 6, the sign bit of y is kept.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
  float a = __builtin_fabsf(y);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(y) >> 28) & 8u);
}

// Value of an e2m1 code (low 4 bits of c) as float.
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  uint32_t m = c & 7u;
  // m >= 2: exponent (m >> 1) - 1, fraction bit m & 1; m == 1: 0.5; m == 0: 0
  uint32_t bits = (m >= 2u) ? ((m + 252u) << 22) : (m ? 0x3F000000u : 0u);
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// ----------------------------------------------------------------- gfx950 conversions
//
// v_cvt_scalef32_pk_* convert two e2m1 values to or from a wider type.  Their
// scale operand contributes only its exponent (a power of two, as for MX
// block scales), so every call here passes 1.0 and the NVFP4 block scale is
// applied with an ordinary float32 multiply.  With unit scale the encode is
// round-to-nearest-even with saturation at 6 and keeps the sign of zero,
// which equals e2m1_encode above for every float32 input; the decodes are
// exact.  Element 2j of a byte is its low nibble.

// Encode 8 values into the 8 nibbles of a dword (element i in bits 4i..4i+3).
__device__ __forceinline__ uint32_t e2m1_encode8(const float (&y)[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// Decode the two nibbles of byte B of w.
template <int B>
__device__ __forceinline__ f32x2 e2m1_decode2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}
template <int B>
__device__ __forceinline__ bf16x2 e2m1_decode2_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B);
}
template <int B>
__device__ __forceinline__ f16x2 e2m1_decode2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B);
}

// Decode the 8 nibbles of a dword to float32.
__device__ __forceinline__ void e2m1_decode8_f32(uint32_t w, float (&v)[8]) {
  f32x2 a = e2m1_decode2_f32<0>(w), b = e2m1_decode2_f32<1>(w);
  f32x2 c = e2m1_decode2_f32<2>(w), d = e2m1_decode2_f32<3>(w);
  v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
  v[4] = c.x; v[5] = c.y; v[6] = d.x; v[7] = d.y;
}

// ----------------------------------------------------------------- group encode

// Encode one group of 16 ("mlx 0.30.7.2 -> 0.30.7.6" diff page 7,
// fp_quantize_rowwise): from the block amax, the decode scale (amax / 6) * enc
// stored as e4m3, and the block encode factor enc / float(scale) (0 when the
// scale is 0, so such a block encodes to signed zeros); each value is then
// multiplied by that factor and rounded to e2m1.  Float32 throughout, no
// contraction.
struct GroupScale {
  uint32_t byte;
  float enc_b;
};

__device__ __forceinline__ GroupScale group_scale_from_amax(float amax, float enc) {
#pragma clang fp contract(off)
  float sd = (amax / kE2M1Max) * enc;
  uint32_t s = e4m3_encode_nonneg(sd);
  float sf = e4m3_decode(s);
  GroupScale gs;
  gs.byte = s;
  gs.enc_b = (sf == 0.0f) ? 0.0f : enc / sf;
  return gs;
}

__device__ __forceinline__ uint32_t e2m1_encode_scaled(float x, float enc_b) {
#pragma clang fp contract(off)
  return e2m1_encode(x * enc_b);
}

// Encode 8 values of a half group whose group amax is `amax`: returns the 8
// codes as one dword and sets `byte` to the group's scale byte.
__device__ __forceinline__ uint32_t encode_half_group(const float (&v)[8], float amax, float enc,
                                                      uint32_t& byte) {
  GroupScale gs = group_scale_from_amax(amax, enc);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
    y[i] = v[i] * gs.enc_b;
  }
  byte = gs.byte;
  return e2m1_encode8(y);
}

// ----------------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over the 64 lanes, returned as a wave-uniform value: four DPP steps
// reduce each row of 16 lanes (xor 1, xor 2, half-row mirror, row mirror),
// then the four row sums are read from lanes 0, 16, 32 and 48.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// ----------------------------------------------------------------- x round trip

// Load 8 consecutive elements (half group h, elements 8h .. 8h + 7) of x as floats.
// 8 16-bit values (4 dwords, element 2i in the low half of dword i) as floats.
template <int DT>
__device__ __forceinline__ void unpack8(u32x4 w, float (&v)[8]) {
  const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == kBF16) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
    } else {
      f16x2 hv = __builtin_bit_cast(f16x2, q[i]);
      v[2 * i] = (float)hv.x;
      v[2 * i + 1] = (float)hv.y;
    }
  }
}

template <int DT>
__device__ __forceinline__ void load8x(const void* base, int64_t h, float (&v)[8]) {
  if constexpr (DT == kF32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(base) + 2 * h;
    f32x4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    unpack8<DT>(reinterpret_cast<const u32x4*>(base)[h], v);
  }
}

// Streaming load of 8 consecutive elements of type DT (element 8h ..) as
// floats (nontemporal: the data is read once).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t h, float (&v)[8]) {
  if constexpr (DT == kF32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(base) + 2 * h;
    f32x4 a = __builtin_nontemporal_load(p);
    f32x4 b = __builtin_nontemporal_load(p + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + h);
    uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == kBF16) {
        v[2 * i] = __uint_as_float(q[i] << 16);
        v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
      } else {
        f16x2 hv = __builtin_bit_cast(f16x2, q[i]);
        v[2 * i] = (float)hv.x;
        v[2 * i + 1] = (float)hv.y;
      }
    }
  }
}

// Store 8 floats as type DT at element 8h.
template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t h, const float (&v)[8]) {
  if constexpr (DT == kF32) {
    f32x4* p = reinterpret_cast<f32x4*>(base) + 2 * h;
    p[0] = f32x4{v[0], v[1], v[2], v[3]};
    p[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    using T = typename Elem<DT>::T;
    typedef T T8 __attribute__((ext_vector_type(8)));
    T8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = from_f32<DT>(v[i]);
    reinterpret_cast<T8*>(base)[h] = o;
  }
}

// x_hat of one half group (8 values at element 8h), rounded to T, as floats.
// The pair partner (lane ^ 1) holds the other half of the group.
template <int DT>
__device__ __forceinline__ void xhat_half_group(const float (&v)[8], float enc, float dec,
                                                float (&o)[8]) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
  a = fmaxf(a, __shfl_xor(a, 1, 64));
  uint32_t byte;
  uint32_t codes = encode_half_group(v, a, enc, byte);
  float sc;
  {
#pragma clang fp contract(off)
    sc = e4m3_decode(byte) * dec;
  }
  float q[8];
  e2m1_decode8_f32(codes, q);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
    o[i] = to_f32<DT>(from_f32<DT>(q[i] * sc));
  }
}

// ----------------------------------------------------------------- weight decode to 16-bit

// Two 16-bit values (element 2j low) from two floats.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  using T = typename Elem<DT>::T;
  typedef T T2 __attribute__((ext_vector_type(2)));
  T2 v;
  v[0] = from_f32<DT>(a);
  v[1] = from_f32<DT>(b);
  return __builtin_bit_cast(uint32_t, v);
}

// Dword P of a decoded weight fragment: the two codes of byte P of the code
// word, times the effective block scale, as two 16-bit values.
template <int DT, int P>
__device__ __forceinline__ uint32_t decode_dword(uint32_t codes, float se) {
  const f32x2 v = e2m1_decode2_f32<P>(codes);
  float a, b;
  {
#pragma clang fp contract(off)
    a = v.x * se;
    b = v.y * se;
  }
  return pack2<DT>(a, b);
}

// ----------------------------------------------------------------- E8M0 (mx modes)
//
// The mx modes' block scale: byte b stands for 2^(b - 127), 0xFF for NaN
// ("mlx 0.30.7.2 -> 0.30.7.6" diff page 8, fp_dequantize fallback).  The
// encode rounds up: the smallest power of two >= v (the pull request
// referenced from the "[Metal] global scale for qmm" page, "mxfp8 block
// scales round up", section "Why"), clamped to 2^-127 .. 2^127.

// v >= 0 (finite): the biased exponent, plus one when any fraction bit is
// set; 2^-127 and below (zero included) give byte 0.
__device__ __forceinline__ uint32_t e8m0_encode_up(float v) {
  const uint32_t u = __float_as_uint(v);
  if (u <= 0x00400000u) return 0u;
  const uint32_t b = (u >> 23) + ((u & 0x7FFFFFu) ? 1u : 0u);
  return b > 254u ? 254u : b;
}

// 2^(b - 127) for b in 0..254 (2^-127 is the float32 subnormal 0x00400000),
// NaN for 255: the bits b << 23, plus bit 22 for bytes 0 and 255 (those
// with (b + 1) & 0xFF below 2).  Plain integer arithmetic, no compare: a
// select on a just-loaded byte may be compiled into a branch, which the
// hand-scheduled matrix-core loops must not contain.
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  const uint32_t special = (((b + 1u) & 0xFFu) - 2u) >> 31;  // 1 for b = 0 and b = 255
  return __uint_as_float((b << 23) | (special << 22));
}

// 1 / 2^(b - 127) = 2^(127 - b), exact, for b in 0..254.
__device__ __forceinline__ float e8m0_inverse(uint32_t b) {
  return b == 254u ? __uint_as_float(0x00400000u) : __uint_as_float((254u - b) << 23);
}

// e4m3 code of a float32 of either sign (nearest, ties to even, saturating at
// +-448, the sign bit kept, also for zero).
__device__ __forceinline__ uint32_t e4m3_encode_signed(float y) {
  return e4m3_encode_nonneg(__builtin_fabsf(y)) | ((__float_as_uint(y) >> 24) & 0x80u);
}

// ----------------------------------------------------------------- buffer resources

// A raw buffer resource over `bytes` bytes (32-bit data format, no swizzle,
// range checked: loads past the end return zeros).
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const int n = bytes >= 0xFFFFFFFFull ? -1 : (int)(uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRsrcWord3);
}

// ----------------------------------------------------------------- output rows

// Zeros to output row q of `out` (row_bytes bytes per row), written by the
// whole wave: the rows of gather pairs whose expert lies outside [0, e).
__device__ __forceinline__ void zero_row_wave(uint8_t* __restrict__ out, int64_t q, int64_t row_bytes) {
  uint8_t* row = out + q * row_bytes;
  const int lane = threadIdx.x & 63;
  if ((row_bytes & 15) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0) {
    for (int64_t o = 16 * lane; o < row_bytes; o += 1024)
      *reinterpret_cast<u32x4*>(row + o) = u32x4{0u, 0u, 0u, 0u};
  } else {
    for (int64_t o = 2 * lane; o < row_bytes; o += 128) *reinterpret_cast<uint16_t*>(row + o) = 0;
  }
}

// ----------------------------------------------------------------- barriers

// LDS barrier without a memory fence: finish this wave's LDS operations, then
// meet the other waves.  The "memory" clobber keeps the compiler from moving
// memory accesses across it; outstanding global loads stay in flight (a
// __syncthreads() would first wait for all of them).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace nvfp4
