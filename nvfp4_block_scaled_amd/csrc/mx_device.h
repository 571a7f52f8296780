// mx_device.h -- device helpers of the mx modes (mxfp4, mxfp8) shared by the
// mx codec (mx_codec.hip) and the mx matrix-vector product (mx_qmv.hip):
// the group scale, the codes of 8 values and their decode.  The steps are
// those of the pages' rowwise quantize with an E8M0 scale ("mlx 0.30.7.2 ->
// 0.30.7.6" diff, page 7, fp_quantize_rowwise with use_mx_scale; page 8,
// fp_quantize / fp_dequantize; the E8M0 round-up of the pull request
// referenced from "[Metal] global scale for qmm").
#pragma once

#include "nvfp4_device.h"

namespace nvfp4 {

template <int BITS> struct MxFormat;
template <> struct MxFormat<4> {
  static constexpr float kMax = kE2M1Max;
  static constexpr int kPieces = 2;  // 16-byte pieces per row and 64-wide step
};
template <> struct MxFormat<8> {
  static constexpr float kMax = kE4M3Max;
  static constexpr int kPieces = 4;
};

// Scale byte and encode factor of a group with amax `a`.
template <int BITS>
__device__ __forceinline__ uint32_t mx_scale(float a, float& enc_b) {
#pragma clang fp contract(off)
  const uint32_t s = e8m0_encode_up(a / MxFormat<BITS>::kMax);
  enc_b = e8m0_inverse(s);
  return s;
}

// Codes of 8 values times enc_b: one dword of 8 nibbles (mxfp4) or two
// dwords of 8 bytes (mxfp8), element order.
__device__ __forceinline__ uint32_t mx_codes4(const float (&v)[8], float enc_b) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
    y[i] = v[i] * enc_b;
  }
  return e2m1_encode8(y);
}
__device__ __forceinline__ u32x2 mx_codes8(const float (&v)[8], float enc_b) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y;
    {
#pragma clang fp contract(off)
      y = v[i] * enc_b;
    }
    w[i / 4] |= e4m3_encode_signed(y) << (8 * (i % 4));
  }
  return u32x2{w[0], w[1]};
}

// Values of 8 codes (as encoded above) times the scale 2^(s - 127).
__device__ __forceinline__ void mx_values4(uint32_t w, float sc, float (&o)[8]) {
  float q[8];
  e2m1_decode8_f32(w, q);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
    o[i] = q[i] * sc;
  }
}
__device__ __forceinline__ void mx_values8(u32x2 w, float sc, float (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
    o[i] = e4m3_decode((i < 4 ? w.x : w.y) >> (8 * (i % 4))) * sc;
  }
}

}  // namespace nvfp4
