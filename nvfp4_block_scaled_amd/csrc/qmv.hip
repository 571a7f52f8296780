// qmv.hip -- M = 1 NVFP4 matrix-vector product for gfx950:
//     out[n] = T( sum_k x_hat[k] * w[n, k] )
// with x_hat the NVFP4 round trip of x under g_x and w decoded with g_w on
// every block scale ("mlx 0.30.7.2 -> 0.30.7.6" diff page 7,
// QQMatmul::eval_gpu, M == 1 branch; "[Metal] global scale for qmm" PR 4458,
// statement: the global factor belongs inside the dequantization).
//
// Design (HBM-bound: the weight stream is 9/16 byte per element):
//   * every workgroup first rebuilds x_hat from x (k/8 half groups spread over
//     its 512 lanes) into LDS as float32; the first weight rows are already in
//     flight while it does so;
//   * each wave then owns a contiguous range of rows; for a row, lane l holds
//     GPL consecutive groups of 16 (GPL = 4: 32 B of codes + 4 B of scales,
//     two 16-byte loads and one dword), so one wave reads a 4096-wide row in
//     one coalesced sweep;
//   * the block partial sum_i x_hat_i * e2m1(q_i) is formed in float32 and
//     multiplied by the block's effective scale e4m3(s) * g_w/2688, i.e. the
//     global factor sits on the block scale as in the pages;
//   * a wave-wide reduction and one store per row.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreadsQ = kWaves * 64;

template <int DT>
__device__ __forceinline__ void load8x(const void* base, int64_t h, float (&v)[8]) {
  if constexpr (DT == kF32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(base) + 2 * h;
    f32x4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    u32x4 w = reinterpret_cast<const u32x4*>(base)[h];
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

// Sum over one group of 16 of x_hat_i * e2m1(q_i); codes lo/hi hold the 16
// nibbles (element 2j in the low nibble of byte j).
__device__ __forceinline__ float group_dot(const float* xg, uint32_t lo, uint32_t hi) {
  float p = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) p = __builtin_fmaf(xg[i], e2m1_decode(lo >> (4 * i)), p);
#pragma unroll
  for (int i = 0; i < 8; ++i) p = __builtin_fmaf(xg[8 + i], e2m1_decode(hi >> (4 * i)), p);
  return p;
}

template <int DT, int GPL>
__global__ void __launch_bounds__(kThreadsQ)
qmv_kernel(const void* __restrict__ x, const float* __restrict__ gx,
           const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
           const float* __restrict__ gw, int n, int k, void* __restrict__ out) {
  extern __shared__ float xs[];  // x_hat, k floats
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int groups = k >> 4;

  // ---- x_hat = dequantize(quantize(x, g_x), g_x), rounded to T, into LDS
  {
    const float enc = global_encode(gx);
    const float dec = global_decode(gx);
    const int halves = k >> 3;  // even
    for (int h = threadIdx.x; h < halves; h += kThreadsQ) {
      float v[8];
      load8x<DT>(x, h, v);
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(v[i]));
      a = fmaxf(a, __shfl_xor(a, 1, 64));
      GroupScale gs = group_scale_from_amax(a, enc);
      float sc;
      {
#pragma clang fp contract(off)
        sc = e4m3_decode(gs.byte) * dec;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
        float o = e2m1_decode(e2m1_encode_scaled(v[i], gs.enc_b)) * sc;
        xs[8 * h + i] = to_f32<DT>(from_f32<DT>(o));
      }
    }
  }
  __syncthreads();

  const float dec_w = global_decode(gw);
  const int total_waves = gridDim.x * kWaves;
  const int gwave = blockIdx.x * kWaves + wave;
  const int rpw = (n + total_waves - 1) / total_waves;
  const int r0 = gwave * rpw;
  const int r1 = min(n, r0 + rpw);
  const int per_step = 64 * GPL;  // groups covered by one wave sweep

  for (int r = r0; r < r1; ++r) {
    const uint8_t* crow = wc + (int64_t)r * (k >> 1);
    const uint8_t* srow = ws + (int64_t)r * groups;
    float acc = 0.0f;
    for (int g0 = 0; g0 < groups; g0 += per_step) {
      const int gb = g0 + lane * GPL;
      if constexpr (GPL == 4) {
        // groups gb..gb+3: 32 code bytes, 4 scale bytes
        const u32x4* cp = reinterpret_cast<const u32x4*>(crow + (int64_t)gb * 8);
        u32x4 c0 = __builtin_nontemporal_load(cp);
        u32x4 c1 = __builtin_nontemporal_load(cp + 1);
        uint32_t sw = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(srow + gb));
        uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float se;
          {
#pragma clang fp contract(off)
            se = e4m3_decode((sw >> (8 * j)) & 0xFFu) * dec_w;
          }
          float p = group_dot(xs + (gb + j) * 16, cw[2 * j], cw[2 * j + 1]);
          acc = __builtin_fmaf(p, se, acc);
        }
      } else {
        if (gb < groups) {
          u32x2 c = *reinterpret_cast<const u32x2*>(crow + (int64_t)gb * 8);
          float se;
          {
#pragma clang fp contract(off)
            se = e4m3_decode(srow[gb]) * dec_w;
          }
          float p = group_dot(xs + gb * 16, c.x, c.y);
          acc = __builtin_fmaf(p, se, acc);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) reinterpret_cast<typename Elem<DT>::T*>(out)[r] = from_f32<DT>(acc);
  }
}

template <int DT>
hipError_t launch_qmv_t(const void* x, const float* gx, const uint8_t* wc, const uint8_t* ws,
                        const float* gw, int64_t n, int64_t k, void* out, hipStream_t s) {
  // aim for ~7 rows per wave, at most one workgroup per row group
  int64_t blocks = (n + kWaves * 7 - 1) / (kWaves * 7);
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  size_t lds = (size_t)k * sizeof(float);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(k % 4096 == 0 ? qmv_kernel<DT, 4> : qmv_kernel<DT, 1>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (k % 4096 == 0)
    qmv_kernel<DT, 4><<<(int)blocks, kThreadsQ, lds, s>>>(x, gx, wc, ws, gw, (int)n, (int)k, out);
  else
    qmv_kernel<DT, 1><<<(int)blocks, kThreadsQ, lds, s>>>(x, gx, wc, ws, gw, (int)n, (int)k, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qmv(const void* x, int dt, const float* gx, const uint8_t* wc,
                      const uint8_t* ws, const float* gw, int64_t n, int64_t k, void* out,
                      hipStream_t s) {
  switch (dt) {
    case kF32: return launch_qmv_t<kF32>(x, gx, wc, ws, gw, n, k, out, s);
    case kF16: return launch_qmv_t<kF16>(x, gx, wc, ws, gw, n, k, out, s);
    default: return launch_qmv_t<kBF16>(x, gx, wc, ws, gw, n, k, out, s);
  }
}

}  // namespace nvfp4
