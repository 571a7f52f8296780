// mx_qmv.hip -- the mx modes' matrix-vector product for gfx950: qqmm in
// mxfp4 / mxfp8 with one row of x,
//     out[n] = T( sum_k x_hat[k] * w_hat[n, k] ),
// x_hat the mx round trip of x (its own E8M0 scale per group of 32) and w_hat
// the decode of the mx weight, both kept as float32 values, not rounded to T
// ("mlx 0.30.7.2 -> 0.30.7.6" diff, page 8, qqmm with the fp modes; page 7,
// QQMatmul::eval_gpu and the matrix-vector path of the fp modes).
//
// HBM-bound like the NVFP4 qmv, with the same design: every wave owns up to R
// consecutive weight rows and issues all of their loads first; meanwhile the
// workgroup quantizes x into LDS; then each lane keeps its pieces of x in
// registers.  Load j of a wave reads bytes 1024 j .. + 1023 of a row's codes,
// 16 per lane: a whole group of 32 (mxfp4) or half of one (mxfp8).  A row of
// k * BITS / 8 bytes takes NP = 1, 2, 4 or 8 such loads (the smallest that
// covers it); lanes past the row's end load nothing and add zero, so any k %
// 32 == 0 up to 8 KB of codes per row runs here (k <= 16384 for mxfp4, 8192
// for mxfp8).  FULL instances (rows of exactly NP KB, k = 4096 among them)
// leave those checks out, so that the loads are one straight run.  Within a piece both operands carry one power-of-two scale each,
// so the piece's partial sum runs over the unscaled code values (exact bf16
// values -- e2m1 or e4m3 -- in v_dot2_f32_bf16, whose products are exact,
// float32 sums) and is then multiplied by 2^(s_w - 127) and by 2^(s_x - 127),
// both exact scalings of a float32.
#include "mx_device.h"
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kMxqWaves = 8;
constexpr int kMxqThreads = 64 * kMxqWaves;
constexpr int kMxqMaxRows = 2;      // rows per wave: more, shorter waves (as the NVFP4 qmv)
constexpr int kMxqMaxRowBytes = 8192;  // NP = 8 pieces of 1 KB

// Per row and lane: NP pieces of 16 code bytes, EP = 128 / BITS elements
// each (32 = a group for mxfp4, 16 = half a group for mxfp8), and the
// piece's scale byte.
template <int BITS> struct MxqShape {
  static constexpr int EP = 128 / BITS;  // elements per piece
  static constexpr int PP = EP / 2;      // bf16 pairs per piece
};
struct MxqPiece {
  u32x4 c;
  uint32_t s;
};

// The bf16 pairs of a piece's codes, element order.
template <int BITS>
__device__ __forceinline__ void mxq_pairs(u32x4 cv, bf16x2 (&d)[MxqShape<BITS>::PP]) {
  const uint32_t c[4] = {cv.x, cv.y, cv.z, cv.w};
  if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d[4 * i] = e2m1_decode2_bf16<0>(c[i]);
      d[4 * i + 1] = e2m1_decode2_bf16<1>(c[i]);
      d[4 * i + 2] = e2m1_decode2_bf16<2>(c[i]);
      d[4 * i + 3] = e2m1_decode2_bf16<3>(c[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, false);
      d[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.0f, true);
    }
  }
}

template <int DT, int BITS, int R, int NP, bool FULL>
__global__ void __launch_bounds__(kMxqThreads)
mx_qmv_kernel(const void* __restrict__ x, const uint8_t* __restrict__ wc,
              const uint8_t* __restrict__ ws, int n, int k, void* __restrict__ out) {
  constexpr int KMAX = NP * 1024 * 8 / BITS;         // elements of the longest row covered
  constexpr int XC = KMAX >= 4096 ? KMAX / 4096 : 1;  // quarter groups of x per thread
  constexpr int EP = MxqShape<BITS>::EP, PP = MxqShape<BITS>::PP;
  __shared__ __attribute__((aligned(16))) u32x4 xq[KMAX / 8];  // x's code values as bf16, 8 per entry
  __shared__ float xsc[KMAX / 32];                              // x's group scales 2^(s - 127)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row_bytes = FULL ? NP * 1024 : k * BITS / 8;
  const int quarters = FULL ? KMAX / 8 : k / 8;  // quarter groups of x

  // 1. this thread's quarter groups of x, tid + 512 c, first in the queue
  float xv[XC][8];
#pragma unroll
  for (int c = 0; c < XC; ++c) {
    const int q = tid + kMxqThreads * c;
    if ((FULL && KMAX >= 4096) || q < quarters) {
      load8x<DT>(x, q, xv[c]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[c][i] = 0.0f;
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. every weight load of this wave's R rows (rows past n re-read row n - 1;
  //    pieces past the row's end load nothing: zero codes, scale 2^0)
  const int r0 = (blockIdx.x * kMxqWaves + wave) * R;
  MxqPiece wp[R][NP];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = min(r0 + i, n - 1);
    const uint8_t* crow = wc + (int64_t)r * row_bytes;
    const uint8_t* srow = ws + (int64_t)r * (k / 32);
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int e0 = EP * (64 * j + lane);  // first element of the piece
      if (FULL || 1024 * j + 16 * lane < row_bytes) {
        wp[i][j].c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + 1024 * j + 16 * lane));
        wp[i][j].s = __builtin_nontemporal_load(srow + e0 / 32);
      } else {
        wp[i][j].c = u32x4{0u, 0u, 0u, 0u};
        wp[i][j].s = 127u;
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // rows arrive in the order they are used
  }

  // 3. the mx round trip of x: the group amax over the four lanes of a group,
  //    the E8M0 scale, the codes; their values (unscaled) into LDS as bf16
#pragma unroll
  for (int c = 0; c < XC; ++c) {
    const int q = tid + kMxqThreads * c;
    const float (&xc)[8] = xv[c];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, __builtin_fabsf(xc[i]));
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    a = fmaxf(a, __shfl_xor(a, 2, 64));
    float enc_b;
    const uint32_t s = mx_scale<BITS>(a, enc_b);
    u32x4 t;
    if constexpr (BITS == 4) {
      const uint32_t w = mx_codes4(xc, enc_b);
      t.x = __builtin_bit_cast(uint32_t, e2m1_decode2_bf16<0>(w));
      t.y = __builtin_bit_cast(uint32_t, e2m1_decode2_bf16<1>(w));
      t.z = __builtin_bit_cast(uint32_t, e2m1_decode2_bf16<2>(w));
      t.w = __builtin_bit_cast(uint32_t, e2m1_decode2_bf16<3>(w));
    } else {
      const u32x2 w = mx_codes8(xc, enc_b);
      t.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
      t.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
      t.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
      t.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
    }
    if ((FULL && KMAX >= 4096) || q < quarters) {
      xq[q] = t;
      if ((q & 3) == 0) xsc[q >> 2] = e8m0_value(s);
    }
  }
  lds_barrier();  // the weight loads stay in flight

  // 4. this lane's pieces of x: code values and scales
  uint32_t xp[NP][PP];
  float sx[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int e0 = EP * (64 * j + lane);
    const bool in = FULL || 1024 * j + 16 * lane < row_bytes;
#pragma unroll
    for (int q = 0; q < EP / 8; ++q) {
      const u32x4 t = in ? xq[e0 / 8 + q] : u32x4{0u, 0u, 0u, 0u};
      xp[j][4 * q] = t.x;
      xp[j][4 * q + 1] = t.y;
      xp[j][4 * q + 2] = t.z;
      xp[j][4 * q + 3] = t.w;
    }
    sx[j] = in ? xsc[e0 / 32] : 1.0f;
  }

  // 5. rows: per group the code-value dot product, times 2^(s_w - 127) and
  //    2^(s_x - 127); lane i keeps row r0 + i
  float mine = 0.0f;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      bf16x2 d[PP];
      mxq_pairs<BITS>(wp[i][j].c, d);
      float p = 0.0f;
#pragma unroll
      for (int u = 0; u < PP; ++u)
        p = __builtin_amdgcn_fdot2_f32_bf16(d[u], __builtin_bit_cast(bf16x2, xp[j][u]), p, false);
      float t;
      {
#pragma clang fp contract(off)
        t = p * e8m0_value(wp[i][j].s & 0xFFu);
      }
      acc = __builtin_fmaf(t, sx[j], acc);
    }
    const float v = wave_sum_uniform(acc);
    mine = (lane == i) ? v : mine;
    __builtin_amdgcn_sched_barrier(0);  // consume rows in load order
  }
  if (lane < R && r0 + lane < n) reinterpret_cast<typename Elem<DT>::T*>(out)[r0 + lane] = from_f32<DT>(mine);
}

template <int DT, int BITS, int R>
void launch_r(const void* x, const uint8_t* wc, const uint8_t* ws, int64_t n, int64_t k, void* out,
              int64_t blocks, hipStream_t s) {
  const int64_t row_bytes = k * BITS / 8;
  const int np = row_bytes <= 1024 ? 1 : row_bytes <= 2048 ? 2 : row_bytes <= 4096 ? 4 : 8;
  const bool full = row_bytes == 1024 * np;
#define NVFP4_MXQ(P)                                                                                 \
  if (full)                                                                                         \
    mx_qmv_kernel<DT, BITS, R, P, true><<<(int)blocks, kMxqThreads, 0, s>>>(x, wc, ws, (int)n, (int)k, \
                                                                            out);                    \
  else                                                                                              \
    mx_qmv_kernel<DT, BITS, R, P, false><<<(int)blocks, kMxqThreads, 0, s>>>(x, wc, ws, (int)n,        \
                                                                             (int)k, out)
  switch (np) {
    case 1: NVFP4_MXQ(1); break;
    case 2: NVFP4_MXQ(2); break;
    case 4: NVFP4_MXQ(4); break;
    default: NVFP4_MXQ(8); break;
  }
#undef NVFP4_MXQ
}

template <int DT, int BITS>
hipError_t launch_t(const void* x, const uint8_t* wc, const uint8_t* ws, int64_t n, int64_t k,
                    void* out, hipStream_t s) {
  // at least one workgroup per CU, at most kMxqMaxRows rows per wave
  int64_t blocks = (n + kMxqWaves * kMxqMaxRows - 1) / (kMxqWaves * kMxqMaxRows);
  if (blocks < 256) blocks = 256;
  const int rpw = (int)((n + blocks * kMxqWaves - 1) / (blocks * kMxqWaves));
  static_assert(kMxqMaxRows == 2, "one or two rows per wave");
  blocks = (n + (int64_t)kMxqWaves * rpw - 1) / ((int64_t)kMxqWaves * rpw);
  if (rpw == 1)
    launch_r<DT, BITS, 1>(x, wc, ws, n, k, out, blocks, s);
  else
    launch_r<DT, BITS, 2>(x, wc, ws, n, k, out, blocks, s);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const void* x, int dt, const uint8_t* wc, const uint8_t* ws, int64_t n,
                       int64_t k, void* out, hipStream_t s) {
  switch (dt) {
    case kF32: return launch_t<kF32, BITS>(x, wc, ws, n, k, out, s);
    case kF16: return launch_t<kF16, BITS>(x, wc, ws, n, k, out, s);
    default: return launch_t<kBF16, BITS>(x, wc, ws, n, k, out, s);
  }
}

}  // namespace

bool mx_qmv_ok(int mode, int64_t m, int64_t n, int64_t k) {
  return m == 1 && k > 0 && k % 32 == 0 && k * mode / 8 <= kMxqMaxRowBytes && n >= 1 && n < 0x7FFFFFFF;
}

hipError_t launch_mx_qmv(const void* x, int dt, int mode, const uint8_t* wc, const uint8_t* ws,
                         int64_t n, int64_t k, void* out, hipStream_t s) {
  return mode == 8 ? launch_bits<8>(x, dt, wc, ws, n, k, out, s)
                   : launch_bits<4>(x, dt, wc, ws, n, k, out, s);
}

}  // namespace nvfp4
