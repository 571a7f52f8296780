// qmv.hip -- M = 1 NVFP4 matrix-vector product for gfx950:
//     out[n] = T( sum_k x_hat[k] * w[n, k] )
// with x_hat the NVFP4 round trip of x under g_x and w decoded with g_w on
// every block scale ("mlx 0.30.7.2 -> 0.30.7.6" diff page 7,
// QQMatmul::eval_gpu, M == 1 branch; "[Metal] global scale for qmm" PR 4458,
// statement: the global factor belongs inside the dequantization).
//
// The kernel is HBM-bound: the weight stream is 9/16 byte per element and
// nothing is reused, so the design is about keeping enough bytes in flight.
//
// Register path (k = 4096 * CH, CH = 1 or 2 for 16-bit x, 1 for float32):
//   * every wave owns up to R consecutive rows and issues the loads of all of
//     them (per row and lane: CH x 32 code bytes + CH x 4 scale bytes, the
//     lanes of a wave covering each 2 KB chunk of a row contiguously) before
//     doing anything else, so the whole matrix is requested at once;
//   * meanwhile the workgroup rebuilds x_hat = T(dequant(quant(x, g_x))) in
//     LDS (one half group of 8 per lane and chunk) and every lane then keeps
//     the 64 * CH x_hat values of its k slice in registers;
//   * per row, each group of 16 is decoded two codes per instruction
//     (v_cvt_scalef32_pk_*_fp4, exact) and contracted with x_hat two at a time
//     (v_dot2_f32_bf16 / _f16: exact products, float32 sums, or float32 FMAs),
//     and the block's partial sum is multiplied by its effective scale
//     e4m3(s) * g_w/2688 -- the global factor rides on the block scale;
//   * a DPP row reduction plus four lane reads give the row sum.
// Generic path (any k % 16 == 0 up to 32768): one group per lane per sweep,
// x_hat in LDS as float32 padded to 17 words per group (conflict-free reads).
//
// A few rows (qmv_rows_kernel, 1 <= m <= 2 rows of 16-bit x, k = 4096): the
// register path with one accumulator per x row.  The weight stream is the
// same; each decoded code pair feeds m v_dot2 products, so the VALU work per
// weight element grows as 0.5 + 0.5 m instructions while the bytes stay put
// (past two rows it outgrows the stream, and the matrix-core kernels of
// smallm.hip do better).
// x_hat is x's round trip under g_x (qqmm) or x as given (quantized_matmul).
// With m = 1 and the round trip of x done beforehand the sums are qmv's,
// operation for operation.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreadsQ = kWaves * 64;
// Rows per wave on the register path.  Fewer rows per wave means more
// workgroups (896 for n = 14336) and a shorter compute tail after each wave's
// last bytes arrive; all loads are in flight either way.  Measured per launch
// at n = 14336 (cold weights): 1 row 9.0 us, 2 rows 8.3 us, 4 rows 8.45 us,
// 7 rows (one workgroup per CU) 8.9-9.0 us.
constexpr int kMaxRows = 2;
constexpr int kRowsMaxR = 8;  // rows per wave of qmv_rows_kernel

// Partial dot product of one group of 16 (codes in dwords c0, c1) with
// x_hat (16-bit pairs xp[0..7], or floats xf[0..15]).
template <int DT>
__device__ __forceinline__ float group_dot16(uint32_t c0, uint32_t c1, const uint32_t* xp,
                                             const float* xf) {
  if constexpr (DT == kBF16) {
    float p = 0.0f;
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1_decode2_bf16<0>(c0), __builtin_bit_cast(bf16x2, xp[0]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1_decode2_bf16<1>(c0), __builtin_bit_cast(bf16x2, xp[1]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1_decode2_bf16<2>(c0), __builtin_bit_cast(bf16x2, xp[2]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1_decode2_bf16<3>(c0), __builtin_bit_cast(bf16x2, xp[3]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1_decode2_bf16<0>(c1), __builtin_bit_cast(bf16x2, xp[4]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1_decode2_bf16<1>(c1), __builtin_bit_cast(bf16x2, xp[5]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1_decode2_bf16<2>(c1), __builtin_bit_cast(bf16x2, xp[6]), p, false);
    p = __builtin_amdgcn_fdot2_f32_bf16(e2m1_decode2_bf16<3>(c1), __builtin_bit_cast(bf16x2, xp[7]), p, false);
    return p;
  } else if constexpr (DT == kF16) {
    float p = 0.0f;
    p = __builtin_amdgcn_fdot2(e2m1_decode2_f16<0>(c0), __builtin_bit_cast(f16x2, xp[0]), p, false);
    p = __builtin_amdgcn_fdot2(e2m1_decode2_f16<1>(c0), __builtin_bit_cast(f16x2, xp[1]), p, false);
    p = __builtin_amdgcn_fdot2(e2m1_decode2_f16<2>(c0), __builtin_bit_cast(f16x2, xp[2]), p, false);
    p = __builtin_amdgcn_fdot2(e2m1_decode2_f16<3>(c0), __builtin_bit_cast(f16x2, xp[3]), p, false);
    p = __builtin_amdgcn_fdot2(e2m1_decode2_f16<0>(c1), __builtin_bit_cast(f16x2, xp[4]), p, false);
    p = __builtin_amdgcn_fdot2(e2m1_decode2_f16<1>(c1), __builtin_bit_cast(f16x2, xp[5]), p, false);
    p = __builtin_amdgcn_fdot2(e2m1_decode2_f16<2>(c1), __builtin_bit_cast(f16x2, xp[6]), p, false);
    p = __builtin_amdgcn_fdot2(e2m1_decode2_f16<3>(c1), __builtin_bit_cast(f16x2, xp[7]), p, false);
    return p;
  } else {
    float q[16];
    float(&lo)[8] = *reinterpret_cast<float(*)[8]>(q);
    float(&hi)[8] = *reinterpret_cast<float(*)[8]>(q + 8);
    e2m1_decode8_f32(c0, lo);
    e2m1_decode8_f32(c1, hi);
    float p = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) p = __builtin_fmaf(q[i], xf[i], p);
    return p;
  }
}

// ------------------------------------------------------------------ register path

// One 16-byte code load covers 32 elements = 2 groups; its two scale bytes
// come from one 2-byte load.  For chunk c of a row (4096 elements), lane l
// takes the 32 elements at 32 l and at 2048 + 32 l, so each of the two code
// loads of a wave reads 1 KB of contiguous memory.
struct RowPiece {
  u32x4 code;
  uint32_t scale;  // the aligned scale dword holding this piece's two bytes
};

template <int DT, int CH, int R>
__global__ void __launch_bounds__(kThreadsQ)
qmv_reg_kernel(const void* __restrict__ x, const float* __restrict__ gx,
               const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
               const float* __restrict__ gw, int n, void* __restrict__ out) {
  constexpr int K = 4096 * CH;
  constexpr bool kF = (DT == kF32);
  // x_hat in LDS: 16-bit values for 16-bit T, float32 otherwise
  __shared__ __attribute__((aligned(16))) uint32_t xs[kF ? K : K / 2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // 1. this thread's half groups of x (K / 8 = 512 * CH of them), first in the
  //    load queue so that waiting for them leaves the weight loads in flight
  float xv[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c) load8x<DT>(x, tid + kThreadsQ * c, xv[c]);
  __builtin_amdgcn_sched_barrier(0);  // keep the x loads ahead of the weight loads

  // 2. every weight load of this wave's R rows (rows past n re-read row n - 1)
  const int r0 = (blockIdx.x * kWaves + wave) * R;
  RowPiece wp[R][CH][2];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = min(r0 + i, n - 1);
    const uint8_t* crow = wc + (int64_t)r * (K / 2);
    const uint8_t* srow = ws + (int64_t)r * (K / 16);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int e0 = c * 4096 + hh * 2048 + 32 * lane;  // first element
        wp[i][c][hh].code =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + e0 / 2));
        wp[i][c][hh].scale = __builtin_nontemporal_load(
            reinterpret_cast<const uint32_t*>(srow + ((e0 / 16) & ~3)));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // rows arrive in the order they are used
  }

  // 3. x_hat into LDS
  {
    const float enc = global_encode(gx);
    const float dec = global_decode(gx);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int h = tid + kThreadsQ * c;
      float o[8];
      xhat_half_group<DT>(xv[c], enc, dec, o);
      if constexpr (kF) {
        f32x4* p = reinterpret_cast<f32x4*>(xs) + 2 * h;
        p[0] = f32x4{o[0], o[1], o[2], o[3]};
        p[1] = f32x4{o[4], o[5], o[6], o[7]};
      } else {
        using T = typename Elem<DT>::T;
        typedef T T8 __attribute__((ext_vector_type(8)));
        T8 t;
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = from_f32<DT>(o[i]);
        reinterpret_cast<T8*>(xs)[h] = t;
      }
    }
  }
  lds_barrier();  // x_hat written; the weight loads stay in flight

  // 4. this lane's x_hat pieces into registers: 32 elements per piece
  uint32_t xp[CH][2][16];  // 16-bit pairs (16-bit T)
  float xf[CH][2][32];     // float32 values (T = float32)
#pragma unroll
  for (int c = 0; c < CH; ++c) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int e0 = c * 4096 + hh * 2048 + 32 * lane;
      if constexpr (kF) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          f32x4 t = reinterpret_cast<const f32x4*>(xs)[e0 / 4 + q];
          xf[c][hh][4 * q] = t.x; xf[c][hh][4 * q + 1] = t.y;
          xf[c][hh][4 * q + 2] = t.z; xf[c][hh][4 * q + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x4 t = reinterpret_cast<const u32x4*>(xs)[e0 / 8 + q];
          xp[c][hh][4 * q] = t.x; xp[c][hh][4 * q + 1] = t.y;
          xp[c][hh][4 * q + 2] = t.z; xp[c][hh][4 * q + 3] = t.w;
        }
      }
    }
  }

  // 5. rows: group partial sums times e4m3(s) * g_w/2688, then the row sum
  const float dec_w = global_decode(gw);
  const int sshift = 8 * ((2 * lane) & 3);  // this lane's two bytes inside the scale dword
  float rs[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const RowPiece& pc = wp[i][c][hh];
        float se0, se1;
        {
#pragma clang fp contract(off)
          const uint32_t sc = pc.scale >> sshift;
          se0 = e4m3_decode_byte<0>(sc) * dec_w;
          se1 = e4m3_decode_byte<1>(sc) * dec_w;
        }
        float p0 = group_dot16<DT>(pc.code.x, pc.code.y, &xp[c][hh][0], &xf[c][hh][0]);
        float p1 = group_dot16<DT>(pc.code.z, pc.code.w, &xp[c][hh][8], &xf[c][hh][16]);
        acc = __builtin_fmaf(p0, se0, acc);
        acc = __builtin_fmaf(p1, se1, acc);
      }
    }
    rs[i] = wave_sum_uniform(acc);
    __builtin_amdgcn_sched_barrier(0);  // consume rows in load order
  }
  // 6. lane i stores row r0 + i
  float mine = rs[0];
#pragma unroll
  for (int i = 1; i < R; ++i) mine = (lane == i) ? rs[i] : mine;
  if (lane < R && r0 + lane < n) reinterpret_cast<typename Elem<DT>::T*>(out)[r0 + lane] = from_f32<DT>(mine);
}

// ------------------------------------------------------------------ generic path

template <int DT>
__global__ void __launch_bounds__(kThreadsQ)
qmv_generic_kernel(const void* __restrict__ x, const float* __restrict__ gx,
                   const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                   const float* __restrict__ gw, int n, int k, void* __restrict__ out) {
  extern __shared__ float xs[];  // x_hat, group g at words [17 g, 17 g + 16)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int groups = k >> 4;
  {
    const float enc = global_encode(gx);
    const float dec = global_decode(gx);
    const int halves = k >> 3;  // even: pair partners are both in range
    for (int h = threadIdx.x; h < halves; h += kThreadsQ) {
      float v[8], o[8];
      load8x<DT>(x, h, v);
      xhat_half_group<DT>(v, enc, dec, o);
      float* dst = xs + 17 * (h >> 1) + 8 * (h & 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = o[i];
    }
  }
  __syncthreads();

  const float dec_w = global_decode(gw);
  const int total_waves = gridDim.x * kWaves;
  for (int r = blockIdx.x * kWaves + wave; r < n; r += total_waves) {
    const uint8_t* crow = wc + (int64_t)r * (k >> 1);
    const uint8_t* srow = ws + (int64_t)r * groups;
    float acc = 0.0f;
    for (int g = lane; g < groups; g += 64) {
      u32x2 c = *reinterpret_cast<const u32x2*>(crow + (int64_t)g * 8);
      float se;
      {
#pragma clang fp contract(off)
        se = e4m3_decode(srow[g]) * dec_w;
      }
      float q[16];
      float(&lo)[8] = *reinterpret_cast<float(*)[8]>(q);
      float(&hi)[8] = *reinterpret_cast<float(*)[8]>(q + 8);
      e2m1_decode8_f32(c.x, lo);
      e2m1_decode8_f32(c.y, hi);
      const float* xg = xs + 17 * g;
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) p = __builtin_fmaf(q[i], xg[i], p);
      acc = __builtin_fmaf(p, se, acc);
    }
    float s = wave_sum_uniform(acc);
    if (lane == 0) reinterpret_cast<typename Elem<DT>::T*>(out)[r] = from_f32<DT>(s);
  }
}

// ------------------------------------------------------------------ a few x rows

constexpr int kRowsMaxM = 2;

template <int DT> struct Dot2;
template <> struct Dot2<kBF16> {
  using V = bf16x2;
  template <int B> static __device__ __forceinline__ V dec(uint32_t w) { return e2m1_decode2_bf16<B>(w); }
  static __device__ __forceinline__ float dot(V a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), c, false);
  }
};
template <> struct Dot2<kF16> {
  using V = f16x2;
  template <int B> static __device__ __forceinline__ V dec(uint32_t w) { return e2m1_decode2_f16<B>(w); }
  static __device__ __forceinline__ float dot(V a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(f16x2, b), c, false);
  }
};

// Rows of x past m are never computed; their loads read zeros (buffer range).
template <int DT, int R>
__global__ void __launch_bounds__(kThreadsQ)
qmv_rows_kernel(const void* __restrict__ x, int m, bool qx, const float* __restrict__ gx,
                const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                const float* __restrict__ gw, int n, void* __restrict__ out) {
  constexpr int K = 4096;
  constexpr int HPR = K / 8;  // half groups per x row: one per thread
  using T = typename Elem<DT>::T;
  using D = Dot2<DT>;
  __shared__ __attribute__((aligned(16))) u32x4 xs[kRowsMaxM * HPR];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // 1. half group tid of every x row, first in the load queue
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint64_t)m * K * 2);
  u32x4 xr[kRowsMaxM];
#pragma unroll
  for (int j = 0; j < kRowsMaxM; ++j)
    xr[j] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(j * HPR + tid) * 16u, 0, 0));
  __builtin_amdgcn_sched_barrier(0);

  // 2. every weight load of this wave's R rows (rows past n re-read row n - 1)
  const int r0 = (blockIdx.x * kWaves + wave) * R;
  RowPiece wp[R][2];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = min(r0 + i, n - 1);
    const uint8_t* crow = wc + (int64_t)r * (K / 2);
    const uint8_t* srow = ws + (int64_t)r * (K / 16);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int e0 = hh * 2048 + 32 * lane;
      wp[i][hh].code = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(crow + e0 / 2));
      wp[i][hh].scale =
          __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(srow + ((e0 / 16) & ~3)));
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // 3. the x_hat rows into LDS
  {
    const float enc = global_encode(gx);
    const float dec = global_decode(gx);
#pragma unroll
    for (int j = 0; j < kRowsMaxM; ++j) {
      if (j < m) {
        u32x4 v = xr[j];
        if (qx) {
          float f[8], o[8];
          unpack8<DT>(v, f);
          xhat_half_group<DT>(f, enc, dec, o);  // lane pairs hold the two halves of a group
          typedef T T8 __attribute__((ext_vector_type(8)));
          T8 t;
#pragma unroll
          for (int i = 0; i < 8; ++i) t[i] = from_f32<DT>(o[i]);
          v = __builtin_bit_cast(u32x4, t);
        }
        xs[j * HPR + tid] = v;
      }
    }
  }
  lds_barrier();  // the weight loads stay in flight

  // 4. this lane's x_hat pieces (elements 2048 hh + 32 lane .. + 31 of each row)
  uint32_t xp[kRowsMaxM][2][16];
#pragma unroll
  for (int j = 0; j < kRowsMaxM; ++j) {
    if (j < m) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 t = xs[j * HPR + (hh * 2048 + 32 * lane) / 8 + q];
          xp[j][hh][4 * q] = t.x; xp[j][hh][4 * q + 1] = t.y;
          xp[j][hh][4 * q + 2] = t.z; xp[j][hh][4 * q + 3] = t.w;
        }
      }
    }
  }

  // 5. rows: per group, the 8 decoded pairs dotted with each x row, the
  //    partial sums times e4m3(s) * g_w/2688; lane i keeps row r0 + i
  const float dec_w = global_decode(gw);
  const int sshift = 8 * ((2 * lane) & 3);
  float mine[kRowsMaxM];
#pragma unroll
  for (int j = 0; j < kRowsMaxM; ++j) mine[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float acc[kRowsMaxM];
#pragma unroll
    for (int j = 0; j < kRowsMaxM; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const RowPiece& pc = wp[i][hh];
      float se0, se1;
      {
#pragma clang fp contract(off)
        const uint32_t sc = pc.scale >> sshift;
        se0 = e4m3_decode_byte<0>(sc) * dec_w;
        se1 = e4m3_decode_byte<1>(sc) * dec_w;
      }
      const uint32_t cw[4] = {pc.code.x, pc.code.y, pc.code.z, pc.code.w};
      typename D::V d[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        d[4 * u] = D::template dec<0>(cw[u]);
        d[4 * u + 1] = D::template dec<1>(cw[u]);
        d[4 * u + 2] = D::template dec<2>(cw[u]);
        d[4 * u + 3] = D::template dec<3>(cw[u]);
      }
#pragma unroll
      for (int j = 0; j < kRowsMaxM; ++j) {
        if (j < m) {
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int t = 0; t < 8; ++t) p0 = D::dot(d[t], xp[j][hh][t], p0);
#pragma unroll
          for (int t = 0; t < 8; ++t) p1 = D::dot(d[8 + t], xp[j][hh][8 + t], p1);
          acc[j] = __builtin_fmaf(p0, se0, acc[j]);
          acc[j] = __builtin_fmaf(p1, se1, acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kRowsMaxM; ++j) {
      if (j < m) {
        const float v = wave_sum_uniform(acc[j]);
        mine[j] = (lane == i) ? v : mine[j];
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // consume rows in load order
  }
  // 6. lane i stores row r0 + i of every output row
  if (lane < R && r0 + lane < n) {
#pragma unroll
    for (int j = 0; j < kRowsMaxM; ++j)
      if (j < m) reinterpret_cast<T*>(out)[(int64_t)j * n + r0 + lane] = from_f32<DT>(mine[j]);
  }
}

template <int DT, int R>
void launch_rows(const void* x, int m, bool qx, const float* gx, const uint8_t* wc,
                 const uint8_t* ws, const float* gw, int64_t n, void* out, int64_t blocks,
                 hipStream_t s) {
  qmv_rows_kernel<DT, R><<<(int)blocks, kThreadsQ, 0, s>>>(x, m, qx, gx, wc, ws, gw, (int)n, out);
}

template <int DT>
hipError_t launch_rows_t(const void* x, int m, bool qx, const float* gx, const uint8_t* wc,
                         const uint8_t* ws, const float* gw, int64_t n, void* out, hipStream_t s) {
  int64_t blocks = (n + kWaves * kRowsMaxR - 1) / (kWaves * kRowsMaxR);
  if (blocks < 256) blocks = 256;
  const int rpw = (int)((n + blocks * kWaves - 1) / (blocks * kWaves));
  blocks = (n + (int64_t)kWaves * rpw - 1) / ((int64_t)kWaves * rpw);
  switch (rpw) {
    case 1: launch_rows<DT, 1>(x, m, qx, gx, wc, ws, gw, n, out, blocks, s); break;
    case 2: launch_rows<DT, 2>(x, m, qx, gx, wc, ws, gw, n, out, blocks, s); break;
    case 3: launch_rows<DT, 3>(x, m, qx, gx, wc, ws, gw, n, out, blocks, s); break;
    case 4: launch_rows<DT, 4>(x, m, qx, gx, wc, ws, gw, n, out, blocks, s); break;
    case 5: launch_rows<DT, 5>(x, m, qx, gx, wc, ws, gw, n, out, blocks, s); break;
    case 6: launch_rows<DT, 6>(x, m, qx, gx, wc, ws, gw, n, out, blocks, s); break;
    case 7: launch_rows<DT, 7>(x, m, qx, gx, wc, ws, gw, n, out, blocks, s); break;
    default: launch_rows<DT, 8>(x, m, qx, gx, wc, ws, gw, n, out, blocks, s); break;
  }
  return hipGetLastError();
}

template <int DT, int CH, int R>
void launch_reg(const void* x, const float* gx, const uint8_t* wc, const uint8_t* ws,
                const float* gw, int64_t n, void* out, int64_t blocks, hipStream_t s) {
  qmv_reg_kernel<DT, CH, R><<<(int)blocks, kThreadsQ, 0, s>>>(x, gx, wc, ws, gw, (int)n, out);
}

template <int DT, int CH>
void launch_reg_r(int r, const void* x, const float* gx, const uint8_t* wc, const uint8_t* ws,
                  const float* gw, int64_t n, void* out, int64_t blocks, hipStream_t s) {
  switch (r) {
    case 1: launch_reg<DT, CH, 1>(x, gx, wc, ws, gw, n, out, blocks, s); break;
    case 2: launch_reg<DT, CH, 2>(x, gx, wc, ws, gw, n, out, blocks, s); break;
    case 3: launch_reg<DT, CH, 3>(x, gx, wc, ws, gw, n, out, blocks, s); break;
    case 4: launch_reg<DT, CH, 4>(x, gx, wc, ws, gw, n, out, blocks, s); break;
    case 5: launch_reg<DT, CH, 5>(x, gx, wc, ws, gw, n, out, blocks, s); break;
    case 6: launch_reg<DT, CH, 6>(x, gx, wc, ws, gw, n, out, blocks, s); break;
    case 7: launch_reg<DT, CH, 7>(x, gx, wc, ws, gw, n, out, blocks, s); break;
    default: launch_reg<DT, CH, 8>(x, gx, wc, ws, gw, n, out, blocks, s); break;
  }
}

template <int DT>
hipError_t launch_qmv_t(const void* x, const float* gx, const uint8_t* wc, const uint8_t* ws,
                        const float* gw, int64_t n, int64_t k, void* out, hipStream_t s) {
  const int chunks = (k % 4096 == 0) ? (int)(k / 4096) : 0;
  const bool reg_path = chunks == 1 || (chunks == 2 && DT != kF32);
  if (reg_path) {
    // at least one workgroup per CU, at most kMaxRows rows per wave
    int64_t blocks = (n + kWaves * kMaxRows - 1) / (kWaves * kMaxRows);
    if (blocks < 256) blocks = 256;
    const int64_t waves = blocks * kWaves;
    const int rpw = (int)((n + waves - 1) / waves);
    blocks = (n + (int64_t)kWaves * rpw - 1) / ((int64_t)kWaves * rpw);
    if constexpr (DT == kF32) {
      launch_reg_r<DT, 1>(rpw, x, gx, wc, ws, gw, n, out, blocks, s);
    } else {
      if (chunks == 1)
        launch_reg_r<DT, 1>(rpw, x, gx, wc, ws, gw, n, out, blocks, s);
      else
        launch_reg_r<DT, 2>(rpw, x, gx, wc, ws, gw, n, out, blocks, s);
    }
    return hipGetLastError();
  }
  int64_t blocks = (n + kWaves - 1) / kWaves;
  if (blocks > 1024) blocks = 1024;
  size_t lds = (size_t)(k / 16) * 17 * sizeof(float);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(qmv_generic_kernel<DT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  qmv_generic_kernel<DT><<<(int)blocks, kThreadsQ, lds, s>>>(x, gx, wc, ws, gw, (int)n, (int)k, out);
  return hipGetLastError();
}

}  // namespace

bool qmv_rows_ok(int dt, int64_t m, int64_t n, int64_t k) {
  return (dt == kBF16 || dt == kF16) && m >= 1 && m <= kRowsMaxM && k == 4096 && n >= 1 &&
         n < 0x7FFFFFFF;
}

hipError_t launch_qmv_rows(const void* x, int dt, int64_t m, bool quantize_x, const float* gx,
                           const uint8_t* wc, const uint8_t* ws, const float* gw, int64_t n,
                           void* out, hipStream_t s) {
  return dt == kF16 ? launch_rows_t<kF16>(x, (int)m, quantize_x, gx, wc, ws, gw, n, out, s)
                    : launch_rows_t<kBF16>(x, (int)m, quantize_x, gx, wc, ws, gw, n, out, s);
}

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
