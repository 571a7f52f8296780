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
// Streaming path (16-bit x, k = 4096; qmv_stream_kernel): one 16-wave
// workgroup per compute unit, each wave up to kStreamRows consecutive rows.
//   * a compute unit streams at the rate its loads in flight allow (their
//     number per unit is bounded), so the rows are split evenly over the
//     workgroups first (56 each at n = 14336) and then over their waves;
//     giving whole waves 4 rows and the rest 3 left half the units with 64
//     rows and half with 48 (measured: 7.5 us per launch);
//   * the global scales and x are the first loads of every wave, and a
//     barrier puts every such load of the workgroup ahead of its weight
//     loads: a vector load issued behind a compute unit's weight stream
//     returns only after most of that stream (measured: x_hat ready 3.5-4 us
//     into a 7.5 us kernel when it was loaded after the weights);
//   * each wave then issues one row, builds x_hat for its share of x (a
//     quarter group of 4 elements per lane, the whole vector per workgroup),
//     and after the workgroup barrier reads its x_hat pieces, issues two
//     more rows, and from then on computes a row and issues the row
//     kStreamAhead further.  A compute unit accepts only so many weight loads
//     in flight; a wave issuing beyond that stalls, so the row loads are
//     spread over the loop instead of all issued up front, and x_hat is
//     built while only one row per wave is in flight (measured at n = 14336:
//     7.5 us per launch, against 8.45 us with rows 1 and 2 issued ahead of
//     the barrier);
//   * a row is 3 loads: two 1 KB code runs and its 256 scale bytes (one
//     dword per lane; each lane's two scale bytes per piece come from the
//     lane holding them, ds_bpermute);
//   * the arithmetic per row is the register path's below, operation for
//     operation, so both give the same bits.
// Register path (float32 x with k = 4096, 16-bit x with k = 8192):
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
// A few rows (1 <= m <= 2 rows of 16-bit x, k = 4096; qmv_stream_kernel with
// MR = 2): the streaming path with one accumulator per x row.  The weight
// stream is the same; each decoded code pair feeds one v_dot2 per row, so the
// VALU work per weight element grows as 0.5 + 0.5 m instructions while the
// bytes stay put (past two rows it outgrows the stream, and the matrix-core
// kernels of smallm.hip do better).  Measured at n = 14336 (cold weights):
// qqmm with two rows 9.5 us, against 12.1 us for the register design that
// issued all of a wave's rows up front.  x_hat is x's round trip under g_x
// (qqmm) or x as given (quantized_matmul); row j's sums are those of qmv on
// x_hat row j, operation for operation.
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


// ------------------------------------------------------------------ streaming path

constexpr int kStreamWaves = 16;
constexpr int kStreamThreads = kStreamWaves * 64;
constexpr int kStreamRows = 4;   // rows per wave at most
constexpr int kStreamAhead = 3;  // rows in flight per wave in the loop

// One row of the streaming path: lane l's 32 elements at 32 l and 2048 +
// 32 l (two 1 KB runs per wave) and scale bytes 4 l .. 4 l + 3 of the row.
struct StreamRow {
  u32x4 code[2];
  uint32_t scale;
};

// exact e2m1 pair decode and 16-bit dot product of one x type
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

// Two e2m1 codes times the 16-bit pairs at xp of MR rows of x_hat (each
// decoded pair feeds one v_dot2 per row; row j's sum is group_dot16's).
template <int DT, int MR>
__device__ __forceinline__ void group_dot16_rows(uint32_t c0, uint32_t c1, const uint32_t (*xp)[2][16],
                                                 int hh, int off, float (&p)[MR]) {
  using D = Dot2<DT>;
#pragma unroll
  for (int j = 0; j < MR; ++j) p[j] = 0.0f;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint32_t w = b < 4 ? c0 : c1;
    typename D::V d;
    switch (b & 3) {
      case 0: d = D::template dec<0>(w); break;
      case 1: d = D::template dec<1>(w); break;
      case 2: d = D::template dec<2>(w); break;
      default: d = D::template dec<3>(w); break;
    }
#pragma unroll
    for (int j = 0; j < MR; ++j) p[j] = D::dot(d, xp[j][hh][off + b], p[j]);
  }
}

// MR rows of x (MR = 1: qmv; MR = 2: two-row qqmm / quantized_matmul, rows
// past m read zeros and are not stored); QX: x goes through the round trip
// (else it is taken as given)
template <int DT, int MR, bool QX>
__global__ void __launch_bounds__(kStreamThreads)
qmv_stream_kernel(const void* __restrict__ x, int m, const float* __restrict__ gx,
                  const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                  const float* __restrict__ gw, int n, int qw, int remw, void* __restrict__ out) {
  constexpr int K = 4096;
  using T = typename Elem<DT>::T;
  __shared__ __attribute__((aligned(16))) uint32_t xs[MR * K / 2];  // x_hat, 16-bit
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // rows: the workgroups split n as evenly as possible (qw or qw + 1 each),
  // then each workgroup's waves split its rows (a compute unit's stream is
  // what one workgroup reads, so the balance that matters is per workgroup)
  const int g = blockIdx.x;
  const int rb = g * qw + min(g, remw);
  const int rw = qw + (g < remw ? 1 : 0);
  const int r0 = rb + (rw * wave) / kStreamWaves;
  const int cnt = rb + (rw * (wave + 1)) / kStreamWaves - r0;  // at most kStreamRows

  // 1. the global scales, by scalar loads (they take no slot of the compute
  //    unit's vector-load queue, which the weight stream needs from the
  //    start), and x: quarter group tid, elements 4 tid .. 4 tid + 3
  const float gxs = gx ? *gx : kE4M3Max * kE2M1Max;
  const float gws = gw ? *gw : kE4M3Max * kE2M1Max;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint64_t)m * K * sizeof(T));
  u32x2 xr[MR];
#pragma unroll
  for (int j = 0; j < MR; ++j)
    xr[j] = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rx, (uint32_t)(j * K / 4 + tid) * 8u, 0, 0));
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");  // the workgroup's x and scale loads go first
  __builtin_amdgcn_sched_barrier(0);

  // 2. this wave's rows: a buffer range over exactly them, so that loads of
  //    rows past cnt read zeros and every load can be issued unconditionally
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(wc + (int64_t)r0 * (K / 2), (uint64_t)cnt * (K / 2));
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(ws + (int64_t)r0 * (K / 16), (uint64_t)cnt * (K / 16));
  StreamRow wr[kStreamRows];
  auto issue = [&](int i) {
    const uint32_t co = (uint32_t)(i * (K / 2)) + 16u * lane;
    wr[i].code[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 2));
    wr[i].code[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, co + 1024u, 0, 2));
    wr[i].scale = __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(i * (K / 16)) + 4u * lane, 0, 2);
  };
  issue(0);
  __builtin_amdgcn_sched_barrier(0);

  // 3. the factors 2688/g_x, g_x/2688, g_w/2688: one division, three lanes
  float enc, dec, dec_w;
  {
    const float num = lane == 0 ? kE4M3Max * kE2M1Max : (lane == 1 ? gxs : gws);
    const float den = lane == 0 ? gxs : kE4M3Max * kE2M1Max;
    float qv;
    {
#pragma clang fp contract(off)
      qv = num / den;
    }
    enc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qv), 0));
    dec = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qv), 1));
    dec_w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qv), 2));
  }

  // 4. x_hat of this quarter group of each row (lanes 4j .. 4j + 3 hold one
  //    group of 16), or x as given
#pragma unroll
  for (int j = 0; j < MR; ++j) {
    if constexpr (!QX) {
      reinterpret_cast<u32x2*>(xs)[j * K / 4 + tid] = xr[j];
      continue;
    }
    float v[8];
    unpack8<DT>(u32x4{xr[j].x, xr[j].y, 0u, 0u}, v);
    float a = fmaxf(fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                    fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])));
    a = fmaxf(a, dpp_mov<0xB1>(a));  // quad_perm [1,0,3,2]
    a = fmaxf(a, dpp_mov<0x4E>(a));  // quad_perm [2,3,0,1]
    const GroupScale gs = group_scale_from_amax(a, enc);
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma clang fp contract(off)
      y[i] = v[i] * gs.enc_b;
    }
    uint32_t cw = 0;
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, y[0], y[1], 1.0f, 0);
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, y[2], y[3], 1.0f, 1);
    float sc;
    {
#pragma clang fp contract(off)
      sc = e4m3_decode(gs.byte) * dec;
    }
    const f32x2 d0 = e2m1_decode2_f32<0>(cw), d1 = e2m1_decode2_f32<1>(cw);
    float o[4];
    {
#pragma clang fp contract(off)
      o[0] = d0.x * sc; o[1] = d0.y * sc; o[2] = d1.x * sc; o[3] = d1.y * sc;
    }
    reinterpret_cast<u32x2*>(xs)[j * K / 4 + tid] = u32x2{pack2<DT>(o[0], o[1]), pack2<DT>(o[2], o[3])};
  }
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();  // x_hat written; row 0's loads stay in flight
  __builtin_amdgcn_sched_barrier(0);

  // 5. this lane's x_hat pieces: elements 32 lane .. + 31 and 2048 + 32 lane ..
  uint32_t xp[MR][2][16];
#pragma unroll
  for (int j = 0; j < MR; ++j)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const u32x4 t = reinterpret_cast<const u32x4*>(xs)[(j * K + hh * 2048 + 32 * lane) / 8 + qd];
        xp[j][hh][4 * qd] = t.x; xp[j][hh][4 * qd + 1] = t.y;
        xp[j][hh][4 * qd + 2] = t.z; xp[j][hh][4 * qd + 3] = t.w;
      }
    }

  __builtin_amdgcn_sched_barrier(0);
  // the rest of the window, one row after the other (the wait counter retires
  // loads in order, so a row's loads must not interleave with the next's).
  // Issued only now: a wave whose loads exceed what the compute unit accepts
  // stalls at the issue, and a stall ahead of the barrier above would hold
  // every wave of the workgroup
#pragma unroll
  for (int i = 1; i < kStreamAhead; ++i) {
    issue(i);
    __builtin_amdgcn_sched_barrier(0);
  }

  // 6. rows: once row i is in (its scale dword, the row's last load, is
  //    read), issue row i + kStreamAhead, then compute row i
  const int sshift = 8 * ((2 * lane) & 3);
  float mine[MR];
#pragma unroll
  for (int j = 0; j < MR; ++j) mine[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < kStreamRows; ++i) {
    // the two scale bytes of piece hh sit in lane 32 hh + lane / 2
    uint32_t swv[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      swv[hh] = (uint32_t)__builtin_amdgcn_ds_bpermute((32 * hh + (lane >> 1)) * 4, (int)wr[i].scale);
    __builtin_amdgcn_sched_barrier(0);
    if (i + kStreamAhead < kStreamRows) issue(i + kStreamAhead);
    __builtin_amdgcn_sched_barrier(0);
    float acc[MR];
#pragma unroll
    for (int j = 0; j < MR; ++j) acc[j] = 0.0f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t sw = swv[hh];
      float se0, se1;
      {
#pragma clang fp contract(off)
        const uint32_t sb = sw >> sshift;
        se0 = e4m3_decode_byte<0>(sb) * dec_w;
        se1 = e4m3_decode_byte<1>(sb) * dec_w;
      }
      const u32x4 c = wr[i].code[hh];
      float p0[MR], p1[MR];
      group_dot16_rows<DT, MR>(c.x, c.y, xp, hh, 0, p0);
      group_dot16_rows<DT, MR>(c.z, c.w, xp, hh, 8, p1);
#pragma unroll
      for (int j = 0; j < MR; ++j) {
        acc[j] = __builtin_fmaf(p0[j], se0, acc[j]);
        acc[j] = __builtin_fmaf(p1[j], se1, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < MR; ++j) {
      const float v = wave_sum_uniform(acc[j]);
      mine[j] = (lane == i) ? v : mine[j];
    }
  }
  if (lane < cnt) {
#pragma unroll
    for (int j = 0; j < MR; ++j)
      if (j < m) reinterpret_cast<T*>(out)[(int64_t)j * n + r0 + lane] = from_f32<DT>(mine[j]);
  }
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

template <int DT, int CH, int R>
void launch_reg(const void* x, const float* gx, const uint8_t* wc, const uint8_t* ws,
                const float* gw, int64_t n, void* out, int64_t blocks, hipStream_t s) {
  qmv_reg_kernel<DT, CH, R><<<(int)blocks, kThreadsQ, 0, s>>>(x, gx, wc, ws, gw, (int)n, out);
}

// rows per wave r <= kMaxRows: the launcher takes at least ceil(n / (8 kMaxRows)) workgroups
template <int DT, int CH>
void launch_reg_r(int r, const void* x, const float* gx, const uint8_t* wc, const uint8_t* ws,
                  const float* gw, int64_t n, void* out, int64_t blocks, hipStream_t s) {
  static_assert(kMaxRows == 2, "rows per wave");
  if (r <= 1)
    launch_reg<DT, CH, 1>(x, gx, wc, ws, gw, n, out, blocks, s);
  else
    launch_reg<DT, CH, 2>(x, gx, wc, ws, gw, n, out, blocks, s);
}

// the streaming kernel (16-bit x, k = 4096, n < 2^31) with MR rows of x:
// one 16-wave workgroup per compute unit, more when a wave would get more
// than kStreamRows rows
template <int DT, int MR>
hipError_t launch_stream(const void* x, int m, bool qx, const float* gx, const uint8_t* wc,
                         const uint8_t* ws, const float* gw, int64_t n, void* out, hipStream_t s) {
  const int64_t per_wg = (int64_t)kStreamWaves * kStreamRows;
  int64_t blocks = (n + kStreamWaves - 1) / kStreamWaves;
  if (blocks > device_cu_count()) blocks = device_cu_count();
  if (blocks < (n + per_wg - 1) / per_wg) blocks = (n + per_wg - 1) / per_wg;
  if (qx)
    qmv_stream_kernel<DT, MR, true><<<(int)blocks, kStreamThreads, 0, s>>>(
        x, m, gx, wc, ws, gw, (int)n, (int)(n / blocks), (int)(n % blocks), out);
  else
    qmv_stream_kernel<DT, MR, false><<<(int)blocks, kStreamThreads, 0, s>>>(
        x, m, gx, wc, ws, gw, (int)n, (int)(n / blocks), (int)(n % blocks), out);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_qmv_t(const void* x, const float* gx, const uint8_t* wc, const uint8_t* ws,
                        const float* gw, int64_t n, int64_t k, void* out, hipStream_t s) {
  const int chunks = (k % 4096 == 0) ? (int)(k / 4096) : 0;
  if constexpr (DT != kF32) {
    if (chunks == 1 && n < 0x7FFFFFFF) return launch_stream<DT, 1>(x, 1, true, gx, wc, ws, gw, n, out, s);
  }
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
  return (dt == kBF16 || dt == kF16) && m >= 1 && m <= 2 && k == 4096 && n >= 1 && n < 0x7FFFFFFF;
}

hipError_t launch_qmv_rows(const void* x, int dt, int64_t m, bool quantize_x, const float* gx,
                           const uint8_t* wc, const uint8_t* ws, const float* gw, int64_t n,
                           void* out, hipStream_t s) {
  if (m == 1)
    return dt == kF16 ? launch_stream<kF16, 1>(x, 1, quantize_x, gx, wc, ws, gw, n, out, s)
                      : launch_stream<kBF16, 1>(x, 1, quantize_x, gx, wc, ws, gw, n, out, s);
  return dt == kF16 ? launch_stream<kF16, 2>(x, (int)m, quantize_x, gx, wc, ws, gw, n, out, s)
                    : launch_stream<kBF16, 2>(x, (int)m, quantize_x, gx, wc, ws, gw, n, out, s);
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
