// smallm.hip -- NVFP4 contractions with a handful of activation rows
// (1 <= m <= 16) for gfx950:
//   qqmm  out[m, n] = T( sum_k x_hat[m, k] * w[n, k] ),  x_hat the NVFP4 round
//         trip of x under g_x ("mlx 0.30.7.2 -> 0.30.7.6" diff page 8, qqmm);
//   qmm   out[m, n] = T( sum_k x[m, k] * w[n, k] ),  x used as given (the
//         quantized_matmul of the same pages);
// with w decoded with g_w on every block scale ("[Metal] global scale for
// qmm" PR 4458, statement: the global factor sits inside the dequantization).
//
// With at most 16 rows the contraction is as HBM-bound as qmv: the weight
// (9/16 byte per element) is read once and each element feeds at most 16
// products.  The 256-row-tile matrix-core kernels would leave most of the chip
// idle (56 tiles for n = 14336) and pay the MFMA work of a whole tile, so these
// kernels stream the weight like qmv and use the matrix cores only to absorb
// the m dimension:
//   * one workgroup per CU (fewer when there is little work); it builds x_hat
//     (or copies x) for all m rows into LDS once -- its x loads go out first,
//     then its first weight loads, so that waiting for x leaves those in
//     flight -- then covers a slice of the weight rows;
//   * its 8 waves split the slice into row tiles and each tile's k range into
//     parts; every load is issued unconditionally (pieces past a wave's range
//     read zeros from beyond the buffer's end), two batches of 4 k-chunks in
//     flight, so the compiler counts the loads outstanding and each wave
//     waits for one batch at a time, overlapping the decode with the stream;
//   * the codes are decoded to T with the effective block scale
//     e4m3(s) * g_w/2688 (float32 product, rounded to T, as in the large
//     matrix-core kernels) and multiplied on the matrix cores with the weight
//     tile as the first operand and the x rows (padded by repeating the last
//     row, whose products are never stored) as the second;
//   * the k parts of a tile are summed through LDS in a fixed order.
// Packed weight with k = 2048 / 4096 and m <= 16 (smallm_px_kernel): the codes
// decoded exactly, one block of 16 per matrix-core product, each block's
// partial sums scaled in float32 (described at the kernel).  Row-major weight
// with k = 4096 and m <= 2: qmv's register kernel with one accumulator per row
// (qmv.hip).  Otherwise:
// Row-major weight: v_mfma_f32_16x16x32 over strips of 16 rows; per 128-wide
// k chunk a lane loads 16 code bytes of its row (four lanes cover 64
// contiguous bytes) and two scale bytes.  Packed weight (mfma_pack_kernel):
// v_mfma_f32_32x32x16 over its 32-row tiles; per 64-wide k step a wave loads
// the step's whole 1 KB code block (lane l: row l % 32, codes 32 (l / 32) ..
// + 31) and the row's scale dword -- contiguous loads, which the row-major
// layout cannot give a 16-row operand.
#include <algorithm>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kSmWaves = 8;
constexpr int kSmThreads = 64 * kSmWaves;
constexpr int kSmChunk = 128;   // row-major: k per chunk (4 lane quarters x 32 codes)
constexpr int kPkStep = 64;     // packed: k per block
constexpr int kSmBatch = 4;     // chunks / blocks per batch of loads
constexpr int kSmXRounds = 16;  // x half groups per thread: m k / 8 / 512 <= 16
constexpr uint32_t kSmOutside = 0x7FF00000u;  // an offset past the end of every buffer

template <int DT> struct SmMfma;
template <> struct SmMfma<kBF16> {
  using V8 = bf16x8;
  static __device__ __forceinline__ f32x4 run16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 run32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct SmMfma<kF16> {
  using V8 = f16x8;
  static __device__ __forceinline__ f32x4 run16(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 run32(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// One k piece of one lane: 32 codes of a weight row and their scales (the
// two bytes of its two groups, or the row's scale dword of the packed step).
struct SmPiece {
  u32x4 code;
  uint32_t scale;
};

// 8 codes of one dword, times the effective block scale, as 8 16-bit values.
template <int DT>
__device__ __forceinline__ typename SmMfma<DT>::V8 decode_word(uint32_t w, float se) {
  u32x4 v;
  v.x = decode_dword<DT, 0>(w, se);
  v.y = decode_dword<DT, 1>(w, se);
  v.z = decode_dword<DT, 2>(w, se);
  v.w = decode_dword<DT, 3>(w, se);
  return __builtin_bit_cast(typename SmMfma<DT>::V8, v);
}

// ---------------------------------------------------------------- x rows in LDS
//
// x rows [M][ldr] of T in LDS (ldr = K + 8: 16 bytes of padding per row put
// the fragment reads of different rows in different banks).  Half group h =
// elements 8 h .. 8 h + 7 of x (row h / (K / 8)); thread t of NT takes
// h = t + NT r.

template <int NT>
__device__ __forceinline__ void issue_x_loads(const void* x, int H, int tid,
                                              u32x4 (&xr)[kSmXRounds]) {
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(x, (uint64_t)H * 16);
#pragma unroll
  for (int r = 0; r < kSmXRounds; ++r)  // past the end of x: zeros
    xr[r] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_x, (uint32_t)(tid + NT * r) * 16u, 0, 0));
}

template <int DT, bool QX, int NT>
__device__ __forceinline__ void write_x_rows(const u32x4 (&xr)[kSmXRounds], const float* gx, int M,
                                             int K, int ldr, int tid, typename Elem<DT>::T* xs) {
  using T = typename Elem<DT>::T;
  const int hpr = K / 8;  // half groups per row
  const int H = M * hpr;  // even: pair partners (h, h ^ 1) share a round
  const int rounds = (H + NT - 1) / NT;
  const float enc = global_encode(gx);
  const float dec = global_decode(gx);
#pragma unroll
  for (int r = 0; r < kSmXRounds; ++r) {
    if (r < rounds) {
      const int h = tid + NT * r;
      T* dst = xs + (h / hpr) * ldr + 8 * (h % hpr);
      if constexpr (QX) {
        float v[8], o[8];
        unpack8<DT>(xr[r], v);
        xhat_half_group<DT>(v, enc, dec, o);  // both partners of a pair take part
        if (h < H) {
          typedef T T8 __attribute__((ext_vector_type(8)));
          T8 t8;
#pragma unroll
          for (int i = 0; i < 8; ++i) t8[i] = from_f32<DT>(o[i]);
          *reinterpret_cast<T8*>(dst) = t8;
        }
      } else {
        if (h < H) *reinterpret_cast<u32x4*>(dst) = xr[r];
      }
    }
  }
}

// ---------------------------------------------------------------- row-major weight

// Row tile = strip of 16 rows; lane (fr = l % 16, q = l / 16) takes row fr
// and, in chunk c, codes k = 128 c + 32 q .. + 31; MFMA t of the chunk takes
// from lane quarter q the k values 32 q + 8 t .. + 7, for both operands.
template <int DT, bool QX>
__global__ void __launch_bounds__(kSmThreads)
smallm_rm_kernel(const void* __restrict__ x, const float* __restrict__ gx,
                 const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                 const float* __restrict__ gw, int M, int N, int K, int RW, bool vec_store,
                 void* __restrict__ out) {
  using T = typename Elem<DT>::T;
  using V8 = typename SmMfma<DT>::V8;
  extern __shared__ __attribute__((aligned(16))) uint8_t sm_lds[];
  const int ldr = K + 8;
  T* const xs = reinterpret_cast<T*>(sm_lds);
  f32x4* const red = reinterpret_cast<f32x4*>(sm_lds + (size_t)M * ldr * sizeof(T));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar chunk range
  const int fr = lane & 15;
  const int q = lane >> 4;

  const int SP = RW <= 16 ? 1 : (RW <= 32 ? 2 : 4);  // strips per pass
  const int KS = kSmWaves / SP;                       // k parts per strip
  const int strip = wave % SP, kpart = wave / SP;
  const int C = K / kSmChunk;
  const int c0 = kpart * C / KS, c1 = (kpart + 1) * C / KS;
  const int xm = min(fr, M - 1);

  const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(wc, (uint64_t)N * (K / 2));
  const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(ws, (uint64_t)N * (K / 16));
  // this lane's row at chunk 0 (outside the slice: past the buffers' ends)
  auto offsets_of = [&](int64_t r0, uint32_t& oc, uint32_t& os) {
    const int64_t n = r0 + 16 * strip + fr;
    const bool inside = n < min<int64_t>(r0 + RW, N);
    oc = inside ? (uint32_t)n * (uint32_t)(K / 2) + 16u * q : kSmOutside;
    os = inside ? (uint32_t)n * (uint32_t)(K / 16) + 2u * q : kSmOutside;
  };

  SmPiece bufA[kSmBatch], bufB[kSmBatch];
  auto load_batch = [&](SmPiece (&buf)[kSmBatch], uint32_t oc, uint32_t os, int cb) {
#pragma unroll
    for (int i = 0; i < kSmBatch; ++i) {
      const bool in = cb + i < c1;
      const int c = in ? cb + i : 0;
      buf[i].code = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs_c, in ? oc : kSmOutside, c * (kSmChunk / 2), 0));
      buf[i].scale = __builtin_amdgcn_raw_buffer_load_b16(rs_s, in ? os : kSmOutside,
                                                          c * (kSmChunk / 16), 0);
    }
  };
  const float dec_w = global_decode(gw);
  auto compute_batch = [&](const SmPiece (&buf)[kSmBatch], int cb, f32x4& acc) {
#pragma unroll
    for (int i = 0; i < kSmBatch; ++i) {
      if (cb + i < c1) {
        const int c = cb + i;
        float se0, se1;
        {
#pragma clang fp contract(off)
          se0 = e4m3_decode_byte<0>(buf[i].scale) * dec_w;
          se1 = e4m3_decode_byte<1>(buf[i].scale) * dec_w;
        }
        const uint32_t cw[4] = {buf[i].code.x, buf[i].code.y, buf[i].code.z, buf[i].code.w};
        const T* xrow = xs + xm * ldr + kSmChunk * c + 32 * q;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const V8 xv = *reinterpret_cast<const V8*>(xrow + 8 * t);
          acc = SmMfma<DT>::run16(decode_word<DT>(cw[t], t < 2 ? se0 : se1), xv, acc);
        }
      }
    }
  };

  u32x4 xr[kSmXRounds];
  issue_x_loads<kSmThreads>(x, M * (K / 8), tid, xr);
  __builtin_amdgcn_sched_barrier(0);  // x loads ahead of the weight loads
  const int64_t pass_rows = (int64_t)gridDim.x * RW;
  int64_t r0 = (int64_t)blockIdx.x * RW;
  uint32_t oc, os;
  offsets_of(r0, oc, os);
  load_batch(bufA, oc, os, c0);
  load_batch(bufB, oc, os, c0 + kSmBatch);
  __builtin_amdgcn_sched_barrier(0);
  write_x_rows<DT, QX, kSmThreads>(xr, gx, M, K, ldr, tid, xs);
  lds_barrier();  // x rows written; the weight loads stay in flight

  for (; r0 < N; r0 += pass_rows) {
    const int rend = (int)min<int64_t>(r0 + RW, N);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int cb = c0; cb < c1; cb += 2 * kSmBatch) {
      compute_batch(bufA, cb, acc);
      load_batch(bufA, oc, os, cb + 2 * kSmBatch);
      compute_batch(bufB, cb + kSmBatch, acc);
      load_batch(bufB, oc, os, cb + 3 * kSmBatch);
    }
    // the next pass's first loads (zeros after the last pass)
    offsets_of(r0 + pass_rows, oc, os);
    load_batch(bufA, oc, os, c0);
    load_batch(bufB, oc, os, c0 + kSmBatch);

    // k parts of the strip: parts 1.. through LDS, summed by part 0 in order
    if (kpart > 0) red[(kpart - 1) * SP * 64 + strip * 64 + lane] = acc;
    lds_barrier();
    if (kpart == 0) {
      for (int p = 1; p < KS; ++p) acc += red[(p - 1) * SP * 64 + strip * 64 + lane];
      // lane holds out[fr][n .. n + 3], n = r0 + 16 strip + 4 q
      const int n = (int)r0 + 16 * strip + 4 * q;
      if (fr < M && n < rend) {
        T* o = reinterpret_cast<T*>(out) + (int64_t)fr * N + n;
        if (vec_store && n + 3 < rend) {
          typedef T T4 __attribute__((ext_vector_type(4)));
          T4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = from_f32<DT>(acc[i]);
          *reinterpret_cast<T4*>(o) = v;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (n + i < rend) o[i] = from_f32<DT>(acc[i]);
        }
      }
    }
    lds_barrier();  // red is reused by the next pass
  }
}

// ---------------------------------------------------------------- packed weight

// Row tile = a 32-row tile T of the packed layout; in its block (T, s) lane l
// holds row l % 32, codes k = 64 s + 32 h .. + 31 (h = l / 32), and MFMA u
// (u < 4) of the block takes from lane half h the k values 32 h + 8 u .. + 7
// (the order of the large kernels), for both operands.  The output lane l
// holds D[8 (v / 4) + 4 h + v % 4][l % 32] (v < 16): tile rows 8 (v / 4) + 4 h
// .. + 3 of x row l % 32.
template <int DT, bool QX>
__global__ void __launch_bounds__(kSmThreads)
smallm_pk_kernel(const void* __restrict__ x, const float* __restrict__ gx,
                 const uint8_t* __restrict__ pc, const uint8_t* __restrict__ ps,
                 const float* __restrict__ gw, int M, int N, int K, int TPW, bool vec_store,
                 void* __restrict__ out) {
  using T = typename Elem<DT>::T;
  using V8 = typename SmMfma<DT>::V8;
  extern __shared__ __attribute__((aligned(16))) uint8_t sm_lds[];
  const int ldr = K + 8;
  T* const xs = reinterpret_cast<T*>(sm_lds);
  f32x16* const red = reinterpret_cast<f32x16*>(sm_lds + (size_t)M * ldr * sizeof(T));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int xm = min(lane & 31, M - 1);

  const int KS = kSmWaves / TPW;  // k parts per tile
  const int slot = wave % TPW, kpart = wave / TPW;
  const int KT = K / kPkStep;
  const int s0 = kpart * KT / KS, s1 = (kpart + 1) * KT / KS;
  const int tiles = (N + 31) / 32;

  const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(pc, (uint64_t)tiles * KT * kPackCodeBytes);
  const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(ps, (uint64_t)tiles * KT * kPackScaleBytes);
  auto offsets_of = [&](int tile, uint32_t& oc, uint32_t& os) {
    const bool inside = tile < tiles;
    const uint32_t blk = (uint32_t)tile * (uint32_t)KT;
    oc = inside ? blk * (uint32_t)kPackCodeBytes + 16u * lane : kSmOutside;
    os = inside ? blk * (uint32_t)kPackScaleBytes + 4u * (lane & 31) : kSmOutside;
  };

  SmPiece bufA[kSmBatch], bufB[kSmBatch];
  auto load_batch = [&](SmPiece (&buf)[kSmBatch], uint32_t oc, uint32_t os, int sb) {
#pragma unroll
    for (int i = 0; i < kSmBatch; ++i) {
      const bool in = sb + i < s1;
      const int st = in ? sb + i : 0;
      buf[i].code = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rs_c, in ? oc : kSmOutside, st * kPackCodeBytes, 0));
      buf[i].scale = __builtin_amdgcn_raw_buffer_load_b32(rs_s, in ? os : kSmOutside,
                                                          st * kPackScaleBytes, 0);
    }
  };
  const float dec_w = global_decode(gw);
  auto compute_batch = [&](const SmPiece (&buf)[kSmBatch], int sb, f32x16& acc) {
#pragma unroll
    for (int i = 0; i < kSmBatch; ++i) {
      if (sb + i < s1) {
        const int st = sb + i;
        // this lane's groups 4 s + 2 h, + 1: scale bytes 2 h, 2 h + 1
        const uint32_t sw = buf[i].scale >> (16 * h);
        float se0, se1;
        {
#pragma clang fp contract(off)
          se0 = e4m3_decode_byte<0>(sw) * dec_w;
          se1 = e4m3_decode_byte<1>(sw) * dec_w;
        }
        const uint32_t cw[4] = {buf[i].code.x, buf[i].code.y, buf[i].code.z, buf[i].code.w};
        const T* xrow = xs + xm * ldr + kPkStep * st + 32 * h;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const V8 xv = *reinterpret_cast<const V8*>(xrow + 8 * u);
          acc = SmMfma<DT>::run32(decode_word<DT>(cw[u], u < 2 ? se0 : se1), xv, acc);
        }
      }
    }
  };

  u32x4 xr[kSmXRounds];
  issue_x_loads<kSmThreads>(x, M * (K / 8), tid, xr);
  __builtin_amdgcn_sched_barrier(0);
  const int pass_tiles = gridDim.x * TPW;
  int t0 = blockIdx.x * TPW;
  uint32_t oc, os;
  offsets_of(t0 + slot, oc, os);
  load_batch(bufA, oc, os, s0);
  load_batch(bufB, oc, os, s0 + kSmBatch);
  __builtin_amdgcn_sched_barrier(0);
  write_x_rows<DT, QX, kSmThreads>(xr, gx, M, K, ldr, tid, xs);
  lds_barrier();

  for (; t0 < tiles; t0 += pass_tiles) {
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    for (int sb = s0; sb < s1; sb += 2 * kSmBatch) {
      compute_batch(bufA, sb, acc);
      load_batch(bufA, oc, os, sb + 2 * kSmBatch);
      compute_batch(bufB, sb + kSmBatch, acc);
      load_batch(bufB, oc, os, sb + 3 * kSmBatch);
    }
    const int tile = t0 + slot;
    offsets_of(t0 + pass_tiles + slot, oc, os);
    load_batch(bufA, oc, os, s0);
    load_batch(bufB, oc, os, s0 + kSmBatch);

    if (kpart > 0) red[(kpart - 1) * TPW * 64 + slot * 64 + lane] = acc;
    lds_barrier();
    if (kpart == 0 && tile < tiles) {
      for (int p = 1; p < KS; ++p) acc += red[(p - 1) * TPW * 64 + slot * 64 + lane];
      const int m = lane & 31;
      if (m < M) {
        T* orow = reinterpret_cast<T*>(out) + (int64_t)m * N;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = 32 * tile + 8 * g + 4 * h;  // rows n .. n + 3 from acc[4 g .. 4 g + 3]
          if (vec_store && n + 3 < N) {
            typedef T T4 __attribute__((ext_vector_type(4)));
            T4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = from_f32<DT>(acc[4 * g + i]);
            *reinterpret_cast<T4*>(orow + n) = v;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < N) orow[n + i] = from_f32<DT>(acc[4 * g + i]);
          }
        }
      }
    }
    lds_barrier();
  }
}

// ---------------------------------------------------------------- packed weight, exact decode
//
// Up to kPxMaxM rows of x against the packed weight (K = 2048 or 4096), one
// or two 32-row tiles per workgroup, 4 waves per tile, each wave a quarter of
// the tile's k steps (K = 256 SW), all of its weight loads issued before
// anything else.  The codes are decoded exactly
// (e2m1 to T, one conversion per two codes), each 16-wide block is contracted
// on the matrix cores on its own, and its partial sums are scaled by
// e4m3(s) * g_w/2688 in float32, as qmv does per group -- no rounding of the
// decoded weight.
//
// One v_mfma_f32_32x32x16 contracts two blocks at once, block-diagonally.  The
// second operand is the weight: lane (n = l % 32, h = l / 32) holds dword j of
// its codes, codes 32 h + 8 j .. + 7 of the step (block 2 h + j / 2).  The
// first operand is x: in lane half h its row i carries x row i - 16 h, and
// zeros (an all-zero LDS row) outside 0 <= i - 16 h < M.  So output rows
// i < 16 see only the block of lane half 0 and rows i >= 16 only that of lane
// half 1: with dwords 0, 1 the MFMA pair gives block 0 in rows i and block 2 in
// rows 16 + i, with dwords 2, 3 blocks 1 and 3.  Output lane l holds rows
// 8 (v / 4) + 4 h + v % 4 of column n, so x row m = 8 (v / 4) + 4 h + v % 4
// (v < MV: 4 accumulators cover m < 8, 8 cover m < 16) sits in elements v
// (blocks 0 / 1) and 8 + v (blocks 2 / 3) of one lane.

constexpr int kPxWaves = 4;  // waves per tile: its k quarters
constexpr int kPxMaxM = 16;

template <int DT, bool QX, int SW, int TPW, int MV>
__global__ void __launch_bounds__(64 * kPxWaves * TPW)
smallm_px_kernel(const void* __restrict__ x, const float* __restrict__ gx,
                 const uint8_t* __restrict__ pc, const uint8_t* __restrict__ ps,
                 const float* __restrict__ gw, int M, int N, void* __restrict__ out) {
  using T = typename Elem<DT>::T;
  using V8 = typename SmMfma<DT>::V8;
  constexpr int K = kPkStep * kPxWaves * SW;
  constexpr int KT = K / kPkStep;
  constexpr int ldr = K + 16;  // 32 bytes of padding per row
  constexpr int NT = 64 * kPxWaves * TPW;
  extern __shared__ __attribute__((aligned(16))) uint8_t sm_lds[];
  T* const xs = reinterpret_cast<T*>(sm_lds);  // M rows of x_hat, then a zero row
  f32x4* const red = reinterpret_cast<f32x4*>(sm_lds + (size_t)(M + 1) * ldr * sizeof(T));
  constexpr int NV4 = MV / 4;  // f32x4 per lane in the k-quarter reduction

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int li = lane & 31;
  const int tiles = (N + 31) / 32;
  const int tile = TPW * blockIdx.x + wave / kPxWaves;
  const int quarter = wave % kPxWaves;

  // 1. x first, then every weight load of this wave's SW steps (a tile past
  //    the last one reads zeros and stores nothing)
  u32x4 xr[kSmXRounds];
  issue_x_loads<NT>(x, M * (K / 8), tid, xr);
  __builtin_amdgcn_sched_barrier(0);
  const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(pc, (uint64_t)tiles * KT * kPackCodeBytes);
  const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(ps, (uint64_t)tiles * KT * kPackScaleBytes);
  const uint32_t blk0 = (uint32_t)tile * (uint32_t)KT + (uint32_t)(quarter * SW);
  SmPiece wp[SW];
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    wp[s].code = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rs_c, (blk0 + s) * (uint32_t)kPackCodeBytes + 16u * lane, 0, 0));
    wp[s].scale = __builtin_amdgcn_raw_buffer_load_b32(
        rs_s, (blk0 + s) * (uint32_t)kPackScaleBytes + 4u * li, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. x_hat rows and the zero row into LDS; the weight loads stay in flight
  write_x_rows<DT, QX, NT>(xr, gx, M, K, ldr, tid, xs);
  for (int e = tid; e < ldr / 8; e += NT)
    reinterpret_cast<u32x4*>(xs + (size_t)M * ldr)[e] = u32x4{0u, 0u, 0u, 0u};
  lds_barrier();

  // 3. the steps
  const float dec_w = global_decode(gw);
  const int xi = li - 16 * h;  // x row of this lane's first-operand slots
  const T* const xrow = xs + (size_t)((xi >= 0 && xi < M) ? xi : M) * ldr + 32 * h;
  const f32x16 zero = {};
  float acc[MV];
#pragma unroll
  for (int v = 0; v < MV; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int s = 0; s < SW; ++s) {
    const T* xp = xrow + kPkStep * (quarter * SW + s);
    const uint32_t cw[4] = {wp[s].code.x, wp[s].code.y, wp[s].code.z, wp[s].code.w};
    V8 xa[4], wb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xa[j] = *reinterpret_cast<const V8*>(xp + 8 * j);
      u32x4 d;
      if constexpr (DT == kBF16) {
        d.x = __builtin_bit_cast(uint32_t, e2m1_decode2_bf16<0>(cw[j]));
        d.y = __builtin_bit_cast(uint32_t, e2m1_decode2_bf16<1>(cw[j]));
        d.z = __builtin_bit_cast(uint32_t, e2m1_decode2_bf16<2>(cw[j]));
        d.w = __builtin_bit_cast(uint32_t, e2m1_decode2_bf16<3>(cw[j]));
      } else {
        d.x = __builtin_bit_cast(uint32_t, e2m1_decode2_f16<0>(cw[j]));
        d.y = __builtin_bit_cast(uint32_t, e2m1_decode2_f16<1>(cw[j]));
        d.z = __builtin_bit_cast(uint32_t, e2m1_decode2_f16<2>(cw[j]));
        d.w = __builtin_bit_cast(uint32_t, e2m1_decode2_f16<3>(cw[j]));
      }
      wb[j] = __builtin_bit_cast(V8, d);
    }
    f32x16 pa = SmMfma<DT>::run32(xa[0], wb[0], zero);
    pa = SmMfma<DT>::run32(xa[1], wb[1], pa);  // rows < 16: block 0, rows >= 16: block 2
    f32x16 pb = SmMfma<DT>::run32(xa[2], wb[2], zero);
    pb = SmMfma<DT>::run32(xa[3], wb[3], pb);  // blocks 1 and 3
    float se[4];
    {
#pragma clang fp contract(off)
      se[0] = e4m3_decode_byte<0>(wp[s].scale) * dec_w;
      se[1] = e4m3_decode_byte<1>(wp[s].scale) * dec_w;
      se[2] = e4m3_decode_byte<2>(wp[s].scale) * dec_w;
      se[3] = e4m3_decode_byte<3>(wp[s].scale) * dec_w;
    }
#pragma unroll
    for (int v = 0; v < MV; ++v) {
      acc[v] = __builtin_fmaf(pa[v], se[0], acc[v]);
      acc[v] = __builtin_fmaf(pb[v], se[1], acc[v]);
      acc[v] = __builtin_fmaf(pa[8 + v], se[2], acc[v]);
      acc[v] = __builtin_fmaf(pb[8 + v], se[3], acc[v]);
    }
  }

  // 4. the four k quarters of a tile summed in order; lane (n, h) holds x
  //    rows 8 (v / 4) + 4 h + v % 4
  const int slot = (wave / kPxWaves) * (kPxWaves - 1);
  if (quarter > 0) {
#pragma unroll
    for (int c = 0; c < NV4; ++c)
      red[((slot + quarter - 1) * NV4 + c) * 64 + lane] =
          f32x4{acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
  }
  lds_barrier();
  if (quarter == 0) {
#pragma unroll
    for (int p = 0; p < kPxWaves - 1; ++p) {
#pragma unroll
      for (int c = 0; c < NV4; ++c) {
        const f32x4 r = red[((slot + p) * NV4 + c) * 64 + lane];
        acc[4 * c] += r.x; acc[4 * c + 1] += r.y; acc[4 * c + 2] += r.z; acc[4 * c + 3] += r.w;
      }
    }
    const int n = 32 * tile + li;
    if (n < N) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        const int m = 8 * (v / 4) + 4 * h + v % 4;
        if (m < M) reinterpret_cast<T*>(out)[(int64_t)m * N + n] = from_f32<DT>(acc[v]);
      }
    }
  }
}

// ---------------------------------------------------------------- launch

// LDS of a launch: the x rows and the k-part partial sums
size_t rm_lds(int64_t m, int64_t k) {
  return (size_t)m * (size_t)(k + 8) * 2 + (size_t)(kSmWaves - 1) * 64 * sizeof(f32x4);
}
size_t px_lds(int64_t m, int64_t k, int tpw) {
  const int64_t nv4 = m > 8 ? 2 : 1;
  return (size_t)(m + 1) * (size_t)(k + 16) * 2 + (size_t)(tpw * nv4) * (kPxWaves - 1) * 64 * sizeof(f32x4);
}
bool px_ok(int64_t m, int64_t k) {
  return m >= 1 && m <= kPxMaxM && (k == 2048 || k == 4096) && px_lds(m, k, 2) <= kSmallMaxLds;
}
size_t pk_lds(int64_t m, int64_t k) {
  return (size_t)m * (size_t)(k + 8) * 2 + (size_t)(kSmWaves - 1) * 64 * sizeof(f32x16);
}

// code bytes of the weight: row-major n k / 2, packed whole 32-row tiles
uint64_t small_code_bytes(bool packed, int64_t n, int64_t k) {
  const int64_t rows = packed ? (n + 31) / 32 * 32 : n;
  return (uint64_t)rows * (uint64_t)(k / 2);
}

template <typename F>
hipError_t allow_lds(F* kernel) {
  static bool set[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev < 0 || dev >= 64 || set[dev]) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmallMaxLds);
  if (e == hipSuccess) set[dev] = true;
  return e;
}

template <int DT, bool QX>
hipError_t launch_rm(const void* x, const float* gx, const uint8_t* wc, const uint8_t* ws,
                     const float* gw, int64_t m, int64_t n, int64_t k, void* out, hipStream_t s) {
  const int64_t cus = device_cu_count();
  int64_t rw = (n + cus - 1) / cus;
  rw = std::min<int64_t>(64, std::max<int64_t>(8, (rw + 7) / 8 * 8));
  const int64_t blocks = std::min<int64_t>((n + rw - 1) / rw, cus);
  if (hipError_t e = allow_lds(smallm_rm_kernel<DT, QX>)) return e;
  const bool vec = (n % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & 7) == 0);
  smallm_rm_kernel<DT, QX><<<(int)blocks, kSmThreads, rm_lds(m, k), s>>>(
      x, gx, wc, ws, gw, (int)m, (int)n, (int)k, (int)rw, vec, out);
  return hipGetLastError();
}

template <int DT, bool QX>
hipError_t launch_pk(const void* x, const float* gx, const uint8_t* pc, const uint8_t* ps,
                     const float* gw, int64_t m, int64_t n, int64_t k, void* out, hipStream_t s) {
  const int64_t cus = device_cu_count();
  const int64_t tiles = (n + 31) / 32;
  // tiles per workgroup and pass: 1, 2 or 4 (k split over 8, 4 or 2 waves)
  const int64_t tpw = tiles <= cus ? 1 : (tiles <= 2 * cus ? 2 : 4);
  const int64_t blocks = std::min<int64_t>((tiles + tpw - 1) / tpw, cus);
  if (hipError_t e = allow_lds(smallm_pk_kernel<DT, QX>)) return e;
  const bool vec = (n % 4 == 0) && ((reinterpret_cast<uintptr_t>(out) & 7) == 0);
  smallm_pk_kernel<DT, QX><<<(int)blocks, kSmThreads, pk_lds(m, k), s>>>(
      x, gx, pc, ps, gw, (int)m, (int)n, (int)k, (int)tpw, vec, out);
  return hipGetLastError();
}

template <int DT, bool QX, int SW, int TPW, int MV>
hipError_t launch_px_t(const void* x, const float* gx, const uint8_t* pc, const uint8_t* ps,
                       const float* gw, int64_t m, int64_t n, void* out, hipStream_t s) {
  if (hipError_t e = allow_lds(smallm_px_kernel<DT, QX, SW, TPW, MV>)) return e;
  const int64_t tiles = (n + 31) / 32;
  smallm_px_kernel<DT, QX, SW, TPW, MV><<<(int)((tiles + TPW - 1) / TPW), 64 * kPxWaves * TPW,
                                          px_lds(m, 256 * SW, TPW), s>>>(x, gx, pc, ps, gw, (int)m,
                                                                          (int)n, out);
  return hipGetLastError();
}

template <int DT, bool QX>
hipError_t launch_px(const void* x, const float* gx, const uint8_t* pc, const uint8_t* ps,
                     const float* gw, int64_t m, int64_t n, int64_t k, void* out, hipStream_t s) {
  // Every workgroup rebuilds x_hat for its own use: with the round trip in
  // the kernel and more than one row, two tiles per workgroup halve that work
  // per CU (measured faster from m = 2 on); x used as given runs fastest with
  // one tile per workgroup (more workgroups to spread over the CUs).
  // Above 8 rows x fills most of the LDS (one workgroup per CU): two tiles
  // per workgroup keep the grid within one round of the CUs.
  if (m > 8)
    return k == 2048 ? launch_px_t<DT, QX, 8, 2, 8>(x, gx, pc, ps, gw, m, n, out, s)
                     : launch_px_t<DT, QX, 16, 2, 8>(x, gx, pc, ps, gw, m, n, out, s);
  if (QX && m >= 2)
    return k == 2048 ? launch_px_t<DT, QX, 8, 2, 4>(x, gx, pc, ps, gw, m, n, out, s)
                     : launch_px_t<DT, QX, 16, 2, 4>(x, gx, pc, ps, gw, m, n, out, s);
  return k == 2048 ? launch_px_t<DT, QX, 8, 1, 4>(x, gx, pc, ps, gw, m, n, out, s)
                   : launch_px_t<DT, QX, 16, 1, 4>(x, gx, pc, ps, gw, m, n, out, s);
}

template <bool QX>
hipError_t launch_small_q(int dt, const void* x, const float* gx, const uint8_t* wc,
                          const uint8_t* ws, bool packed, const float* gw, int64_t m, int64_t n,
                          int64_t k, void* out, hipStream_t s) {
  if (packed && px_ok(m, k))
    return dt == kF16 ? launch_px<kF16, QX>(x, gx, wc, ws, gw, m, n, k, out, s)
                      : launch_px<kBF16, QX>(x, gx, wc, ws, gw, m, n, k, out, s);
  if (packed)
    return dt == kF16 ? launch_pk<kF16, QX>(x, gx, wc, ws, gw, m, n, k, out, s)
                      : launch_pk<kBF16, QX>(x, gx, wc, ws, gw, m, n, k, out, s);
  return dt == kF16 ? launch_rm<kF16, QX>(x, gx, wc, ws, gw, m, n, k, out, s)
                    : launch_rm<kBF16, QX>(x, gx, wc, ws, gw, m, n, k, out, s);
}

}  // namespace

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

bool small_m_ok(int dt, bool packed, int64_t m, int64_t n, int64_t k) {
  return (dt == kF16 || dt == kBF16) && m >= 1 && m <= kSmallMaxM && k % kSmChunk == 0 &&
         (packed ? pk_lds(m, k) : rm_lds(m, k)) <= kSmallMaxLds &&
         small_code_bytes(packed, n, k) < kSmOutside;
}

hipError_t launch_small_m(const void* x, int dt, bool quantize_x, const float* gx,
                          const uint8_t* wc, const uint8_t* ws, bool packed, const float* gw,
                          int64_t m, int64_t n, int64_t k, void* out, hipStream_t s) {
  if (!packed && qmv_rows_ok(dt, m, n, k))  // qmv's streaming design, one accumulator per row
    return launch_qmv_rows(x, dt, m, quantize_x, gx, wc, ws, gw, n, out, s);
  if (packed && quantize_x && qmv_packed_ok(dt, m, k))  // fp4 codes straight to the matrix cores
    return launch_qmv_packed(x, dt, m, gx, wc, ws, gw, n, k, out, s);
  return quantize_x ? launch_small_q<true>(dt, x, gx, wc, ws, packed, gw, m, n, k, out, s)
                    : launch_small_q<false>(dt, x, gx, wc, ws, packed, gw, m, n, k, out, s);
}

}  // namespace nvfp4
