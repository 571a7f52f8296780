// qmv_packed.hip -- qqmm with 1 to 4 rows of bfloat16 x against the packed
// weight, on the matrix cores with the weight's fp4 codes as they are stored:
//   out[m, n] = T( sum_k x_hat[m, k] * w[n, k] ),  x_hat the NVFP4 round trip
//   of x under g_x ("mlx 0.30.7.2 -> 0.30.7.6" diff page 8, qqmm; page 7,
//   QQMatmul::eval_gpu, the M == 1 case and the small batches beside it), w
//   decoded with g_w on every block scale ("[Metal] global scale for qmm" PR
//   4458, statement).
//
// The register path of qmv.hip spends about one VALU instruction per weight
// element and row of x (a conversion per two codes, a dot product per two
// elements); here the matrix cores do the products:
//   * v_mfma_scale_f32_16x16x128_f8f6f4 (both operands e2m1, unit hardware
//     scales) takes one packed 1 KB code block -- 32 rows x one 64-wide k step
//     -- per instruction and row of x: lane l = i + 16 G loads the block's
//     bytes 16 l .. + 15, which are row i + 16 (G % 2), codes 32 (G / 2) ..
//     + 31 of the step, and serve as the first operand's row i, k slice
//     32 G .. + 31;
//   * x_hat splits exactly into two e2m1 vectors per block b of 16.  With
//     sc_b = e4m3(s_b) * g_x/2688 (float32) and d an element's decoded code,
//     x_hat = T(d * sc_b) = X * T(sc_b) + Y * T(1.5 * sc_b), where X = d for
//     |d| in {0, 0.5, 1, 2, 4} (else 0) and Y = d / 1.5 for |d| in {1.5, 3, 6}
//     (else 0): a power of two passes through the rounding to T unchanged as
//     long as the results stay out of T's subnormal range.  For bfloat16
//     that holds whenever g_x >= 2688 * 2^-116 (about 3.2e-32: the smallest
//     nonzero sc_b is 2^-9 g_x/2688, and half of it must be a normal bfloat16)
//     or without a global scale (sc_b >= 2^-9); float16 x reaches its
//     subnormals with ordinary data (a block of amax below about 4e-4), so
//     float16 x takes the kernels that round every element itself;
//   * the second operand's 16 columns are j = 8 h + 4 xy + bb (row half h,
//     X or Y, block bb of the step).  Column j holds the X (xy = 0) or Y codes
//     of block bb, and zeros at the other blocks and in the k slices where
//     the first operand holds the other row half.  Output C[i][j] is then the
//     exact partial sum over block bb of w[row 16 h + i] * X (or Y);
//   * each partial is multiplied by its x coefficient T(sc_b) or T(1.5 sc_b)
//     and by the weight's block scale e4m3(s), and accumulated in float32;
//     the row sums are taken across lanes and waves in a fixed order and
//     multiplied by g_w/2688 at the end.
// Per 1 KB of codes and row of x a lane spends 16 VALU instructions (4 to
// place its 8 bytes of X or Y codes in the operand, 4 products, 4
// accumulations, and 4 scale decodes shared by the rows of x) instead of
// about 40.
//
// Work split: a workgroup (16 waves, one per CU at k = 4096) takes whole
// 32-row tiles, at most 128 blocks; its waves take contiguous runs of at most
// 8 blocks in (tile, step) order.  The workgroup first writes the X and Y
// codes of every block of x (8 bytes each) and the coefficients into LDS;
// each wave stages its blocks' scales (128 bytes per block, one 16-byte load
// per lane for all 8) in LDS.  As in the streaming qmv, the x loads go first,
// a barrier puts them ahead of the weight loads of every wave, two or four
// blocks are in flight while x_hat is built, and the rest of the run is
// issued as each block arrives.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kQpWaves = 16;
constexpr int kQpThreads = 64 * kQpWaves;
constexpr int kQpRun = 8;        // blocks per wave at most
// blocks in flight while x_hat is built: measured at n = 14336, k = 4096
// (cold weights), four ahead took m = 1 from 7.63 to 7.47 us and m = 4 from
// 11.1 to 10.7, while m = 2 went from 8.2 to 8.7 (two ahead kept there)
template <int M> constexpr int qp_ahead0() { return M == 2 ? 2 : 4; }
constexpr int kQpAhead = 4;      // blocks in flight in the loop
constexpr int kQpMinSteps = 8;   // k >= 512: a run of 8 blocks meets at most two tiles
constexpr int kQpMaxSteps = 128; // k <= 8192
constexpr int kQpMaxRows = 4;    // rows of x

// LDS for M rows of x: X / Y codes (16 bytes per block and row), coefficients
// (8 bytes per block and row), scale stage (1 KB per wave), partial row sums
// (per tile of the workgroup, row of x and wave, 32 floats; kQpWaves *
// kQpRun / steps tiles at most).
constexpr size_t qp_lds(int steps, int M) {
  return (size_t)M * steps * 4 * (16 + 8) + kQpWaves * 1024 +
         (size_t)(kQpWaves * kQpRun / steps) * kQpWaves * M * 32 * sizeof(float);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// M rows of x (m <= M are real: the rows past m read as zeros); XR half
// groups of x per thread (M k / 8192 rounded up).
template <int DT, int M, int XR>
__global__ void __launch_bounds__(kQpThreads)
qmv_packed_kernel(const void* __restrict__ x, int m, const float* __restrict__ gx,
                  const uint8_t* __restrict__ pc, const uint8_t* __restrict__ ps,
                  const float* __restrict__ gw, int n, int steps, int tq, int trem,
                  void* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int nblk = steps * 4;  // blocks of 16 per row of x
  u32x2* ctab = reinterpret_cast<u32x2*>(lds);                    // [M][nblk][X, Y]
  float* coef = reinterpret_cast<float*>(lds + M * nblk * 16);    // [M][nblk][X, Y]
  uint8_t* stage = lds + M * nblk * 24;
  float* part = reinterpret_cast<float*>(stage + kQpWaves * 1024);
  using T = typename Elem<DT>::T;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = steps * 64;
  const int t0 = blockIdx.x * tq + min((int)blockIdx.x, trem);
  const int nt = tq + ((int)blockIdx.x < trem ? 1 : 0);
  const int nbw = nt * steps;  // blocks of this workgroup, <= 128
  const int b0 = (wave * nbw) / kQpWaves;
  const int cnt = ((wave + 1) * nbw) / kQpWaves - b0;  // <= kQpRun
  const int tf = b0 / steps, st0 = b0 - tf * steps;  // the run's first tile and step

  // 1. the global scales, by scalar loads (they take no slot of the compute
  //    unit's vector-load queue, which the weight stream needs from the
  //    start), and x: half groups tid + 1024 r, elements 8 (tid + 1024 r)
  //    .. + 7 of x viewed as one vector of m k
  const float gxs = gx ? *gx : kE4M3Max * kE2M1Max;
  const float gws = gw ? *gw : kE4M3Max * kE2M1Max;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint64_t)m * K * sizeof(T));
  u32x4 xr[XR];
#pragma unroll
  for (int r = 0; r < XR; ++r)
    xr[r] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(tid + kQpThreads * r) * 16u, 0, 0));

  // this wave's partial-sum slots, one per tile of the workgroup and row of
  // x, zero where its run does not reach (its own later writes follow in order)
  for (int e = lane; e < nt * M * 8; e += 64)
    *reinterpret_cast<f32x4*>(part + ((e / (M * 8)) * kQpWaves + wave) * M * 32 + 4 * (e % (M * 8))) =
        f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");  // the workgroup's x loads go first
  __builtin_amdgcn_sched_barrier(0);

  // 2. this wave's run: buffer ranges over exactly its blocks, so that loads
  //    past cnt read zeros and every load can be issued unconditionally
  const int64_t gb0 = (int64_t)t0 * steps + b0;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(pc + gb0 * 1024, (uint64_t)cnt * 1024);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(ps + gb0 * 128, (uint64_t)cnt * 128);
  const u32x4 sv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16u * lane, 0, 2));
  u32x4 a[kQpRun];
  auto issue = [&](int i) {
    a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, (uint32_t)(i * 1024) + 16u * lane, 0, 2));
  };
  constexpr int kQpAhead0 = qp_ahead0<M>();
#pragma unroll
  for (int i = 0; i < kQpAhead0; ++i) {
    issue(i);
    __builtin_amdgcn_sched_barrier(0);
  }

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

  // 4. x's codes, split into X and Y, and the coefficients.  The two lanes
  //    of a pair hold one block (blocks never straddle rows of x), 8 codes
  //    each: each writes its half of the block's X and Y code words, and the
  //    even lane the coefficients.
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int hg = tid + kQpThreads * r;
    if (hg < M * K / 8) {  // K / 8 is even: whole pairs
      float v[8];
      unpack8<DT>(xr[r], v);
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, __builtin_fabsf(v[i]));
      am = fmaxf(am, dpp_mov<0xB1>(am));  // quad_perm [1,0,3,2]: the pair partner
      const GroupScale gs = group_scale_from_amax(am, enc);
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
        y[i] = v[i] * gs.enc_b;
      }
      uint32_t cw = 0;
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, y[0], y[1], 1.0f, 0);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, y[2], y[3], 1.0f, 1);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, y[4], y[5], 1.0f, 2);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, y[6], y[7], 1.0f, 3);
      // per nibble s.mmm: magnitudes 3, 5, 7 (1.5, 3, 6) are Y codes, Y =
      // code - 1 (bit 0 of such a nibble is set: no borrow between nibbles)
      const uint32_t m0 = cw & 0x11111111u, m1 = (cw >> 1) & 0x11111111u, m2 = (cw >> 2) & 0x11111111u;
      const uint32_t isy = m0 & (m1 | m2);
      const uint32_t ymask = isy * 0xFu;
      const int gb = hg >> 1;  // block of x as one vector: row gb / nblk, block gb % nblk
      const int half = hg & 1;
      uint32_t* ct = reinterpret_cast<uint32_t*>(ctab);
      ct[4 * gb + half] = cw & ~ymask;             // X codes, elements 8 half .. + 7
      ct[4 * gb + 2 + half] = (cw - isy) & ymask;  // Y codes
      if (half == 0) {
        float sc, sc15;
        {
#pragma clang fp contract(off)
          sc = e4m3_decode(gs.byte) * dec;
          sc15 = 1.5f * sc;
        }
        *reinterpret_cast<f32x2*>(coef + 2 * gb) =
            f32x2{to_f32<DT>(from_f32<DT>(sc)), to_f32<DT>(from_f32<DT>(sc15))};
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();  // codes and coefficients written; the block loads stay in flight
  __builtin_amdgcn_sched_barrier(0);

  // 5. the rest of the window, then this wave's scales into its stage
#pragma unroll
  for (int i = kQpAhead0; i < kQpAhead; ++i) {
    issue(i);
    __builtin_amdgcn_sched_barrier(0);
  }
  uint8_t* wstage = stage + wave * 1024;
  *reinterpret_cast<u32x4*>(wstage + 16 * lane) = sv;

  // 6. the blocks.  Lane (q = l / 16, j = l % 16) ends with C[4 q + r][j]:
  //    row 16 h + 4 q + r of the tile, block bb of the step, X or Y.  As the
  //    second operand, lane (j, G = l / 16) holds 8 code bytes of block bb
  //    in half bb % 2 when G = 2 (bb / 2) + h, zeros otherwise.
  const int j = lane & 15, q = lane >> 4;
  const int bb = j & 3, xyi = (j >> 2) & 1, h = j >> 3;
  const bool nz = q == 2 * (bb >> 1) + h;
  const uint32_t mlo = (nz && !(bb & 1)) ? 0xFFFFFFFFu : 0u;
  const uint32_t mhi = (nz && (bb & 1)) ? 0xFFFFFFFFu : 0u;
  const uint32_t sel = (uint32_t)bb | ((uint32_t)(4 + bb) << 8) | 0x0C0C0000u;
  f32x4 acc[M];
#pragma unroll
  for (int r = 0; r < M; ++r) acc[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  int seg = 0;
  auto flush = [&](int sg) {  // into the slots of tile tf + sg
    if (tf + sg >= nt) return;  // only blocks past the workgroup's last tile (zeros)
#pragma unroll
    for (int xrow = 0; xrow < M; ++xrow) {
      f32x4 v = acc[xrow];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] += dpp_mov<0xB1>(v[r]);   // quad_perm [1,0,3,2]
        v[r] += dpp_mov<0x4E>(v[r]);   // quad_perm [2,3,0,1]
        v[r] += dpp_mov<0x141>(v[r]);  // row_half_mirror: the 8 lanes of one row half
      }
      if ((j & 7) == 0)
        *reinterpret_cast<f32x4*>(part + (((tf + sg) * kQpWaves + wave) * M + xrow) * 32 + 16 * h + 4 * q) = v;
    }
  };
#pragma unroll
  for (int i = 0; i < kQpRun; ++i) {
    int st = st0 + i;
    st = st >= steps ? st - steps : st;
    if (i > 0 && st == 0) {  // the run enters the next tile
      flush(seg);
#pragma unroll
      for (int r = 0; r < M; ++r) acc[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      ++seg;
    }
    const u32x4 sw = *reinterpret_cast<const u32x4*>(wstage + 128 * i + 16 * (q + 4 * h));
    u32x2 cv8[M];
    float cf[M];
#pragma unroll
    for (int xrow = 0; xrow < M; ++xrow) {
      const int gb = xrow * nblk + 4 * st + bb;
      cv8[xrow] = ctab[2 * gb + xyi];
      cf[xrow] = coef[2 * gb + xyi];
    }
    const i32x8 av = {(int)a[i].x, (int)a[i].y, (int)a[i].z, (int)a[i].w, 0, 0, 0, 0};
    f32x4 cv[M];
#pragma unroll
    for (int xrow = 0; xrow < M; ++xrow) {
      const i32x8 bw = {(int)(cv8[xrow].x & mlo), (int)(cv8[xrow].y & mlo), (int)(cv8[xrow].x & mhi),
                        (int)(cv8[xrow].y & mhi), 0, 0, 0, 0};
      const f32x4 cz = {0.0f, 0.0f, 0.0f, 0.0f};
      cv[xrow] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bw, cz, 4, 4, 0, 127, 0, 127);
    }
    // block i is in: issue block i + kQpAhead while the products complete
    __builtin_amdgcn_sched_barrier(0);
    if (i + kQpAhead < kQpRun) issue(i + kQpAhead);
    __builtin_amdgcn_sched_barrier(0);
    // byte bb of the scale dwords of rows 4 q + r (+ 16 h)
    const f32x2 s01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)__builtin_amdgcn_perm(sw.y, sw.x, sel), false);
    const f32x2 s23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)__builtin_amdgcn_perm(sw.w, sw.z, sel), false);
#pragma unroll
    for (int xrow = 0; xrow < M; ++xrow) {
      acc[xrow].x = __builtin_fmaf(cv[xrow].x * cf[xrow], s01.x, acc[xrow].x);
      acc[xrow].y = __builtin_fmaf(cv[xrow].y * cf[xrow], s01.y, acc[xrow].y);
      acc[xrow].z = __builtin_fmaf(cv[xrow].z * cf[xrow], s23.x, acc[xrow].z);
      acc[xrow].w = __builtin_fmaf(cv[xrow].w * cf[xrow], s23.y, acc[xrow].w);
    }
  }
  flush(seg);
  lds_barrier();

  // 7. row sums: each tile's 16 wave slots in wave order (zeros from the
  //    waves whose runs miss the tile)
  for (int e = tid; e < nt * M * 32; e += kQpThreads) {
    const int tl = e / (M * 32), xrow = (e / 32) % M, r = e % 32;
    const float* ps_ = part + (tl * kQpWaves * M + xrow) * 32 + r;
    float pv[kQpWaves];
#pragma unroll
    for (int w = 0; w < kQpWaves; ++w) pv[w] = ps_[32 * M * w];
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kQpWaves; ++w) s += pv[w];
    const int64_t row = (int64_t)(t0 + tl) * 32 + r;
    if (row < n && xrow < m) reinterpret_cast<T*>(out)[(int64_t)xrow * n + row] = from_f32<DT>(s * dec_w);
  }
}

template <typename F>
hipError_t allow_qp_lds(F* kernel, size_t bytes) {
  static bool set[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev < 0 || dev >= 64 || set[dev]) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) set[dev] = true;
  return e;
}

// the largest LDS any k of the supported range needs with M rows of x
constexpr size_t qp_lds_max(int M) {
  size_t mx = 0;
  for (int s = kQpMinSteps; s <= kQpMaxSteps; ++s)
    if (qp_lds(s, M) > mx) mx = qp_lds(s, M);
  return mx;
}

template <int DT, int M, int XR>
hipError_t launch_qp_t(const void* x, int64_t m, const float* gx, const uint8_t* pc,
                       const uint8_t* ps, const float* gw, int64_t n, int64_t k, void* out,
                       hipStream_t s) {
  static_assert(qp_lds_max(M) <= 160 * 1024, "LDS");
  const int64_t steps = k / 64;
  const int64_t tiles = (n + 31) / 32;
  const int64_t per = (int64_t)kQpWaves * kQpRun / steps;  // tiles per workgroup at most
  int64_t blocks = tiles < device_cu_count() ? tiles : device_cu_count();
  if (blocks < (tiles + per - 1) / per) blocks = (tiles + per - 1) / per;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (hipError_t e = allow_qp_lds(qmv_packed_kernel<DT, M, XR>, qp_lds_max(M))) return e;
  qmv_packed_kernel<DT, M, XR><<<(int)blocks, kQpThreads, qp_lds((int)steps, M), s>>>(
      x, (int)m, gx, pc, ps, gw, (int)n, (int)steps, (int)(tiles / blocks), (int)(tiles % blocks), out);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_qp_dt(const void* x, int64_t m, const float* gx, const uint8_t* pc,
                        const uint8_t* ps, const float* gw, int64_t n, int64_t k, void* out,
                        hipStream_t s) {
  const bool wide = k > 4096;
  if (m == 1)
    return launch_qp_t<DT, 1, 1>(x, m, gx, pc, ps, gw, n, k, out, s);
  if (m == 2)
    return wide ? launch_qp_t<DT, 2, 2>(x, m, gx, pc, ps, gw, n, k, out, s)
                : launch_qp_t<DT, 2, 1>(x, m, gx, pc, ps, gw, n, k, out, s);
  return wide ? launch_qp_t<DT, 4, 4>(x, m, gx, pc, ps, gw, n, k, out, s)
              : launch_qp_t<DT, 4, 2>(x, m, gx, pc, ps, gw, n, k, out, s);
}

}  // namespace

// bfloat16 x only: the split of x_hat above is exact for it (see the top of
// the file); float16 x would reach T's subnormals with ordinary data.
bool qmv_packed_ok(int dt, int64_t m, int64_t k) {
  return dt == kBF16 && m >= 1 && m <= kQpMaxRows && k % 64 == 0 && k >= 64 * kQpMinSteps &&
         k <= 64 * kQpMaxSteps;
}

hipError_t launch_qmv_packed(const void* x, int dt, int64_t m, const float* gx, const uint8_t* pc,
                             const uint8_t* ps, const float* gw, int64_t n, int64_t k, void* out,
                             hipStream_t s) {
  if (dt != kBF16) return hipErrorInvalidValue;
  return launch_qp_dt<kBF16>(x, m, gx, pc, ps, gw, n, k, out, s);
}

}  // namespace nvfp4
