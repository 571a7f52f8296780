// mx_gemm.hip -- the block-scaled matrix-core product of the mx modes on
// gfx950: y[m, n] = T( sum_k x_hat[m, k] * w_hat[n, k] ) with both operands
// in mxfp4 or mxfp8 (the mode of "mlx 0.30.7.2 -> 0.30.7.6" diff, page 8,
// qqmm: x quantized in the same mode as w, the product of the two decodes).
//
// gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 takes e2m1 or e4m3 codes and one
// E8M0 scale per lane and 32-element block, so the codes and scales of the
// packed layout (mx_codec.hip) go to the matrix cores as loaded: no decode,
// no LDS.  Lane l (row i = l % 32, half h = l / 32) of a 32 x 64 operand
// fragment holds
//   mxfp4: codes k 32h .. 32h + 31 of row i (piece h of the step, 16 bytes);
//   mxfp8: codes k 16h .. 16h + 15 and 32 + 16h .. 32 + 16h + 15 (pieces h
//          and 2 + h, 2 x 16 bytes),
// and the scale of row i, block h of the step; with the packed layout each
// fragment is one (mxfp4) or two (mxfp8) contiguous 1 KB wave loads and the
// scales of 4 steps one 256-byte wave load (the MFMA's op_sel picks the
// step's byte).  Every product of two decoded values is exact in float32;
// the MFMA accumulates in float32.
//
// Tiling: a workgroup of 4 waves computes a 256 x 256 output tile, each wave
// 128 x 128 (4 x 4 MFMA tiles, 256 accumulators).  The weight is the MFMA's
// first operand, so a lane's 16 accumulator values of an MFMA tile are, in
// groups of 4, consecutive output columns of one output row.  Operand
// fragments are loaded straight into registers, kStages - 1 steps ahead of
// the MFMAs that use them; the two waves that share a fragment meet in L1.
// Buffer loads past the packed operand's end (padding tiles) return zeros.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

#include <type_traits>

namespace nvfp4 {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kMxgThreads = 256;
constexpr int kMxgTile = 256;                 // output rows and columns per workgroup
constexpr uint32_t kMxgOutside = 0x7FF00000u;  // a load offset past every operand's end

template <int BITS> struct MxgCfg;
template <> struct MxgCfg<4> {
  static constexpr int kFmt = 4;        // e2m1 operand format of the MFMA
  static constexpr int kStepBytes = 1024;
  static constexpr int kStages = 4;
};
template <> struct MxgCfg<8> {
  static constexpr int kFmt = 0;        // e4m3
  static constexpr int kStepBytes = 2048;
  static constexpr int kStages = 2;
};

template <int BITS>
__device__ __forceinline__ i32x8 load_frag(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  if constexpr (BITS == 4) {
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
  } else {
    const u32x4 hi =
        __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024u, 0, 0));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
}

template <int DT, int BITS>
__global__ void __launch_bounds__(kMxgThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
mx_gemm_kernel(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, uint32_t x_code_bytes,
               uint32_t x_scale_bytes, const uint8_t* __restrict__ wc,
               const uint8_t* __restrict__ ws, uint32_t w_code_bytes, uint32_t w_scale_bytes, int M,
               int N, int KQ, void* __restrict__ out, int tiles_m, int tiles) {
  using C = MxgCfg<BITS>;
  constexpr int SB = C::kStepBytes, NS = C::kStages, D = NS - 1;
  using T = typename Elem<DT>::T;

  // XCD-aware order: consecutive workgroups go to the 8 XCDs in turn, so XCD
  // x takes the contiguous tile range [x per, (x + 1) per), m fastest: the
  // workgroups of one XCD share weight tiles in its L2.
  const int per = (tiles + 7) / 8;
  const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (t >= tiles) return;
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KS = 4 * KQ;
  const int xt0 = tm * 8 + (wave >> 1) * 4;  // first 32-row tile of x (output rows)
  const int wt0 = tn * 8 + (wave & 1) * 4;   // first 32-row tile of w (output columns)

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xc, x_code_bytes);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(xs, x_scale_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wc, w_code_bytes);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(ws, w_scale_bytes);

  // this lane's byte offsets at step 0 / quad 0; tiles past an operand's end
  // get the outside offset
  uint32_t xo[4], wo[4], xso[4], wso[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t a = (uint64_t)(xt0 + i) * KS * SB, b = (uint64_t)(wt0 + i) * KS * SB;
    xo[i] = a < x_code_bytes ? (uint32_t)a + 16u * lane : kMxgOutside;
    wo[i] = b < w_code_bytes ? (uint32_t)b + 16u * lane : kMxgOutside;
    const uint64_t c = (uint64_t)(xt0 + i) * KQ * 256, d = (uint64_t)(wt0 + i) * KQ * 256;
    xso[i] = c < x_scale_bytes ? (uint32_t)c + 4u * lane : kMxgOutside;
    wso[i] = d < w_scale_bytes ? (uint32_t)d + 4u * lane : kMxgOutside;
  }

  i32x8 xf[NS][4], wf[NS][4];
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Fragments of step `st` into stage S, and the scales of quad q.  The
  // prefetches run up to D steps (one quad) past k: those read the next
  // tile's data or, past the operand's end, zeros (the buffer range check);
  // their values are never used.  No load is conditional, so the compiler
  // can count the loads in flight exactly.
  auto load_step = [&](auto stage_c, int st) {
    constexpr int S = decltype(stage_c)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xf[S][i] = load_frag<BITS>(rx, xo[i] + (uint32_t)st * SB);
      wf[S][i] = load_frag<BITS>(rw, wo[i] + (uint32_t)st * SB);
    }
  };
  uint32_t xsc[4], wsc[4], nxs[4], nws[4];
  auto load_scales = [&](uint32_t(&xd)[4], uint32_t(&wd)[4], int q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xd[i] = __builtin_amdgcn_raw_buffer_load_b32(rxs, xso[i] + (uint32_t)q * 256u, 0, 0);
      wd[i] = __builtin_amdgcn_raw_buffer_load_b32(rws, wso[i] + (uint32_t)q * 256u, 0, 0);
    }
  };
  // the 16 MFMAs of step s of a quad (op_sel s picks the step's scale byte)
  auto mfma_step = [&](auto s_c) {
    constexpr int S = decltype(s_c)::value;
    constexpr int st = S % NS;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            wf[st][j], xf[st][i], acc[i][j], C::kFmt, C::kFmt, S, (int)wsc[j], S, (int)xsc[i]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using J1 = std::integral_constant<int, (0 + D) % NS>;
  using J2 = std::integral_constant<int, (1 + D) % NS>;
  using J3 = std::integral_constant<int, (2 + D) % NS>;
  using J4 = std::integral_constant<int, (3 + D) % NS>;

  load_scales(xsc, wsc, 0);
  load_step(I0{}, 0);
  if constexpr (D >= 2) load_step(std::integral_constant<int, 1 % NS>{}, 1);
  if constexpr (D >= 3) load_step(std::integral_constant<int, 2 % NS>{}, 2);
  // the scheduling barriers keep each step's prefetch ahead of its MFMAs
  // (left alone, the scheduler sinks the loads next to their first use)
  for (int q = 0; q < KQ; ++q) {
    const int t0 = 4 * q;
    __builtin_amdgcn_sched_barrier(0);
    load_scales(nxs, nws, q + 1);
    load_step(J1{}, t0 + D);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(I0{});
    __builtin_amdgcn_sched_barrier(0);
    load_step(J2{}, t0 + 1 + D);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(I1{});
    __builtin_amdgcn_sched_barrier(0);
    load_step(J3{}, t0 + 2 + D);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(I2{});
    __builtin_amdgcn_sched_barrier(0);
    load_step(J4{}, t0 + 3 + D);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(I3{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xsc[i] = nxs[i];
      wsc[i] = nws[i];
    }
  }

  // epilogue: acc[i][j][4r + e] is output row 32 (xt0 + i) + lane % 32,
  // column 32 (wt0 + j) + 8 r + 4 (lane / 32) + e
  T* O = reinterpret_cast<T*>(out);
  typedef T T4 __attribute__((ext_vector_type(4)));
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * (xt0 + i) + (lane & 31);
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = 32 * (wt0 + j) + 8 * r + 4 * (lane >> 5);
        T4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = from_f32<DT>(acc[i][j][4 * r + e]);
        T* op = O + (int64_t)row * N + col;
        if (vec && col + 4 <= N) {
          *reinterpret_cast<T4*>(op) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < N) op[e] = v[e];
        }
      }
  }
}

}  // namespace

hipError_t launch_mx_gemm(const uint8_t* xpc, const uint8_t* xps, const uint8_t* wpc,
                          const uint8_t* wps, int bits, int64_t m, int64_t n, int64_t k, void* out,
                          int dt, hipStream_t s) {
  if (m == 0 || n == 0) return hipSuccess;
  const int KQ = (int)mx_packed_quads(k);
  const int tiles_m = (int)((m + kMxgTile - 1) / kMxgTile);
  const int tiles = tiles_m * (int)((n + kMxgTile - 1) / kMxgTile);
  const int blocks = 8 * ((tiles + 7) / 8);
  const uint32_t xcb = (uint32_t)mx_packed_code_bytes(m, k, bits);
  const uint32_t xsb = (uint32_t)mx_packed_scale_bytes(m, k);
  const uint32_t wcb = (uint32_t)mx_packed_code_bytes(n, k, bits);
  const uint32_t wsb = (uint32_t)mx_packed_scale_bytes(n, k);
#define MXG(D, B)                                                                                 \
  mx_gemm_kernel<D, B><<<blocks, kMxgThreads, 0, s>>>(xpc, xps, xcb, xsb, wpc, wps, wcb, wsb, (int)m, \
                                                       (int)n, KQ, out, tiles_m, tiles)
  if (bits == 4) {
    if (dt == kF32) MXG(kF32, 4);
    else if (dt == kF16) MXG(kF16, 4);
    else MXG(kBF16, 4);
  } else {
    if (dt == kF32) MXG(kF32, 8);
    else if (dt == kF16) MXG(kF16, 8);
    else MXG(kBF16, 8);
  }
#undef MXG
  return hipGetLastError();
}

}  // namespace nvfp4
