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
};
template <> struct MxgCfg<8> {
  static constexpr int kFmt = 0;        // e4m3
  static constexpr int kStepBytes = 2048;
};

// LDS staging.  One workgroup's operands of a step (its 8 x and 8 w
// fragments, 16 KB for mxfp4, 32 KB for mxfp8) are fetched once from L2
// straight into LDS (buffer_load ... lds, 16 bytes per lane: a 1 KB
// fragment piece lands as is) and read from there by the two waves that use
// each fragment.  NS stages are in flight (fetches run NS - 1 steps ahead);
// the E8M0 scales of a quad of steps travel the same way (one dword per lane
// and tile) into a ring of 4 quad slots.  Every step each wave issues the
// same number of fetches (its L code pieces and one scale piece), so one
// fixed vmcnt wait before each step's barrier covers "the next stage has
// landed", and the barrier also covers "every wave has read the stage that
// the next fetch overwrites".
template <int BITS> struct MxgLds;
template <> struct MxgLds<4> {
  static constexpr int kStages = 8;   // 8 x 16 KB
  static constexpr int kPieces = 4;   // 1 KB code pieces per wave and step
};
template <> struct MxgLds<8> {
  static constexpr int kStages = 4;   // 4 x 32 KB
  static constexpr int kPieces = 8;
};
constexpr int kScaleSlots = 4;        // quads of scales in flight (4 KB each)

template <int BITS>
constexpr size_t mx_gemm_lds_bytes() {
  return (size_t)MxgLds<BITS>::kStages * 16 * MxgCfg<BITS>::kStepBytes + kScaleSlots * 4096;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One fetch straight into LDS: lane l's 16 (or 4) bytes at `voff` land at
// dst + 16 l (4 l).  Device functions, not lambdas: the host pass then never
// instantiates the gfx950-only 16-byte form.
__device__ __forceinline__ void fetch16(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void fetch4(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 4, voff, 0, 0, 0);
}

template <int DT, int BITS>
__global__ void __launch_bounds__(kMxgThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
mx_gemm_kernel(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, uint32_t x_code_bytes,
               uint32_t x_scale_bytes, const uint8_t* __restrict__ wc,
               const uint8_t* __restrict__ ws, uint32_t w_code_bytes, uint32_t w_scale_bytes, int M,
               int N, int KQ, void* __restrict__ out, int tiles_m, int tiles) {
  using C = MxgCfg<BITS>;
  constexpr int SB = C::kStepBytes;                 // bytes of one fragment per step
  constexpr int NS = MxgLds<BITS>::kStages, L = MxgLds<BITS>::kPieces;
  constexpr int CPF = SB / 1024;                    // 1 KB pieces per fragment
  constexpr int kStageBytes = 16 * SB;
  constexpr int kWait = (NS - 2) * (L + 1);         // fetches allowed in flight at a step's barrier
  static_assert(kWait < 64, "vmcnt holds at most 63");
  using T = typename Elem<DT>::T;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* const scale_lds = lds + NS * kStageBytes;

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

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xc, x_code_bytes);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(xs, x_scale_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wc, w_code_bytes);
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(ws, w_scale_bytes);

  // Fragment f of a stage: f < 8 the x tile 8 tm + f, else the w tile
  // 8 tn + f - 8.  This wave fetches pieces c = wave + 4 j (j < L): fragment
  // c / CPF, piece c % CPF -- x for j < L / 2, w above.
  uint32_t go[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const int c = wave + 4 * j, f = c / CPF, sub = c % CPF;
    const bool isx = j < L / 2;
    const int tile = isx ? 8 * tm + f : 8 * tn + f - 8;
    const uint64_t a = (uint64_t)tile * KS * SB;
    go[j] = a < (isx ? x_code_bytes : w_code_bytes) ? (uint32_t)a + sub * 1024u + 16u * lane
                                                    : kMxgOutside;
  }
  // scale piece of part p (0..3) of a quad: fragment 4 p + wave
  uint32_t so[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int f = 4 * p + wave;
    const bool isx = f < 8;
    const int tile = isx ? 8 * tm + f : 8 * tn + f - 8;
    const uint64_t a = (uint64_t)tile * KQ * 256;
    so[p] = a < (isx ? x_scale_bytes : w_scale_bytes) ? (uint32_t)a + 4u * lane : kMxgOutside;
  }

  // the fetches of slot v: the code pieces of step v into stage v % NS, and
  // part v % 4 of the scales of quad v / 4 + 1 into its ring slot
  auto fetch_codes = [&](int v) {
    uint8_t* st = lds + (v % NS) * kStageBytes;
#pragma unroll
    for (int j = 0; j < L / 2; ++j) fetch16(rx, st + (wave + 4 * j) * 1024, go[j] + (uint32_t)v * SB);
#pragma unroll
    for (int j = L / 2; j < L; ++j) fetch16(rw, st + (wave + 4 * j) * 1024, go[j] + (uint32_t)v * SB);
  };
  auto fetch_scales = [&](int q, int p) {
    uint8_t* dst = scale_lds + (q % kScaleSlots) * 4096 + (4 * p + wave) * 256;
    fetch4(p < 2 ? rxs : rws, dst, so[p] + (uint32_t)q * 256u);
  };
  auto fetch_slot = [&](int v) {
    fetch_codes(v);
    fetch_scales(v / 4 + 1, v % 4);
  };
  // the wait through the builtin (the compiler then knows every LDS read has
  // returned), the barrier as an asm statement with a memory clobber (no
  // fetch or LDS read moves across it)
  auto step_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt((kWait & 15) | ((kWait >> 4) << 14) | (0x7 << 4));  // vmcnt(kWait) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
  };

  // operand registers of two steps, scales of two quads
  i32x8 xf[2][4], wf[2][4];
  uint32_t xsc[2][4], wsc[2][4];
  const int wm = wave >> 1, wn = wave & 1;
  auto read_step = [&](auto buf_c, int v) {
    constexpr int B = decltype(buf_c)::value;
    const uint8_t* st = lds + (v % NS) * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint8_t* px = st + (4 * wm + i) * SB + 16 * lane;
      const uint8_t* pw = st + (8 + 4 * wn + i) * SB + 16 * lane;
      const u32x4 a = *reinterpret_cast<const u32x4*>(px);
      const u32x4 b = *reinterpret_cast<const u32x4*>(pw);
      if constexpr (BITS == 4) {
        xf[B][i] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
        wf[B][i] = i32x8{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
      } else {
        const u32x4 a2 = *reinterpret_cast<const u32x4*>(px + 1024);
        const u32x4 b2 = *reinterpret_cast<const u32x4*>(pw + 1024);
        xf[B][i] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)a2.x, (int)a2.y, (int)a2.z, (int)a2.w};
        wf[B][i] = i32x8{(int)b.x, (int)b.y, (int)b.z, (int)b.w, (int)b2.x, (int)b2.y, (int)b2.z, (int)b2.w};
      }
    }
  };
  auto read_scales = [&](auto buf_c, int q) {
    constexpr int B = decltype(buf_c)::value;
    const uint8_t* sl = scale_lds + (q % kScaleSlots) * 4096 + 4 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xsc[B][i] = *reinterpret_cast<const uint32_t*>(sl + (4 * wm + i) * 256);
      wsc[B][i] = *reinterpret_cast<const uint32_t*>(sl + (8 + 4 * wn + i) * 256);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // the 16 MFMAs of a step at position S of its quad (op_sel S picks the
  // step's scale byte), operands from register set B, scales from set Q
  auto mfma_step = [&](auto s_c, auto b_c, auto q_c) {
    constexpr int S = decltype(s_c)::value, B = decltype(b_c)::value, Q = decltype(q_c)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            wf[B][j], xf[B][i], acc[i][j], C::kFmt, C::kFmt, S, (int)wsc[Q][j], S, (int)xsc[Q][i]);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  // prologue: quad 0's scales (all four parts), slots 0 .. NS - 2; then, as
  // at every step, wait for the next stage, meet, refill, read it
#pragma unroll
  for (int p = 0; p < 4; ++p) fetch_scales(0, p);
  for (int v = 0; v < NS - 1; ++v) fetch_slot(v);
  step_barrier();
  fetch_slot(NS - 1);
  read_step(I0{}, 0);
  read_scales(I0{}, 0);

  // step t: wait until stage t + 1 has landed and every wave has read stage
  // t, refill stage t with step t + NS, read step t + 1 (and at a quad's last
  // step the next quad's scales), then the MFMAs of step t
  auto step = [&](auto pos_c, auto qb_c, int tt) {
    constexpr int P = decltype(pos_c)::value, QB = decltype(qb_c)::value;
    constexpr int B = P % 2;
    __builtin_amdgcn_sched_barrier(0);
    step_barrier();
    fetch_slot(tt + NS);
    read_step(std::integral_constant<int, 1 - B>{}, tt + 1);
    if constexpr (P == 3) read_scales(std::integral_constant<int, 1 - QB>{}, tt / 4 + 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(pos_c, std::integral_constant<int, B>{}, qb_c);
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  int tt = 0;
  for (; tt + 8 <= KS; tt += 8) {
    step(I0{}, Q0{}, tt);
    step(I1{}, Q0{}, tt + 1);
    step(I2{}, Q0{}, tt + 2);
    step(I3{}, Q0{}, tt + 3);
    step(I0{}, Q1{}, tt + 4);
    step(I1{}, Q1{}, tt + 5);
    step(I2{}, Q1{}, tt + 6);
    step(I3{}, Q1{}, tt + 7);
  }
  if (tt < KS) {  // one quad left (KS is a multiple of 4)
    step(I0{}, Q0{}, tt);
    step(I1{}, Q0{}, tt + 1);
    step(I2{}, Q0{}, tt + 2);
    step(I3{}, Q0{}, tt + 3);
  }
  // no fetch may still be writing this workgroup's LDS when it ends
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

  // Epilogue through LDS: acc[i][j][4r + e] is output row 32 (4 wm + i) +
  // lane % 32 of the tile, column 32 (4 wn + j) + 8 r + 4 (lane / 32) + e.
  // The tile's rows (512 bytes of 16-bit output, 1 KB of float32) are staged
  // as 16-byte chunks, chunk c of tile row r in slot c ^ (r % 32) (the 32
  // rows written by one instruction land in different banks), then leave as
  // whole row segments, 16 bytes per lane.  A 16-bit tile (128 KB) goes in
  // one pass; a float32 tile in two of 128 rows (the rows of waves wm = 0,
  // then wm = 1).
  __syncthreads();  // every wave is done with the stages
  T* O = reinterpret_cast<T*>(out);
  constexpr int kChunks = 256 * (int)sizeof(T) / 16;   // 16-byte chunks per tile row
  constexpr int kPasses = sizeof(T) == 4 ? 2 : 1;
  constexpr int kRowsPerPass = 256 / kPasses;
  const int row0 = 256 * tm, col0 = 256 * tn;
  const bool vec = ((int64_t)N * (int64_t)sizeof(T)) % 16 == 0;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    if (kPasses == 1 || wm == pass) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int trow = 32 * (4 * wm + i) + (lane & 31) - pass * kRowsPerPass;
            const int tcol = 32 * (4 * wn + j) + 8 * r + 4 * (lane >> 5);  // first of 4 columns
            const int c = tcol * (int)sizeof(T) / 16;                       // its 16-byte chunk
            const int within = (tcol * (int)sizeof(T)) % 16;
            uint8_t* dst = lds + trow * (kChunks * 16) + ((c ^ (trow & 31)) * 16) + within;
            if constexpr (sizeof(T) == 4) {
              *reinterpret_cast<f32x4*>(dst) =
                  f32x4{acc[i][j][4 * r], acc[i][j][4 * r + 1], acc[i][j][4 * r + 2], acc[i][j][4 * r + 3]};
            } else {
              typedef T T4 __attribute__((ext_vector_type(4)));
              T4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = from_f32<DT>(acc[i][j][4 * r + e]);
              *reinterpret_cast<T4*>(dst) = v;
            }
          }
    }
    lds_barrier();
    // kChunks lanes per tile row
    constexpr int kRowsPerIter = kMxgThreads / kChunks;
    constexpr int kPer = 16 / (int)sizeof(T);
    for (int tr = threadIdx.x / kChunks; tr < kRowsPerPass; tr += kRowsPerIter) {
      const int c = threadIdx.x % kChunks;
      const int row = row0 + pass * kRowsPerPass + tr;
      const int col = col0 + c * kPer;
      if (row >= M || col >= N) continue;
      const u32x4 d = *reinterpret_cast<const u32x4*>(lds + tr * (kChunks * 16) + ((c ^ (tr & 31)) * 16));
      T* op = O + (int64_t)row * N + col;
      if (vec && col + kPer <= N) {
        *reinterpret_cast<u32x4*>(op) = d;
      } else {
        typedef T TV __attribute__((ext_vector_type(kPer)));
        const TV ev = __builtin_bit_cast(TV, d);
#pragma unroll
        for (int e = 0; e < kPer; ++e)
          if (col + e < N) op[e] = ev[e];
      }
    }
    if (kPasses > 1) lds_barrier();
  }
}

}  // namespace

namespace {

// the kernel's LDS exceeds the default limit: raise it once per device
template <typename F>
hipError_t allow_mx_lds(F* kernel, size_t bytes) {
  static bool set[64] = {false};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev < 0 || dev >= 64 || set[dev]) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) set[dev] = true;
  return e;
}

template <int DT, int BITS>
hipError_t launch_mx_gemm_t(const uint8_t* xpc, const uint8_t* xps, const uint8_t* wpc,
                            const uint8_t* wps, int64_t m, int64_t n, int64_t k, void* out,
                            hipStream_t s) {
  const int KQ = (int)mx_packed_quads(k);
  const int tiles_m = (int)((m + kMxgTile - 1) / kMxgTile);
  const int tiles = tiles_m * (int)((n + kMxgTile - 1) / kMxgTile);
  const int blocks = 8 * ((tiles + 7) / 8);
  const uint32_t xcb = (uint32_t)mx_packed_code_bytes(m, k, BITS);
  const uint32_t xsb = (uint32_t)mx_packed_scale_bytes(m, k);
  const uint32_t wcb = (uint32_t)mx_packed_code_bytes(n, k, BITS);
  const uint32_t wsb = (uint32_t)mx_packed_scale_bytes(n, k);
  if (hipError_t e = allow_mx_lds(mx_gemm_kernel<DT, BITS>, mx_gemm_lds_bytes<BITS>())) return e;
  mx_gemm_kernel<DT, BITS><<<blocks, kMxgThreads, mx_gemm_lds_bytes<BITS>(), s>>>(
      xpc, xps, xcb, xsb, wpc, wps, wcb, wsb, (int)m, (int)n, KQ, out, tiles_m, tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_gemm(const uint8_t* xpc, const uint8_t* xps, const uint8_t* wpc,
                          const uint8_t* wps, int bits, int64_t m, int64_t n, int64_t k, void* out,
                          int dt, hipStream_t s) {
  if (m == 0 || n == 0) return hipSuccess;
  if (bits == 4) {
    if (dt == kF32) return launch_mx_gemm_t<kF32, 4>(xpc, xps, wpc, wps, m, n, k, out, s);
    if (dt == kF16) return launch_mx_gemm_t<kF16, 4>(xpc, xps, wpc, wps, m, n, k, out, s);
    return launch_mx_gemm_t<kBF16, 4>(xpc, xps, wpc, wps, m, n, k, out, s);
  }
  if (dt == kF32) return launch_mx_gemm_t<kF32, 8>(xpc, xps, wpc, wps, m, n, k, out, s);
  if (dt == kF16) return launch_mx_gemm_t<kF16, 8>(xpc, xps, wpc, wps, m, n, k, out, s);
  return launch_mx_gemm_t<kBF16, 8>(xpc, xps, wpc, wps, m, n, k, out, s);
}

}  // namespace nvfp4
