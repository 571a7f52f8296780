// gemm.hip -- the M > 1 NVFP4 contractions for gfx950:
//   qqmm        out[m, n]    = T( sum_k x_hat[m, k] * w[n, k] )
//   gather_qmm  out[t, j, n] = T( sum_k x[t, k] * w_e[n, k] ),  e = idx[t, j]
// with w decoded with its global scale on every block scale ("mlx 0.30.7.2 ->
// 0.30.7.6" diff page 8, qqmm and page 7, QQMatmul::eval_gpu; "[Metal]
// global scale for qmm" PR 4458, statement: the global factor sits inside
// the dequantization, per expert for gather_qmm).
//
// 16-bit inputs run on the matrix cores (v_mfma_f32_16x16x32_bf16 / _f16):
//   * workgroup tile 256 x 256 x 64, four waves in a 2 x 2 grid, each wave a
//     128 x 128 block of 8 x 8 MFMA tiles with float32 accumulators;
//   * A (x_hat or the gathered x rows) is copied to LDS as is; B is read as
//     packed e2m1 codes + e4m3 scales, decoded by the VALU to T with the
//     effective scale e4m3(s) * g/2688 and written to LDS, so every weight
//     element is decoded once per workgroup;
//   * both LDS tiles are double-buffered: the global loads for k-step i + 1
//     are in flight while the MFMAs of step i run;
//   * LDS rows are 64 elements (128 B) with the 16-byte chunks XOR-swizzled by
//     row, so fragment reads of 16 consecutive rows hit distinct banks;
//   * the MFMA takes the weight fragment as its first operand, so each lane
//     ends with 4 consecutive output columns of one row (one 8-byte store).
// float32 inputs use a plain LDS-tiled FMA kernel with float32 weights.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmThreads = 256;
constexpr int kTileElems = BM * BK;  // 16-bit elements per LDS tile

template <int DT> struct Mfma;
template <> struct Mfma<kBF16> {
  using V8 = bf16x8;
  static __device__ __forceinline__ f32x4 run(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<kF16> {
  using V8 = f16x8;
  static __device__ __forceinline__ f32x4 run(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// element offset of chunk c (8 elements) of row r inside a 64-wide LDS tile
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ (r & 7)) << 3); }

// Decode 8 e2m1 codes of one dword with the effective block scale into T.
template <int DT>
__device__ __forceinline__ typename Mfma<DT>::V8 decode8(uint32_t word, float se) {
  typename Mfma<DT>::V8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
    o[i] = from_f32<DT>(e2m1_decode(word >> (4 * i)) * se);
  }
  return o;
}

template <int DT, bool GATHER>
__global__ void __launch_bounds__(kGemmThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_gemm_kernel(const void* __restrict__ a_base, const uint8_t* __restrict__ wc,
                 const uint8_t* __restrict__ ws, const float* __restrict__ gw, int M, int N, int K,
                 void* __restrict__ out, const int32_t* __restrict__ offsets,
                 const int32_t* __restrict__ perm, int top_k, int E) {
  using T = typename Elem<DT>::T;
  using V8 = typename Mfma<DT>::V8;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kTileElems];  // [buf][A,B]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---------------------------------------------------------------- tile origin
  const int n_tiles = (N + BN - 1) / BN;
  const int tile_n = blockIdx.x % n_tiles;
  int tile_m = blockIdx.x / n_tiles;
  int expert = 0;
  int row_lo = 0, row_count = M;  // rows [row_lo, row_lo + row_count) of the A/out row space
  if constexpr (GATHER) {
    // find the expert owning m-tile tile_m: experts' tiles are laid out in order
    int acc_tiles = 0;
    expert = -1;
    for (int e = 0; e < E; ++e) {
      int cnt = offsets[e + 1] - offsets[e];
      int tiles = (cnt + BM - 1) / BM;
      if (tile_m < acc_tiles + tiles) {
        expert = e;
        tile_m -= acc_tiles;
        row_lo = offsets[e];
        row_count = cnt;
        break;
      }
      acc_tiles += tiles;
    }
    if (expert < 0) return;
  }
  const int bm = tile_m * BM;  // first tile row, relative to row_lo
  const int bn = tile_n * BN;
  const int64_t w_rows_off = (int64_t)expert * N;
  const float dec_w = GATHER ? (gw ? gw[expert] / (kE4M3Max * kE2M1Max) : 1.0f) : global_decode(gw);

  // ---------------------------------------------------------------- A rows of this thread
  // Dense: tile row r is row r of x_hat and of out.  Gather: tile row r is the
  // pair p = perm[row_lo + r] routed to this expert; its A row is x[p / top_k]
  // and its output row is row p of out viewed as [t * top_k, n].
  // A chunk q = tid + 256 i (i < 8): tile row (tid >> 3) + 32 i, chunk tid & 7
  const int a_chunk = tid & 7;
  int64_t a_row[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = bm + (tid >> 3) + 32 * i;
    if (r < row_count) {
      if constexpr (GATHER) {
        int p = perm[row_lo + r];
        a_row[i] = p / top_k;
      } else {
        a_row[i] = r;
      }
    } else {
      a_row[i] = -1;
    }
  }
  // B rows of this thread: tile row (tid >> 1) + 128 i (i < 2), half tid & 1
  const int b_half = tid & 1;
  int64_t b_row[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int n = bn + (tid >> 1) + 128 * i;
    b_row[i] = (n < N) ? (w_rows_off + n) : -1;
  }

  const T* A = reinterpret_cast<const T*>(a_base);
  const int64_t kc = K >> 1;   // code bytes per row
  const int64_t ksc = K >> 4;  // scale bytes per row

  u32x4 a_reg[8];
  u32x4 b_code[2];
  uint32_t b_scale[2];

  // whole 64-wide k tiles with 16-byte aligned code rows and 2-byte aligned
  // scale pairs take the vector path; otherwise every group is loaded alone
  const bool k_aligned = (K % BK) == 0;
  auto load_tile = [&](int k0) {
    const bool full = k_aligned || (k0 + BK <= K);
    const bool bfull = k_aligned;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int kk = k0 + a_chunk * 8;
      if (a_row[i] >= 0 && (full || kk < K))
        a_reg[i] = *reinterpret_cast<const u32x4*>(A + a_row[i] * K + kk);
      else
        a_reg[i] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int g0 = (k0 >> 4) + 2 * b_half;  // first of the two groups
      if (b_row[i] >= 0 && bfull) {
        b_code[i] = *reinterpret_cast<const u32x4*>(wc + b_row[i] * kc + (int64_t)g0 * 8);
        b_scale[i] = *reinterpret_cast<const uint16_t*>(ws + b_row[i] * ksc + g0);
      } else {
        u32x4 c = {0, 0, 0, 0};
        uint32_t s = 0;
        if (b_row[i] >= 0) {
          if (g0 < (K >> 4)) {
            u32x2 lo = *reinterpret_cast<const u32x2*>(wc + b_row[i] * kc + (int64_t)g0 * 8);
            c.x = lo.x; c.y = lo.y;
            s = ws[b_row[i] * ksc + g0];
          }
          if (g0 + 1 < (K >> 4)) {
            u32x2 hi = *reinterpret_cast<const u32x2*>(wc + b_row[i] * kc + (int64_t)(g0 + 1) * 8);
            c.z = hi.x; c.w = hi.y;
            s |= (uint32_t)ws[b_row[i] * ksc + g0 + 1] << 8;
          }
        }
        b_code[i] = c;
        b_scale[i] = s;
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* la = lds[buf][0];
    uint16_t* lb = lds[buf][1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<u32x4*>(la + lds_off(r, a_chunk)) = a_reg[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int r = (tid >> 1) + 128 * i;
      float se0, se1;
      {
#pragma clang fp contract(off)
        se0 = e4m3_decode(b_scale[i] & 0xFFu) * dec_w;
        se1 = e4m3_decode((b_scale[i] >> 8) & 0xFFu) * dec_w;
      }
      uint32_t cw[4] = {b_code[i].x, b_code[i].y, b_code[i].z, b_code[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        V8 v = decode8<DT>(cw[j], j < 2 ? se0 : se1);
        *reinterpret_cast<V8*>(lb + lds_off(r, 4 * b_half + j)) = v;
      }
    }
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ktiles = (K + BK - 1) / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int fr = lane & 15;  // fragment row
  const int fc = lane >> 4;  // fragment chunk within a 32-wide k step
  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) load_tile((kt + 1) * BK);
    const uint16_t* la = lds[buf][0];
    const uint16_t* lb = lds[buf][1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      V8 af[8], bfv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        af[i] = *reinterpret_cast<const V8*>(la + lds_off(wm * 128 + i * 16 + fr, ks * 4 + fc));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bfv[j] = *reinterpret_cast<const V8*>(lb + lds_off(wn * 128 + j * 16 + fr, ks * 4 + fc));
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = Mfma<DT>::run(bfv[j], af[i], acc[j][i]);
    }
    if (kt + 1 < ktiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // acc[j][i][v]: row bm + wm*128 + i*16 + fr, column bn + wn*128 + j*16 + 4*fc + v
  T* O = reinterpret_cast<T*>(out);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = bm + wm * 128 + i * 16 + fr;
    if (r >= row_count) continue;
    int64_t orow;
    if constexpr (GATHER)
      orow = perm[row_lo + r];
    else
      orow = r;
    T* op = O + orow * N;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int c = bn + wn * 128 + j * 16 + 4 * fc;
      if (c + 3 < N && (N & 3) == 0) {
        typedef T T4 __attribute__((ext_vector_type(4)));
        T4 v;
        v[0] = from_f32<DT>(acc[j][i][0]);
        v[1] = from_f32<DT>(acc[j][i][1]);
        v[2] = from_f32<DT>(acc[j][i][2]);
        v[3] = from_f32<DT>(acc[j][i][3]);
        *reinterpret_cast<T4*>(op + c) = v;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (c + v < N) op[c + v] = from_f32<DT>(acc[j][i][v]);
      }
    }
  }
}

// ------------------------------------------------------------------ fast path (k % 64 == 0)
//
// Same tile (256 x 256 x 64) with the work split for gfx950:
//   * the four waves split the 256 output columns (64 each) and all share the
//     256 rows of A, so every weight element is decoded exactly once per
//     workgroup, by the wave that multiplies with it, straight into the MFMA
//     operand registers -- the decoded weights never touch LDS;
//   * A tiles and the raw NVFP4 weight tiles (codes + scales, 9/16 of a byte
//     per element) go global -> LDS with global_load_lds_dwordx4, no VGPRs;
//     A has 3 LDS stages, raw weights 4, so loads are issued two k-steps
//     before their use and one barrier per k-step suffices;
//   * in k-step i a wave runs its 128 MFMAs on stage i while it decodes the
//     weights of step i + 1 (two codes per v_cvt_scalef32_pk_f32_fp4, one
//     multiply by e4m3(s) * g/2688, two values per v_cvt_pk_bf16_f32);
//   * inside a 64-wide k-step, MFMA lane group g (= lane / 16) takes the 16
//     consecutive k of weight group g (8 per 16x16x32 step): one 8-byte code
//     load and one scale byte per column; A is read with the same k order;
//   * workgroups are mapped so that each of the 8 XCDs (round-robin dispatch)
//     works on its own contiguous set of weight column panels.
constexpr int kStagesA = 3, kStagesB = 4;
constexpr int kAStageBytes = BM * BK * 2;                   // 32 KB of 16-bit A
constexpr int kBCodeBytes = BN * BK / 2;                    // 8 KB of codes
constexpr int kBStageBytes = kBCodeBytes + BN * BK / 16;    // + 1 KB of scales
constexpr int kLoadsPerStage = 8 + 2 + 1;                   // per wave: A, codes, scales

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void g2lds16(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* g, uint8_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 4, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <int DT>
__device__ __forceinline__ typename Mfma<DT>::V8 decode_frag(uint32_t codes, float se) {
  float q[8];
  e2m1_decode8_f32(codes, q);
  typename Mfma<DT>::V8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
    o[i] = from_f32<DT>(q[i] * se);
  }
  return o;
}

template <int DT, bool GATHER>
__global__ void __launch_bounds__(kGemmThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_gemm_fast_kernel(const void* __restrict__ a_base, const uint8_t* __restrict__ wc,
                      const uint8_t* __restrict__ ws, const float* __restrict__ gw, int M, int N,
                      int K, void* __restrict__ out, const int32_t* __restrict__ offsets,
                      const int32_t* __restrict__ perm, int top_k, int E, int tiles_m) {
  using T = typename Elem<DT>::T;
  using V8 = typename Mfma<DT>::V8;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStagesA * kAStageBytes + kStagesB * kBStageBytes];
  __shared__ int64_t out_rows[BM];
  uint8_t* const lds_a = smem;
  uint8_t* const lds_b = smem + kStagesA * kAStageBytes;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---------------------------------------------------------------- tile of this workgroup
  int L = blockIdx.x;
  if ((gridDim.x & 7) == 0) L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int tile_n = L / tiles_m;
  int tile_m = L % tiles_m;
  int expert = 0, row_lo = 0, row_count = M;
  if constexpr (GATHER) {
    int acc_tiles = 0;
    expert = -1;
    for (int e = 0; e < E; ++e) {
      const int cnt = offsets[e + 1] - offsets[e];
      const int tiles = (cnt + BM - 1) / BM;
      if (tile_m < acc_tiles + tiles) {
        expert = e;
        tile_m -= acc_tiles;
        row_lo = offsets[e];
        row_count = cnt;
        break;
      }
      acc_tiles += tiles;
    }
    if (expert < 0) return;
  }
  const int bm = tile_m * BM;
  const int bn = tile_n * BN;
  const float dec_w = GATHER ? (gw ? gw[expert] / (kE4M3Max * kE2M1Max) : 1.0f) : global_decode(gw);
  const int64_t w_row0 = (int64_t)expert * N;

  // output row of each tile row (-1: outside the tile's row count)
  for (int r = threadIdx.x; r < BM; r += kGemmThreads) {
    int64_t o = -1;
    if (bm + r < row_count) {
      if constexpr (GATHER)
        o = perm[row_lo + bm + r];
      else
        o = bm + r;
    }
    out_rows[r] = o;
  }

  // ---------------------------------------------------------------- load addresses
  // A: instruction j of wave w fills LDS 16-byte slots (w*8 + j)*64 + lane:
  // tile row r = (w*8 + j)*8 + lane/8, slot p = lane % 8 holding k-chunk p ^ (r % 8).
  const T* A = reinterpret_cast<const T*>(a_base);
  const T* a_src[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (wave * 8 + j) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (r & 7);
    int64_t arow;
    const int rr = (bm + r < row_count) ? r : 0;  // rows past the count re-read row 0
    if constexpr (GATHER)
      arow = perm[row_lo + bm + rr] / top_k;
    else
      arow = bm + rr;
    a_src[j] = A + arow * K + chunk * 8;
  }
  // codes: instruction j of wave w fills bytes ((w*2 + j)*64 + lane)*16 of the code tile:
  // tile column (w*2 + j)*32 + lane/2, half lane % 2 (16 of its 32 bytes per k-step)
  const uint8_t* c_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = (wave * 2 + j) * 32 + (lane >> 1);
    const int64_t wrow = w_row0 + min(bn + col, N - 1);
    c_src[j] = wc + wrow * (K / 2) + (lane & 1) * 16;
  }
  // scales: wave w fills 4-byte slots w*64 + lane = tile column, 4 scale bytes per k-step
  const uint8_t* s_src = ws + (w_row0 + min(bn + wave * 64 + lane, N - 1)) * (K / 16);

  auto issue_a = [&](int kt) {
    uint8_t* dst = lds_a + (kt % kStagesA) * kAStageBytes + wave * 8 * 1024;
#pragma unroll
    for (int j = 0; j < 8; ++j) g2lds16(a_src[j] + kt * BK, dst + j * 1024);
  };
  auto issue_b = [&](int kt) {
    uint8_t* dst = lds_b + (kt % kStagesB) * kBStageBytes;
#pragma unroll
    for (int j = 0; j < 2; ++j) g2lds16(c_src[j] + kt * (BK / 2), dst + (wave * 2 + j) * 1024);
    g2lds4(s_src + kt * (BK / 16), dst + kBCodeBytes + wave * 256);
  };

  // ---------------------------------------------------------------- operand fragments
  const int fr = lane & 15;  // MFMA row / column inside a 16 x 16 tile
  const int fg = lane >> 4;  // k group: elements 16 fg .. 16 fg + 15 of a k-step
  V8 bcur[4][2], bnext[4][2];
  auto decode_b = [&](int kt, V8 (&dst)[4][2]) {
    const uint8_t* src = lds_b + (kt % kStagesB) * kBStageBytes;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int col = wave * 64 + t * 16 + fr;
      const u32x2 code = *reinterpret_cast<const u32x2*>(src + col * 32 + fg * 8);
      const uint32_t sbyte = src[kBCodeBytes + col * 4 + fg];
      float se;
      {
#pragma clang fp contract(off)
        se = e4m3_decode(sbyte) * dec_w;
      }
      dst[t][0] = decode_frag<DT>(code.x, se);
      dst[t][1] = decode_frag<DT>(code.y, se);
    }
  };

  f32x4 acc[4][16];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---------------------------------------------------------------- prologue
  const int KT = K / BK;
  issue_a(0);
  issue_b(0);
  if (KT > 1) { issue_a(1); issue_b(1); }
  if (KT > 2) issue_b(2);
  wait_vmcnt<0>();
  __syncthreads();
  decode_b(0, bcur);

  // ---------------------------------------------------------------- main loop
  for (int kt = 0; kt < KT; ++kt) {
    if (kt > 0) {
      // A(kt) and raw B(kt + 1) were issued two steps ago (or in the
      // prologue); what the previous step issued may stay in flight: A(kt + 1)
      // and B(kt + 2) while both exist, A(kt + 1) alone when B(kt + 2) is past
      // the end, nothing at the last step
      if (kt + 3 <= KT)
        wait_vmcnt<kLoadsPerStage>();
      else if (kt + 2 == KT)
        wait_vmcnt<8>();
      else
        wait_vmcnt<0>();
      __syncthreads();
    }
    if (kt + 2 < KT) issue_a(kt + 2);
    if (kt + 3 < KT) issue_b(kt + 3);
    const uint8_t* la = lds_a + (kt % kStagesA) * kAStageBytes;
    const bool more = (kt + 1 < KT);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = i * 16 + fr;
        const V8 a = *reinterpret_cast<const V8*>(la + m * 128 + (((2 * fg + s) ^ (m & 7)) << 4));
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t][i] = Mfma<DT>::run(bcur[t][s], a, acc[t][i]);
        if (s == 0 && i == 7 && more) decode_b(kt + 1, bnext);
      }
    }
    if (more) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bcur[t][0] = bnext[t][0];
        bcur[t][1] = bnext[t][1];
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  // acc[t][i][v]: tile row 16 i + fr, tile column 64 w + 16 t + 4 fg + v
  T* O = reinterpret_cast<T*>(out);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t orow = out_rows[i * 16 + fr];
    if (orow < 0) continue;
    T* op = O + orow * N;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = bn + wave * 64 + t * 16 + 4 * fg;
      if (c + 3 < N) {
        typedef T T4 __attribute__((ext_vector_type(4)));
        T4 v;
        v[0] = from_f32<DT>(acc[t][i][0]);
        v[1] = from_f32<DT>(acc[t][i][1]);
        v[2] = from_f32<DT>(acc[t][i][2]);
        v[3] = from_f32<DT>(acc[t][i][3]);
        *reinterpret_cast<T4*>(op + c) = v;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (c + v < N) op[c + v] = from_f32<DT>(acc[t][i][v]);
      }
    }
  }
}

// ------------------------------------------------------------------ float32 path

constexpr int FT = 64, FK = 16;

// out tile 64 x 64, 256 threads with 4 x 4 outputs each; the weight tile is
// decoded to float32 e2m1(q) * (e4m3(s) * g/2688) while staged in LDS.
template <bool GATHER>
__global__ void __launch_bounds__(256)
f32_gemm_kernel(const float* __restrict__ A, const uint8_t* __restrict__ wc,
                const uint8_t* __restrict__ ws, const float* __restrict__ gw, int M, int N, int K,
                float* __restrict__ out, const int32_t* __restrict__ offsets,
                const int32_t* __restrict__ perm, int top_k, int E) {
  __shared__ float la[FK][FT + 1];
  __shared__ float lb[FK][FT + 1];
  __shared__ int64_t arow[FT];
  __shared__ int64_t orow_s[FT];
  const int tid = threadIdx.x;
  const int n_tiles = (N + FT - 1) / FT;
  const int tile_n = blockIdx.x % n_tiles;
  int tile_m = blockIdx.x / n_tiles;
  int expert = 0, row_lo = 0, row_count = M;
  if constexpr (GATHER) {
    int acc_tiles = 0;
    expert = -1;
    for (int e = 0; e < E; ++e) {
      int cnt = offsets[e + 1] - offsets[e];
      int tiles = (cnt + FT - 1) / FT;
      if (tile_m < acc_tiles + tiles) {
        expert = e;
        tile_m -= acc_tiles;
        row_lo = offsets[e];
        row_count = cnt;
        break;
      }
      acc_tiles += tiles;
    }
    if (expert < 0) return;
  }
  const int bm = tile_m * FT, bn = tile_n * FT;
  const float dec_w = GATHER ? (gw ? gw[expert] / (kE4M3Max * kE2M1Max) : 1.0f) : global_decode(gw);
  if (tid < FT) {
    int r = bm + tid;
    if (r < row_count) {
      if constexpr (GATHER) {
        int p = perm[row_lo + r];
        arow[tid] = p / top_k;
        orow_s[tid] = p;
      } else {
        arow[tid] = r;
        orow_s[tid] = r;
      }
    } else {
      arow[tid] = -1;
      orow_s[tid] = -1;
    }
  }
  __syncthreads();
  const int64_t wbase = (int64_t)expert * N;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FK) {
    // 64 x 16 of A and of W: 1024 elements each, 4 per thread
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int e = tid + 256 * q;
      int r = e >> 4, kk = e & 15;
      int k = k0 + kk;
      float av = 0.f;
      if (arow[r] >= 0 && k < K) av = A[arow[r] * K + k];
      la[kk][r] = av;
      float wv = 0.f;
      int n = bn + r;
      if (n < N && k < K) {
        int64_t row = wbase + n;
        uint32_t byte = wc[row * (K >> 1) + (k >> 1)];
        uint32_t code = (k & 1) ? (byte >> 4) : (byte & 15u);
        float se;
        {
#pragma clang fp contract(off)
          se = e4m3_decode(ws[row * (K >> 4) + (k >> 4)]) * dec_w;
          wv = e2m1_decode(code) * se;
        }
      }
      lb[kk][r] = wv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = la[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = lb[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t orow = orow_s[ty * 4 + i];
    if (orow < 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int n = bn + tx * 4 + j;
      if (n < N) out[orow * N + n] = acc[i][j];
    }
  }
}

// ------------------------------------------------------------------ routing

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteMaxE = 1024;

// Groups of equal experts inside one wave: returns the lanes (bit mask) that
// share this lane's expert; the lowest lane of each group also records the
// group's expert and size through `on_group`.
template <typename F>
__device__ __forceinline__ uint64_t match_experts(int e, bool valid, F on_group) {
  uint64_t remaining = __ballot(valid);
  uint64_t same = 0;
  while (remaining) {
    const int leader = __builtin_ctzll(remaining);
    const int le = __shfl(e, leader, 64);
    const uint64_t m = __ballot(valid && e == le);
    if (valid && e == le) same = m;
    if ((int)(threadIdx.x & 63) == leader) on_group(le, __builtin_popcountll(m));
    remaining &= ~m;
  }
  return same;
}

// One workgroup of 1024 lanes.  Pass 1 counts pairs per expert (one LDS
// atomic per expert group of a wave), then an exclusive scan gives the
// expert offsets.  Pass 2 walks the pairs again in chunks of 1024 in order:
// a pair's slot is its expert's running base, plus the same-expert pairs of
// earlier waves of the chunk (a per-wave count table), plus its rank among
// the same-expert lanes of its wave -- i.e. ascending pair id within each
// expert.  Out-of-range experts are skipped.
__global__ void __launch_bounds__(kRouteThreads)
moe_route_kernel(const int32_t* __restrict__ idx, int total, int E, int32_t* __restrict__ offsets,
                 int32_t* __restrict__ perm) {
  __shared__ int base[kRouteMaxE];
  __shared__ int scan[kRouteThreads];
  __shared__ int wcnt[kRouteWaves * kRouteMaxE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = tid; e < E; e += kRouteThreads) base[e] = 0;
  __syncthreads();
  for (int c0 = 0; c0 < total; c0 += kRouteThreads) {
    const int p = c0 + tid;
    const int e = (p < total) ? idx[p] : -1;
    const bool valid = (e >= 0 && e < E);
    match_experts(e, valid, [&](int le, int cnt) { atomicAdd(&base[le], cnt); });
  }
  __syncthreads();
  // exclusive scan of the counts (E <= 1024, one entry per lane)
  const int mycount = (tid < E) ? base[tid] : 0;
  scan[tid] = mycount;
  __syncthreads();
  for (int off = 1; off < kRouteThreads; off <<= 1) {
    const int v = (tid >= off) ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    const int excl = scan[tid] - mycount;
    offsets[tid] = excl;
    base[tid] = excl;
  }
  if (tid == kRouteThreads - 1) offsets[E] = scan[tid];
  __syncthreads();

  for (int c0 = 0; c0 < total; c0 += kRouteThreads) {
    for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) wcnt[i] = 0;
    __syncthreads();
    const int p = c0 + tid;
    const int e = (p < total) ? idx[p] : -1;
    const bool valid = (e >= 0 && e < E);
    const uint64_t same =
        match_experts(e, valid, [&](int le, int cnt) { wcnt[wave * E + le] = cnt; });
    __syncthreads();
    if (valid) {
      int pos = base[e] + __builtin_popcountll(same & ((1ull << lane) - 1ull));
      for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
      perm[pos] = p;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kRouteThreads) {
      int add = 0;
      for (int w = 0; w < kRouteWaves; ++w) add += wcnt[w * E + x];
      base[x] += add;
    }
    __syncthreads();
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_qqmm_gemm(const void* xhat, int dt, const uint8_t* wc, const uint8_t* ws,
                            const float* gw, int64_t m, int64_t n, int64_t k, void* out,
                            hipStream_t s) {
  if (dt == kF32) {
    int64_t blocks = ((m + FT - 1) / FT) * ((n + FT - 1) / FT);
    f32_gemm_kernel<false><<<(int)blocks, 256, 0, s>>>(
        reinterpret_cast<const float*>(xhat), wc, ws, gw, (int)m, (int)n, (int)k,
        reinterpret_cast<float*>(out), nullptr, nullptr, 1, 1);
    return hipGetLastError();
  }
  int64_t blocks = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  if (k % BK == 0 && n % 4 == 0) {
    const int tiles_m = (int)((m + BM - 1) / BM);
    if (dt == kF16)
      mfma_gemm_fast_kernel<kF16, false><<<(int)blocks, kGemmThreads, 0, s>>>(
          xhat, wc, ws, gw, (int)m, (int)n, (int)k, out, nullptr, nullptr, 1, 1, tiles_m);
    else
      mfma_gemm_fast_kernel<kBF16, false><<<(int)blocks, kGemmThreads, 0, s>>>(
          xhat, wc, ws, gw, (int)m, (int)n, (int)k, out, nullptr, nullptr, 1, 1, tiles_m);
    return hipGetLastError();
  }
  if (dt == kF16)
    mfma_gemm_kernel<kF16, false><<<(int)blocks, kGemmThreads, 0, s>>>(
        xhat, wc, ws, gw, (int)m, (int)n, (int)k, out, nullptr, nullptr, 1, 1);
  else
    mfma_gemm_kernel<kBF16, false><<<(int)blocks, kGemmThreads, 0, s>>>(
        xhat, wc, ws, gw, (int)m, (int)n, (int)k, out, nullptr, nullptr, 1, 1);
  return hipGetLastError();
}

hipError_t launch_moe_route(const int32_t* idx, int64_t t, int64_t top_k, int64_t e,
                            int32_t* offsets, int32_t* perm, hipStream_t s) {
  moe_route_kernel<<<1, kRouteThreads, 0, s>>>(idx, (int)(t * top_k), (int)e, offsets, perm);
  return hipGetLastError();
}

hipError_t launch_gather_gemm(const void* x, int dt, const uint8_t* wc, const uint8_t* ws,
                              const float* gw, const int32_t* offsets, const int32_t* perm,
                              int64_t t, int64_t top_k, int64_t e, int64_t n, int64_t k,
                              void* out, hipStream_t s) {
  const int64_t pairs = t * top_k;
  if (dt == kF32) {
    int64_t mt = (pairs + FT - 1) / FT + e;
    int64_t blocks = mt * ((n + FT - 1) / FT);
    f32_gemm_kernel<true><<<(int)blocks, 256, 0, s>>>(
        reinterpret_cast<const float*>(x), wc, ws, gw, (int)pairs, (int)n, (int)k,
        reinterpret_cast<float*>(out), offsets, perm, (int)top_k, (int)e);
    return hipGetLastError();
  }
  int64_t mt = (pairs + BM - 1) / BM + e;
  int64_t blocks = mt * ((n + BN - 1) / BN);
  if (k % BK == 0 && n % 4 == 0) {
    if (dt == kF16)
      mfma_gemm_fast_kernel<kF16, true><<<(int)blocks, kGemmThreads, 0, s>>>(
          x, wc, ws, gw, (int)pairs, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e, (int)mt);
    else
      mfma_gemm_fast_kernel<kBF16, true><<<(int)blocks, kGemmThreads, 0, s>>>(
          x, wc, ws, gw, (int)pairs, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e, (int)mt);
    return hipGetLastError();
  }
  if (dt == kF16)
    mfma_gemm_kernel<kF16, true><<<(int)blocks, kGemmThreads, 0, s>>>(
        x, wc, ws, gw, (int)pairs, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e);
  else
    mfma_gemm_kernel<kBF16, true><<<(int)blocks, kGemmThreads, 0, s>>>(
        x, wc, ws, gw, (int)pairs, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e);
  return hipGetLastError();
}

}  // namespace nvfp4
