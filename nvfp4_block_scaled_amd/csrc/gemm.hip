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

// One workgroup: per-expert counts, exclusive scan, then a stable scatter of
// the pair ids in chunks of 1024 (rank inside a wave from ballots of equal
// experts, wave offsets from a per-chunk table).  Out-of-range experts are
// skipped.
__global__ void __launch_bounds__(kRouteThreads)
moe_route_kernel(const int32_t* __restrict__ idx, int total, int E, int32_t* __restrict__ offsets,
                 int32_t* __restrict__ perm) {
  __shared__ int counts[kRouteMaxE];
  __shared__ int base[kRouteMaxE];
  __shared__ int wcount[kRouteWaves][64];  // per wave: counts of the (up to 64) experts it saw
  __shared__ int wexp[kRouteWaves][64];    // ... and which experts they are
  __shared__ int wn[kRouteWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = tid; e < E; e += kRouteThreads) counts[e] = 0;
  __syncthreads();
  for (int p = tid; p < total; p += kRouteThreads) {
    int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&counts[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = run;
      base[e] = run;
      run += counts[e];
    }
    offsets[E] = run;
  }
  __syncthreads();
  for (int c0 = 0; c0 < total; c0 += kRouteThreads) {
    const int p = c0 + tid;
    const int e = (p < total) ? idx[p] : -1;
    const bool valid = (e >= 0 && e < E);
    // groups of equal experts inside this wave, in lane order
    uint64_t remaining = __ballot(valid);
    uint64_t same = 0;
    int ngroups = 0;
    while (remaining) {
      int leader = __builtin_ctzll(remaining);
      int le = __shfl(e, leader, 64);
      uint64_t m = __ballot(valid && e == le);
      if (valid && e == le) same = m;
      if (lane == 0) {
        wexp[wave][ngroups] = le;
        wcount[wave][ngroups] = __builtin_popcountll(m);
      }
      ++ngroups;
      remaining &= ~m;
    }
    if (lane == 0) wn[wave] = ngroups;
    const int rank = __builtin_popcountll(same & ((1ull << lane) - 1ull));
    __syncthreads();
    if (valid) {
      int before = 0;  // same-expert pairs of earlier waves in this chunk
      for (int w = 0; w < wave; ++w)
        for (int g = 0; g < wn[w]; ++g)
          if (wexp[w][g] == e) before += wcount[w][g];
      perm[base[e] + before + rank] = p;
    }
    __syncthreads();
    // advance the per-expert bases by this chunk's counts
    if (tid == 0) {
      for (int w = 0; w < kRouteWaves; ++w)
        for (int g = 0; g < wn[w]; ++g) base[wexp[w][g]] += wcount[w][g];
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
  if (dt == kF16)
    mfma_gemm_kernel<kF16, true><<<(int)blocks, kGemmThreads, 0, s>>>(
        x, wc, ws, gw, (int)pairs, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e);
  else
    mfma_gemm_kernel<kBF16, true><<<(int)blocks, kGemmThreads, 0, s>>>(
        x, wc, ws, gw, (int)pairs, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e);
  return hipGetLastError();
}

}  // namespace nvfp4
