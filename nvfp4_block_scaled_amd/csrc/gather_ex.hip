// gather_ex.hip -- the indexed forms of gather_qmm on gfx950: routing of
// already sorted expert indices, the x-row map of lhs indices, and the
// contraction with weights stored [K, N] (transpose = False).
//
// The op ("[Metal] global scale for qmm" (ml-explore/mlx PR 4458): statement
// and test loops over float32 / float16 / bfloat16 and transpose True /
// False, per-expert global scales [E, 1, 1]; the op's lhs_indices /
// rhs_indices / sorted_indices): x is [b, mr, k]; pair p multiplies x entry
// lhs[p] (p without lhs) by expert rhs[p]; output rows p * mr .. p * mr +
// mr - 1.  With transpose = False expert e's weight is [K, N] quantized along
// N, and the output is x @ w_e.
#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

// Sorted expert indices: the rows of expert e are [mr lb(e), mr lb(e + 1))
// with lb(e) the number of pairs whose expert is below e (a binary search),
// and the permutation is the identity.
__global__ void __launch_bounds__(256)
sorted_route_kernel(const int32_t* __restrict__ rhs, int pairs, int mr, int E,
                    int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                    uint8_t* __restrict__ zero_out, int64_t row_bytes) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  if (tid <= E) {
    int lo = 0, hi = pairs;  // first pair with rhs >= tid
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (rhs[mid] < tid) lo = mid + 1; else hi = mid;
    }
    offsets[tid] = lo * mr;
  }
  const int rows = pairs * mr;
  const int stride = gridDim.x * blockDim.x;
  for (int q = tid; q < rows; q += stride) perm[q] = q;
  if (zero_out) {
    // rows whose expert lies outside [0, E) (before offsets[0] or from
    // offsets[E] on): no product touches them, so they get zeros here
    for (int q0 = tid & ~63; q0 < rows; q0 += stride) {  // wave-uniform
      const int q = q0 + (threadIdx.x & 63);
      int x = 0;
      if (q < rows) x = rhs[q / mr];
      uint64_t bad = __ballot(q < rows && !(x >= 0 && x < E));
      while (bad) {
        zero_row_wave(zero_out, (int64_t)(q0 + __builtin_ctzll(bad)), row_bytes);
        bad &= bad - 1ull;
      }
    }
  }
}

// x row of each routed row: amap[s] = lhs[q / mr] mr + q % mr, q = perm[s].
__global__ void __launch_bounds__(256)
amap_kernel(const int32_t* __restrict__ perm, const int32_t* __restrict__ lhs, int rows, int mr,
            int32_t* __restrict__ amap) {
  for (int s = blockIdx.x * blockDim.x + threadIdx.x; s < rows; s += gridDim.x * blockDim.x) {
    const int q = perm[s];
    amap[s] = lhs[q / mr] * mr + q % mr;
  }
}

// ------------------------------------------------------------------ transpose = False

// 128 x 128 output tiles, k steps of 64.  The weight tile (64 rows of k, 128
// columns of n: 64 code bytes and 8 scales per row) is decoded once per
// workgroup -- each thread 8 consecutive columns (one block scale per row) of
// 4 consecutive rows -- and written transposed into LDS as [n][k], 4 k values
// of a column per 8-byte store, so that both operand fragments of the
// 32x32x16 MFMA are 16-byte LDS reads (8 k values of one row).  The next
// step's raw weights are fetched into registers before this step's MFMAs.
// The A rows are gathered through perm / amap as in the other gather kernels;
// they go from global memory straight into two alternating LDS stages
// (buffer_load ... lds: no registers, no LDS store instructions), each tile
// row 128 bytes with its 16-byte k chunks XOR-swizzled by the row.  An x of
// 2 GB or more (beyond 32-bit offsets) takes them through registers instead.
constexpr int kTT = 128;
constexpr int kTK = 64;
constexpr int kPitch = kTK + 8;  // LDS row pitch in elements (144 bytes)

template <int DT> struct MfmaT;
template <> struct MfmaT<kBF16> {
  typedef __bf16 V8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 run(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct MfmaT<kF16> {
  typedef _Float16 V8 __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ f32x16 run(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

typedef __attribute__((address_space(3))) void* lds_ptr_g;
constexpr uint32_t kGxOutside = 0x7FF00000u;  // a load offset past the end of x

__device__ __forceinline__ void gx_fetch16(__amdgpu_buffer_rsrc_t rs, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_g)dst, 16, voff, 0, 0, 0);
}

template <int DT, bool DMA>
__global__ void __launch_bounds__(256)
gather_t_kernel(const void* __restrict__ x, int64_t x_rows, int K, const uint8_t* __restrict__ wc,
                const uint8_t* __restrict__ ws, const float* __restrict__ gw, int N,
                void* __restrict__ out, const int32_t* __restrict__ offsets,
                const int32_t* __restrict__ perm, int top_k, int E, const int32_t* __restrict__ amap) {
  using T = typename Elem<DT>::T;
  using V8 = typename MfmaT<DT>::V8;
  // A: padded rows (register path) or two swizzled stages (DMA path)
  __shared__ __attribute__((aligned(1024))) T la[DMA ? 2 * kTT * kTK : kTT * kPitch];
  __shared__ __attribute__((aligned(16))) T lb[kTT * kPitch];
  __shared__ int64_t arow_s[kTT];
  __shared__ int orow_s[kTT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // the expert and rows of this tile (tiles of all experts in order)
  const int n_tiles = (N + kTT - 1) / kTT;
  const int tile_n = blockIdx.x % n_tiles;
  int tile_m = blockIdx.x / n_tiles;
  int expert = -1, row_lo = 0, row_count = 0;
  {
    int acc_tiles = 0;
    for (int e = 0; e < E; ++e) {
      const int cnt = offsets[e + 1] - offsets[e];
      const int tiles = (cnt + kTT - 1) / kTT;
      if (tile_m < acc_tiles + tiles) {
        expert = e;
        tile_m -= acc_tiles;
        row_lo = offsets[e];
        row_count = cnt;
        break;
      }
      acc_tiles += tiles;
    }
  }
  if (expert < 0) return;
  const int bm = tile_m * kTT, bn = tile_n * kTT;
  const float dec_w = gw ? gw[expert] / (kE4M3Max * kE2M1Max) : 1.0f;
  if (tid < kTT) {
    const int r = bm + tid;
    if (r < row_count) {
      const int p = perm[row_lo + r];
      arow_s[tid] = amap ? amap[row_lo + r] : p / top_k;
      orow_s[tid] = p;
    } else {
      arow_s[tid] = -1;
      orow_s[tid] = -1;
    }
  }
  __syncthreads();

  const uint8_t* wce = wc + (int64_t)expert * K * (N / 2);
  const uint8_t* wse = ws + (int64_t)expert * K * (N / 16);
  // A, register path: thread t loads tile row t / 2, k 32 (t % 2) .. + 31
  // (four 16-byte pieces)
  const int ar = tid >> 1, ah = tid & 1;
  const int64_t arow = arow_s[ar];
  // A, DMA path: load j of wave w fills tile rows 32 w + 8 j .. + 7 (1 KB);
  // lane l writes slot l % 8 of row 32 w + 8 j + l / 8, i.e. fetches the row's
  // k chunk (l % 8) ^ swz(row); rows past the count read zeros
  auto swz = [](int r) { return (r & 7) ^ ((r >> 3) & 1); };
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(x, (uint64_t)x_rows * K * sizeof(T));
  uint32_t a_off[4] = {0u, 0u, 0u, 0u};
  int a_chunk[4] = {0, 0, 0, 0};
  if constexpr (DMA) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 32 * wave + 8 * j + (lane >> 3);
      a_chunk[j] = (lane & 7) ^ swz(r);
      const int64_t xr = arow_s[r];
      a_off[j] = xr >= 0 ? (uint32_t)((xr * K + 8 * a_chunk[j]) * (int64_t)sizeof(T)) : kGxOutside;
    }
  }
  // B: thread t decodes weight rows k0 + 4 (t / 16) .. + 3, columns
  // bn + 8 (t % 16) .. + 7 (whole 8-column groups: n is a multiple of 16)
  const int bk = 4 * (tid >> 4), bc = tid & 15;
  const int bcol = bn + 8 * bc;
  // LDS slot of B element (n, k): 16-byte chunk k / 8 of row n in slot
  // (k / 8) ^ ((n / 16) % 8), so that the decode's writes (rows n = 8 c + i
  // across the threads' c) spread over the banks
  auto lb_at = [](int n, int k) { return n * kPitch + (((k >> 3) ^ ((n >> 4) & 7)) << 3) + (k & 7); };

  // the next step's raw operands, fetched before this step's MFMAs
  u32x4 ra[4];
  uint32_t rcode[4];
  uint32_t rscale[4];
  auto fetch = [&](int k0, int stage) {
    if constexpr (DMA) {
      T* const dst = la + stage * kTT * kTK;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = k0 + 8 * a_chunk[j] < K;  // k % 8 == 0: a chunk is whole or past the end
        gx_fetch16(rs_x, dst + (32 * wave + 8 * j) * kTK,
                   in ? a_off[j] + (uint32_t)(k0 * (int)sizeof(T)) : kGxOutside);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int k = k0 + 32 * ah + 8 * h;
        ra[h] = u32x4{0u, 0u, 0u, 0u};
        if (arow >= 0 && k < K)
          ra[h] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(x) + arow * K + k);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = k0 + bk + r;
      rcode[r] = 0u;
      rscale[r] = 0u;
      if (k < K && bcol < N) {
        rcode[r] = *reinterpret_cast<const uint32_t*>(wce + (int64_t)k * (N / 2) + bcol / 2);
        rscale[r] = wse[(int64_t)k * (N / 16) + bcol / 16];
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  fetch(0, 0);
  int stage = 0;
  for (int k0 = 0; k0 < K; k0 += kTK, stage ^= 1) {
    // stage this step: A as loaded, B decoded (zeros past k or n decode to 0)
    if constexpr (!DMA) {
#pragma unroll
      for (int h = 0; h < 4; ++h) *reinterpret_cast<u32x4*>(&la[ar * kPitch + 32 * ah + 8 * h]) = ra[h];
    }
    {
      typedef T T4 __attribute__((ext_vector_type(4)));
      T4 col[8];  // column i: rows bk .. bk + 3
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float se;
        {
#pragma clang fp contract(off)
          se = e4m3_decode(rscale[r]) * dec_w;
        }
        float q[8];
        e2m1_decode8_f32(rcode[r], q);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float v;
          {
#pragma clang fp contract(off)
            v = q[i] * se;
          }
          col[i][r] = from_f32<DT>(v);
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<T4*>(&lb[lb_at(8 * bc + i, bk)]) = col[i];
    }
    if constexpr (DMA) __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): this step's A stage landed
    __syncthreads();
    if (k0 + kTK < K) fetch(k0 + kTK, stage ^ 1);
    const T* const las = DMA ? la + stage * kTT * kTK : la;
#pragma unroll
    for (int u = 0; u < kTK / 16; ++u) {  // 16-wide k sub-steps
      V8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tr = 64 * wm + 32 * i + (lane & 31), q = 2 * u + (lane >> 5);  // row, k chunk
        a[i] = DMA ? *reinterpret_cast<const V8*>(&las[tr * kTK + ((q ^ swz(tr)) << 3)])
                   : *reinterpret_cast<const V8*>(&las[tr * kPitch + 8 * q]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = 64 * wn + 32 * j + (lane & 31);
        b[j] = *reinterpret_cast<const V8*>(&lb[lb_at(n, 16 * u + 8 * (lane >> 5))]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = MfmaT<DT>::run(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  // acc[i][j][v]: tile row 64 wm + 32 i + 8 (v / 4) + 4 (lane / 32) + v % 4,
  // column 64 wn + 32 j + lane % 32
  T* O = reinterpret_cast<T*>(out);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tr = 64 * wm + 32 * i + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
      const int orow = orow_s[tr];
      if (orow < 0) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = bn + 64 * wn + 32 * j + (lane & 31);
        if (col < N) O[(int64_t)orow * N + col] = from_f32<DT>(acc[i][j][v]);
      }
    }
}

}  // namespace

hipError_t launch_sorted_route(const int32_t* rhs, int64_t pairs, int64_t mr, int64_t e,
                               int32_t* offsets, int32_t* perm, void* zero_out, int64_t row_bytes,
                               hipStream_t s) {
  const int64_t rows = pairs * mr;
  const int64_t work = rows > e + 1 ? rows : e + 1;
  int blocks = (int)((work + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  sorted_route_kernel<<<blocks, 256, 0, s>>>(rhs, (int)pairs, (int)mr, (int)e, offsets, perm,
                                             reinterpret_cast<uint8_t*>(zero_out), row_bytes);
  return hipGetLastError();
}

hipError_t launch_amap(const int32_t* perm, const int32_t* lhs, int64_t rows, int64_t mr, int32_t* amap,
                       hipStream_t s) {
  if (rows == 0) return hipSuccess;
  int blocks = (int)((rows + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  amap_kernel<<<blocks, 256, 0, s>>>(perm, lhs, (int)rows, (int)mr, amap);
  return hipGetLastError();
}

hipError_t launch_gather_gemm_t(const void* x, int dt, const uint8_t* wc, const uint8_t* ws,
                                const float* gw, const int32_t* offsets, const int32_t* perm,
                                int64_t x_rows, int64_t rows, int64_t top_k, const int32_t* amap,
                                int64_t e, int64_t n, int64_t k, void* out, hipStream_t s) {
  if (dt == kF32)
    return launch_gather_gemm_t_f32(reinterpret_cast<const float*>(x), wc, ws, gw, offsets, perm, rows,
                                    top_k, amap, e, n, k, reinterpret_cast<float*>(out), s);
  const int64_t mt = (rows + kTT - 1) / kTT + e;
  const int64_t blocks = mt * ((n + kTT - 1) / kTT);
  // the DMA path's 32-bit offsets: x below 2 GB, k well below 2^31
  const bool dma = (uint64_t)x_rows * (uint64_t)k * 2u < 0x7F000000ull && k <= 65536;
#define NVFP4_GT(D, M)                                                                             \
  gather_t_kernel<D, M><<<(int)blocks, 256, 0, s>>>(x, x_rows, (int)k, wc, ws, gw, (int)n, out, offsets, \
                                                    perm, (int)top_k, (int)e, amap)
  if (dt == kF16) {
    if (dma) NVFP4_GT(kF16, true); else NVFP4_GT(kF16, false);
  } else {
    if (dma) NVFP4_GT(kBF16, true); else NVFP4_GT(kBF16, false);
  }
#undef NVFP4_GT
  return hipGetLastError();
}

}  // namespace nvfp4
