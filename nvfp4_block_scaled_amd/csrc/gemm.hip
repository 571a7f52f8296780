// gemm.hip -- the M > 1 NVFP4 contractions for gfx950:
//   qqmm        out[m, n]    = T( sum_k x_hat[m, k] * w[n, k] )
//   gather_qmm  out[t, j, n] = T( sum_k x[t, k] * w_e[n, k] ),  e = idx[t, j]
// with w decoded with its global scale on every block scale ("mlx 0.30.7.2 ->
// 0.30.7.6" diff page 8, qqmm and page 7, QQMatmul::eval_gpu; "[Metal]
// global scale for qmm" PR 4458, statement: the global factor sits inside
// the dequantization, per expert for gather_qmm).  gather_qmm also takes
// weights in the mx modes (diff page 8, fp_dequantize: groups of 32, e2m1 or
// e4m3 codes, E8M0 scales 2^(s - 127), no global scale); the kernels'
// weight-format parameter WF selects NVFP4 (kWfNv), mxfp4 (kWfMx4) or mxfp8
// (kWfMx8).
//
// Three kernels, by operand type and shape:
//   * mfma_gemm_fast_kernel / mfma_gemm_fast2_kernel (16-bit x, k % 64 == 0,
//     n % 4 == 0): the matrix-core path on v_mfma_f32_32x32x16 with the
//     weights decoded in registers, A staged through LDS; it reads the weight
//     either row-major or in the packed layout of mfma_pack_kernel (details
//     at the kernel body);
//     (mfma_gemm_mx4_kernel / mfma_gemm_mx4_2_kernel run the same body on
//     row-major mxfp4 weights);
//   * mfma_gemm_kernel (16-bit x, any k % 16 == 0): the general matrix-core
//     path on v_mfma_f32_16x16x32, 256 x 256 x 64 tiles with both A and the
//     decoded weight tile (written by the VALU) in double-buffered LDS;
//   * f32_gemm_kernel (float32 x): an LDS-tiled FMA kernel over float32
//     decoded weights.
// The routing of gather_qmm (moe_route_kernel) is at the end of the file.
#include <type_traits>

#include "nvfp4_device.h"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGemmThreads = 256;
constexpr int kTileElems = BM * BK;  // 16-bit elements per LDS tile

// weight formats: NVFP4 (e2m1, e4m3 scale per 16, global scale), mxfp4
// (e2m1, E8M0 scale per 32), mxfp8 (e4m3, E8M0 scale per 32)
constexpr int kWfNv = 0, kWfMx4 = 4, kWfMx8 = 8;
template <int WF> constexpr int64_t wf_code_bytes(int64_t k) { return WF == kWfMx8 ? k : k / 2; }
template <int WF> constexpr int64_t wf_scale_bytes(int64_t k) { return WF == kWfNv ? k / 16 : k / 32; }

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

// Decode 8 e4m3 codes (lo: elements 0..3, hi: 4..7, byte i = element i) with
// the block scale into T.
template <int DT>
__device__ __forceinline__ typename Mfma<DT>::V8 decode8_fp8(uint32_t lo, uint32_t hi, float se) {
  const float v[8] = {e4m3_decode_byte<0>(lo), e4m3_decode_byte<1>(lo), e4m3_decode_byte<2>(lo),
                      e4m3_decode_byte<3>(lo), e4m3_decode_byte<0>(hi), e4m3_decode_byte<1>(hi),
                      e4m3_decode_byte<2>(hi), e4m3_decode_byte<3>(hi)};
  typename Mfma<DT>::V8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma clang fp contract(off)
    o[i] = from_f32<DT>(v[i] * se);
  }
  return o;
}

// ------------------------------------------------------------------ general path (k % 16 == 0)
//
// Workgroup tile 256 x 256 x 64, four waves in a 2 x 2 grid, each a 128 x 128
// block of 8 x 8 v_mfma_f32_16x16x32 tiles with float32 accumulators.  A is
// copied to LDS as is; the weight tile is read as codes + scales, decoded by
// the VALU to T with e4m3(s) * g/2688 and written to LDS, so every weight
// element is decoded once per workgroup.  Both LDS tiles are double-buffered;
// LDS rows of 64 elements have their 16-byte chunks XOR-swizzled by row; the
// MFMA takes the weight fragment first, so each lane ends with 4 consecutive
// output columns of one row.  Partial k-steps load group by group.  The mx
// formats (WF) load a whole group of 32 per thread half and decode it with
// its E8M0 scale; their k is a multiple of 32, so a group is either whole or
// past the end.
template <int DT, bool GATHER, int WF = kWfNv>
__global__ void __launch_bounds__(kGemmThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_gemm_kernel(const void* __restrict__ a_base, const uint8_t* __restrict__ wc,
                 const uint8_t* __restrict__ ws, const float* __restrict__ gw, int M, int N, int K,
                 void* __restrict__ out, const int32_t* __restrict__ offsets,
                 const int32_t* __restrict__ perm, int top_k, int E,
                 const int32_t* __restrict__ amap) {
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
  // (or amap[row_lo + r] when an x-row map is given) and its output row is row
  // p of out viewed as [t * top_k, n].
  // A chunk q = tid + 256 i (i < 8): tile row (tid >> 3) + 32 i, chunk tid & 7
  const int a_chunk = tid & 7;
  int64_t a_row[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = bm + (tid >> 3) + 32 * i;
    if (r < row_count) {
      if constexpr (GATHER) {
        int p = perm[row_lo + r];
        a_row[i] = amap ? amap[row_lo + r] : p / top_k;
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
  const int64_t kc = wf_code_bytes<WF>(K);    // code bytes per row
  const int64_t ksc = wf_scale_bytes<WF>(K);  // scale bytes per row

  u32x4 a_reg[8];
  u32x4 b_code[2];
  u32x4 b_hi[2];  // mxfp8: the second 16 code bytes of the half's group
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
    if constexpr (WF != kWfNv) {
      (void)bfull;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int g = (k0 >> 5) + b_half;  // this half's group of 32
        u32x4 c = {0, 0, 0, 0}, c2 = {0, 0, 0, 0};
        uint32_t sc = 0;
        if (b_row[i] >= 0 && 32 * g < K) {
          const uint8_t* cp = wc + b_row[i] * kc + (int64_t)g * (WF == kWfMx8 ? 32 : 16);
          c = *reinterpret_cast<const u32x4*>(cp);
          if constexpr (WF == kWfMx8) c2 = *reinterpret_cast<const u32x4*>(cp + 16);
          sc = ws[b_row[i] * ksc + g];
        }
        b_code[i] = c;
        b_hi[i] = c2;
        b_scale[i] = sc;
      }
      return;
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
      if constexpr (WF != kWfNv) {
        const float se = e8m0_value(b_scale[i]);
        const uint32_t cw[8] = {b_code[i].x, b_code[i].y, b_code[i].z, b_code[i].w,
                                b_hi[i].x,   b_hi[i].y,   b_hi[i].z,   b_hi[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          V8 v;
          if constexpr (WF == kWfMx4)
            v = decode8<DT>(cw[j], se);
          else
            v = decode8_fp8<DT>(cw[2 * j], cw[2 * j + 1], se);
          *reinterpret_cast<V8*>(lb + lds_off(r, 4 * b_half + j)) = v;
        }
        continue;
      }
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
// Workgroup tile 256 (or 128) rows x 256 columns x 64 k, four waves:
//   * the four waves split the 256 output columns (64 each) and all share the
//     256 rows of A, so every weight element is decoded exactly once per
//     workgroup, by the wave that multiplies with it, straight into the MFMA
//     operand registers -- the weights never touch LDS: per k-step each lane
//     loads 16 code bytes and one scale dword for each of its two columns,
//     two k-steps ahead of their use;
//   * the products are v_mfma_f32_32x32x16 (32 columns x 32 rows x 16 k): a
//     wave's 64 x 256 block is 2 x 8 of them per 16-k sub-step, 64 per k-step.
//     Per flop this issues half the MFMA instructions of the 16x16x32 form and
//     leaves twice the room between them for the decode, which the single
//     wave per SIMD issues in order with its MFMAs;
//   * k order inside a 64-wide k-step: MFMA lane half h (= lane / 32) at
//     sub-step u takes the 8 k from 32 h + 8 u, i.e. half u & 1 of weight
//     group 2 h + u / 2 -- so a lane's codes for the whole k-step are 16
//     consecutive bytes (groups 2h and 2h + 1), dword u feeding sub-step u; A
//     is read from LDS in the same k order;
//   * A goes through four LDS stages (four separate LDS arrays, so that the
//     compiler can tell a stage being filled from the ones being read): from
//     the middle of step i, right after the step's one barrier, every wave
//     loads its quarter of A(i + 3) from global memory straight into LDS
//     (buffer_load ... lds: no registers, no LDS store instructions), one
//     1 KB load every few MFMA pairs over the second half of the step; the
//     barrier of step i + 2 first waits for those loads.  Issued all at
//     once, the loads of every CU reach the L2 in one burst per step; spread
//     out, the same GEMM measured 4 % faster (2048 x 14336 x 4096: 196.9 ->
//     188.8 us on one machine; a fourth stage alone changed nothing).  The
//     barrier carries no memory fence, so the weight loads stay in flight
//     across it.  A
//     fragments are read three MFMA pairs ahead, running into the first
//     fragments of step i + 1, so a step starts without waiting for LDS;
//   * fragment pair q of a step (sub-step q / 8, row tile q % 8) carries one
//     dword of the decode of step i + 1's weights (two codes by
//     v_cvt_scalef32_pk_f32_fp4, two multiplies by e4m3(s) * g/2688, one
//     conversion to two 16-bit values; every eighth pair also decodes a scale);
//   * the k loop is unrolled by four steps (four A stages, two weight
//     register sets), so every stage and register set is fixed in the code;
//   * workgroups are mapped so that each of the 8 XCDs (round-robin dispatch)
//     works on its own contiguous set of weight column panels;
//   * with 128-row tiles (used up to 128 rows) every number above halves
//     except the weight work per wave, and two workgroups share a CU;
//   * the 256 accumulator registers of a wave fill the AGPR file exactly; the
//     MFMAs are written with AGPR-constrained operands so the register
//     allocator keeps every accumulator in place (left to itself it splits
//     them between the two files and moves them around every k-step).
constexpr int kAStages = 4;                // LDS stages of A
constexpr int kBLoadsPerStep = 4;          // weight loads issued per k-step and wave
constexpr int kPackCodeBlock = 1024;       // packed codes per 32-column tile and k-step
constexpr int kPackScaleBlock = 128;       // packed scales per 32-column tile and k-step

// The 32x32x16 MFMA with its accumulator pinned to AGPRs, as inline asm (the
// register allocator then keeps the 256 accumulators of a 256-row tile in
// place).  The compiler sees neither the instruction's latency nor its
// hazards: the operands are VGPRs written by LDS loads (ordered by waits) or
// by VALU code a k-step earlier, and mfma32_fence() plus the empty asm that
// ties each accumulator after it keep every read of the results behind their
// wait states.
template <int DT> struct Mfma32;
template <> struct Mfma32<kBF16> {
  static __device__ __forceinline__ void run_agpr(bf16x8 a, bf16x8 b, f32x16& c) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
};
template <> struct Mfma32<kF16> {
  static __device__ __forceinline__ void run_agpr(f16x8 a, f16x8 b, f32x16& c) {
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
};

// Wait states before the accumulators of the 32x32 MFMAs are read back.
__device__ __forceinline__ void mfma32_fence() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
  __builtin_amdgcn_sched_barrier(0);
}

// The main loop's barrier in the middle of step i: this wave's global-to-LDS
// loads of A(i + 1) have landed -- issued in step i - 2, they are older than
// the weight loads of steps i + 1 and i + 2 (kBLoadsPerStep each) and the RT
// loads of A(i + 2), which may stay in flight -- then meet the other waves.
template <int RT>
__device__ __forceinline__ void a_stage_barrier() {
  static_assert(kBLoadsPerStep == 4, "the wait counts below count 4 weight loads per step");
  static_assert(RT == 8 || RT == 4 || RT == 2, "the wait counts below count RT loads of A per step");
  if constexpr (RT == 8)
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else if constexpr (RT == 4)
    asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
}

// Raw weights of one k-step for one lane: for each of its 2 column tiles, the
// 16 code bytes of its lane half (groups 2h, 2h + 1) and the dword of the
// column's 4 scales.
struct BRaw {
  u32x4 code[2];
  uint32_t scale[2];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// RT = 32-row tiles per workgroup: 8 (256 rows, 256 accumulators per wave, one
// workgroup per CU), 4 (128 rows, 128 accumulators per wave, two workgroups
// per CU, so that each SIMD interleaves two waves' instruction streams) or 2
// (64 rows, 64 accumulators per wave: the gather's per-expert remainders).
template <int DT, bool GATHER, bool PACKED, int RT, int WF = kWfNv>
__device__ __forceinline__ void
mfma_gemm_fast_body(const void* __restrict__ a_base, int64_t a_rows,
                    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws,
                    const float* __restrict__ gw, int M, int N, int K, void* __restrict__ out,
                    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                    int top_k, int E, int tiles_m, const int32_t* __restrict__ amap, int seg) {
  static_assert(WF == kWfNv || (WF == kWfMx4 && !PACKED), "mxfp4 weights row-major only");
  using T = typename Elem<DT>::T;
  using V8 = typename Mfma<DT>::V8;
  constexpr int TM = 32 * RT;              // tile rows
  constexpr int kStage = TM * BK * 2;      // bytes of one A stage
  constexpr int NQ = 4 * RT;               // fragment pairs per k-step
  constexpr int DPQ = 32 / NQ;             // decoded dwords per fragment pair
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sa1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sa2[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sa3[kStage];
  __shared__ int out_rows[TM];
  uint8_t* const stage[kAStages] = {sa0, sa1, sa2, sa3};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---------------------------------------------------------------- tile of this workgroup
  int L = blockIdx.x;
  if ((gridDim.x & 7) == 0) L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int tile_n = L / tiles_m;
  int tile_m = L % tiles_m;
  int expert = 0, row_lo = 0, row_count = M;
  if constexpr (GATHER) {
    // seg 0: all of each expert's rows; 1: its whole 256-row tiles, plus a
    // remainder of more than 128 rows on one more (partial) 256-row tile; 2:
    // a remainder of at most 128 rows, on one 128-row or up to two 64-row tiles
    int acc_tiles = 0;
    expert = -1;
    for (int e = 0; e < E; ++e) {
      const int all = offsets[e + 1] - offsets[e];
      const int rem = all % 256;
      const int head = rem > 128 ? all : all - rem;  // the rows of seg 1
      const int lo = seg == 2 ? head : 0;
      const int cnt = seg == 1 ? head : all - lo;
      const int tiles = (cnt + TM - 1) / TM;
      if (tile_m < acc_tiles + tiles) {
        expert = e;
        tile_m -= acc_tiles;
        row_lo = offsets[e] + lo;
        row_count = cnt;
        break;
      }
      acc_tiles += tiles;
    }
    if (expert < 0) return;
  }
  const int bm = tile_m * TM;
  const int bn = tile_n * BN;
  const float dec_w = GATHER ? (gw ? gw[expert] / (kE4M3Max * kE2M1Max) : 1.0f) : global_decode(gw);

  // output row of each tile row (-1: outside the tile's row count)
  for (int r = tid; r < TM; r += kGemmThreads) {
    int o = -1;
    if (bm + r < row_count) {
      if constexpr (GATHER)
        o = perm[row_lo + bm + r];
      else
        o = bm + r;
    }
    out_rows[r] = o;
  }

  // ---------------------------------------------------------------- buffer resources / offsets
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(a_base, (uint64_t)a_rows * K * sizeof(T));
  // weights of this expert: row-major codes / scales, or the packed layout
  // (blocks of 1 KB of codes and 128 bytes of scales per 32-column tile and
  // k-step, see mfma_pack_kernel)
  const int KT = K / BK;
  const int64_t col_tiles = (N + 31) / 32;
  const uint64_t wc_bytes = PACKED ? (uint64_t)col_tiles * KT * kPackCodeBlock : (uint64_t)N * (K / 2);
  const uint64_t ws_bytes = PACKED ? (uint64_t)col_tiles * KT * kPackScaleBlock : (uint64_t)N * wf_scale_bytes<WF>(K);
  const __amdgpu_buffer_rsrc_t rs_c = make_rsrc(wc + (int64_t)expert * wc_bytes, wc_bytes);
  const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(ws + (int64_t)expert * ws_bytes, ws_bytes);

  // A stage layout: tile row r at byte 128 r, its 16-byte k-chunk c in slot
  // c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1): any 8 consecutive rows,
  // and each parity class of any 16 consecutive rows, put a given k-chunk in
  // distinct slots, so the fragment reads (16 rows, one chunk per lane half)
  // are free of bank conflicts whether a bank row spans one 128-byte tile row
  // or two.  Wave w fills rows 8 RT w .. 8 RT w + 8 RT - 1 with RT loads of
  // 1 KB: load j, lane l writes slot l % 8 of row 8 RT w + 8 j + l / 8, i.e.
  // fetches k-chunk (l % 8) ^ swz(row) of that row.
  auto swz = [](int r) { return (r & 7) ^ ((r >> 3) & 1); };
  uint32_t a_off[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    const int r = 8 * RT * wave + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    const int rr = (bm + r < row_count) ? r : 0;  // rows past the count re-read row 0
    int64_t arow;
    if constexpr (GATHER)
      arow = amap ? amap[row_lo + bm + rr] : perm[row_lo + bm + rr] / top_k;
    else
      arow = bm + rr;
    a_off[j] = (uint32_t)((arow * K + c * 8) * (int64_t)sizeof(T));
  }
  const int fr = lane & 31;  // MFMA row of A / column of B inside a 32-wide tile
  const int fh = lane >> 5;  // lane half: k 8 fh .. 8 fh + 7 of each 16-k sub-step
  // fragment of row tile mt, sub-step u: tile row 32 mt + fr, k-chunk 4 fh + u
  int a_rd[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) a_rd[u] = fr * 128 + (((4 * fh + u) ^ swz(fr)) << 4);
  // weights: column tile t of this wave is column bn + 64 w + 32 t + fr.
  // Row-major: the lane's 16 code bytes of step kt start at col * K/2 +
  // 32 kt + 16 fh, its scale dword at col * K/16 + 4 kt (32 rows per load).
  // Packed: the 1 KB code block of (tile, kt) holds lane l's 16 bytes at
  // 16 l, the 128-byte scale block column c's dword at 4 c (one contiguous
  // run per load).  Tiles past n read as zeros (buffer range checks).
  // mxfp4 (row-major): the same code bytes; the step's two E8M0 scales, one
  // per lane half, are a 16-bit load at col * K/32 + 2 kt.
  uint32_t c_off[2], s_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if constexpr (PACKED) {
      const uint32_t tile = (uint32_t)((bn + wave * 64 + t * 32) / 32);
      c_off[t] = tile * (uint32_t)KT * kPackCodeBlock + lane * 16;
      s_off[t] = tile * (uint32_t)KT * kPackScaleBlock + fr * 4;
    } else {
      const int col = min(bn + wave * 64 + t * 32 + fr, N - 1);
      c_off[t] = (uint32_t)col * (uint32_t)(K / 2) + fh * 16;
      s_off[t] = (uint32_t)col * (uint32_t)wf_scale_bytes<WF>(K);
    }
  }
  const int c_step = PACKED ? kPackCodeBlock : BK / 2;    // code bytes per k-step
  const int s_step = PACKED ? kPackScaleBlock : (int)wf_scale_bytes<WF>(BK);  // scale bytes per k-step

  // load j (1 KB) of this wave's quarter of A(kt) into stage si, straight
  // from global memory
  auto load_a_one = [&](int kt, int si, int j) {
    const int so = kt * BK * (int)sizeof(T);
    uint8_t* dst = stage[si] + wave * (kStage / 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_ptr_t)(dst + j * 1024), 16, a_off[j], so, 0, 0);
  };
  auto load_a = [&](int kt, int si) {
#pragma unroll
    for (int j = 0; j < RT; ++j) load_a_one(kt, si, j);
  };
  auto load_b_code = [&](int kt, BRaw& b, int t) {
    b.code[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_c, c_off[t], kt * c_step, 0));
  };
  auto load_b_scale = [&](int kt, BRaw& b, int t) {
    if constexpr (WF == kWfMx4)
      b.scale[t] = __builtin_amdgcn_raw_buffer_load_b16(rs_s, s_off[t], kt * s_step, 0);
    else
      b.scale[t] = __builtin_amdgcn_raw_buffer_load_b32(rs_s, s_off[t], kt * s_step, 0);
  };
  auto load_b = [&](int kt, BRaw& b) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      load_b_code(kt, b, t);
      load_b_scale(kt, b, t);
    }
  };
  // effective scale of group 2 fh + gi (gi = 0, 1) of column tile t (mxfp4:
  // of group fh, whatever gi)
  auto scale_of = [&](const BRaw& b, int t, int gi) -> float {
    if constexpr (WF == kWfMx4) return e8m0_value((b.scale[t] >> (8 * fh)) & 0xFFu);
    float se;
    {
#pragma clang fp contract(off)
      se = e4m3_decode(b.scale[t] >> (16 * fh + 8 * gi)) * dec_w;
    }
    return se;
  };
  // dword p of the fragment of column tile t, sub-step u
  auto decode_part = [&](const BRaw& b, int t, int u, int p, float se) -> uint32_t {
    const uint32_t w = b.code[t][u];
    switch (p) {
      case 0: return decode_dword<DT, 0>(w, se);
      case 1: return decode_dword<DT, 1>(w, se);
      case 2: return decode_dword<DT, 2>(w, se);
      default: return decode_dword<DT, 3>(w, se);
    }
  };

  f32x16 acc[2][RT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][i][v] = 0.f;

  u32x4 bf[2][2][4];  // decoded weight fragments [k-step parity][column tile][sub-step]
  BRaw raw[2];        // raw weights of even / odd k-steps
  V8 ar[4];           // A fragment ring: fragment q of a step in ar[q % 4]

  // Step kt, at position P of the four-step cycle (kt = P mod 4): MFMAs on
  // A(kt) (stage P) and the fragments bf[P % 2]; over its first half loads
  // the raw weights of kt + 2 into raw[P % 2] (which held those of kt), one
  // load every NQ / 8 fragment pairs, and decodes raw[1 - P % 2] (kt + 1)
  // into bf[1 - P % 2]; in its middle, after the barrier (every wave is past
  // step kt - 1), starts loading A(kt + 3) into stage (P + 3) % 4, which held
  // A(kt - 1): one load every NQ / (2 RT) fragment pairs.  (The four weight
  // loads spread over the first half instead of issued together measured 3 %
  // faster on the 2048 x 14336 x 4096 product.)  The body
  // is straight-line: past the end of k the loads re-read the last k-step and
  // the extra work is discarded, so every wait the compiler places counts
  // exactly the loads that are in flight.
  auto step = [&](auto pos, int kt) {
    constexpr int P = decltype(pos)::value;
    constexpr int cur = P, nxt = (P + 1) % kAStages, nw = (P + 3) % kAStages, rs = P % 2;
    constexpr int kASpread = NQ / 2 / RT;  // fragment pairs between two A loads
    const int kb = min(kt + 2, KT - 1);
    const uint8_t* la = stage[cur];
    const uint8_t* ln = stage[nxt];
    const BRaw& rnext = raw[1 - rs];
    float se = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int u = q / RT, i = q % RT;
      const V8 a = ar[q & 3];
      {
        const int q3 = q + 3;
        if (q3 < NQ)
          ar[q3 & 3] = *reinterpret_cast<const V8*>(la + a_rd[q3 / RT] + (q3 % RT) * 4096);
        else
          ar[q3 & 3] = *reinterpret_cast<const V8*>(ln + a_rd[(q3 - NQ) / RT] + ((q3 - NQ) % RT) * 4096);
      }
      // decode: dword d of step kt + 1's 32 is column tile d / 16, sub-step
      // (d / 4) % 4, dword d % 4; DPQ of them ride on each fragment pair
      uint32_t part[DPQ];
#pragma unroll
      for (int j = 0; j < DPQ; ++j) {
        const int d = q * DPQ + j, dt = d >> 4, du = (d >> 2) & 3, dp = d & 3;
        if (j == 0) Mfma32<DT>::run_agpr(__builtin_bit_cast(V8, bf[rs][0][u]), a, acc[0][i]);
        if (DPQ > 1 && j == DPQ / 2) Mfma32<DT>::run_agpr(__builtin_bit_cast(V8, bf[rs][1][u]), a, acc[1][i]);
        __builtin_amdgcn_sched_barrier(0);
        if ((d & 7) == 0) se = scale_of(rnext, dt, du >> 1);
        part[j] = decode_part(rnext, dt, du, dp, se);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (DPQ == 1) Mfma32<DT>::run_agpr(__builtin_bit_cast(V8, bf[rs][1][u]), a, acc[1][i]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < DPQ; ++j) {
        const int d = q * DPQ + j;
        bf[1 - rs][d >> 4][(d >> 2) & 3][d & 3] = part[j];
      }
      if (q == 0) load_b_code(kb, raw[rs], 0);
      if (q == NQ / 8) load_b_scale(kb, raw[rs], 0);
      if (q == NQ / 4) load_b_code(kb, raw[rs], 1);
      if (q == 3 * NQ / 8) load_b_scale(kb, raw[rs], 1);
      if (q == NQ / 2 - 1) a_stage_barrier<RT>();
      if (q >= NQ / 2 - 1 && (q - (NQ / 2 - 1)) % kASpread == 0 && (q - (NQ / 2 - 1)) / kASpread < RT)
        load_a_one(min(kt + 3, KT - 1), nw, (q - (NQ / 2 - 1)) / kASpread);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---------------------------------------------------------------- prologue
  // A(0), A(1), A(2) into stages 0 to 2, raw weights of steps 0 and 1, step
  // 0's fragments decoded, the first three A fragments read.
  load_a(0, 0);
  load_a(min(1, KT - 1), 1);
  load_a(min(2, KT - 1), 2);
  load_b(0, raw[0]);
  load_b(min(1, KT - 1), raw[1]);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float se = scale_of(raw[0], t, u >> 1);
#pragma unroll
      for (int p = 0; p < 4; ++p) bf[0][t][u][p] = decode_part(raw[0], t, u, p, se);
    }
  // every load of the prologue (and every scalar load) has landed, then meet
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 3; ++q) ar[q] = *reinterpret_cast<const V8*>(sa0 + a_rd[q / RT] + (q % RT) * 4096);

  // ---------------------------------------------------------------- main loop
  // the zeroed accumulators are materialised in AGPRs before the fence
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < RT; ++i) asm volatile("" : "+a"(acc[t][i]));
  mfma32_fence();
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  int kt = 0;
  for (; kt + 4 <= KT; kt += 4) {
    step(P0{}, kt);
    step(P1{}, kt + 1);
    step(P2{}, kt + 2);
    step(P3{}, kt + 3);
  }
  if (kt < KT) step(P0{}, kt);
  if (kt + 1 < KT) step(P1{}, kt + 1);
  if (kt + 2 < KT) step(P2{}, kt + 2);
  mfma32_fence();
  // the fence carries no data dependence on the accumulators, so the
  // compiler may place their reads (copies to VGPRs) ahead of it; tying
  // each one to an asm after the fence keeps every read behind the wait
  // states (64-row tiles: with few registers in use the copies went to the
  // top of the epilogue, straight after the last MFMAs of a k-step count
  // of 3 mod 4, and read two accumulators before those MFMAs wrote them)
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < RT; ++i) asm volatile("" : "+a"(acc[t][i]));

  // ---------------------------------------------------------------- epilogue
  // acc[t][i][v]: tile row 32 i + fr, tile column 64 w + 32 t + 8 (v / 4) +
  // 4 fh + v % 4.  Each lane holds 4 consecutive columns of 16 rows, so the
  // block goes through LDS (the A stages are free now) to leave as whole
  // rows: per half of the tile's rows, wave w writes its 16 RT x 64 block
  // (16-byte chunk c of row r in slot c ^ (r & 7)) and reads it back with
  // lane l on row 8 j + l / 8, chunk l % 8, so that one store instruction
  // writes 8 full 128-byte row segments.
  // this wave's discarded last stage load has landed and every wave is done
  // with the stages
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  lds_barrier();
  T* O = reinterpret_cast<T*>(out);
  uint8_t* const eb = ((wave >> 1) ? sa1 : sa0) + (wave & 1) * (kStage / 2);
  const int col0 = bn + wave * 64;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < RT / 2; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r = 32 * i + fr, c = 4 * t + g;
          typedef T T4 __attribute__((ext_vector_type(4)));
          T4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = from_f32<DT>(acc[t][(RT / 2) * h + i][4 * g + e]);
          *reinterpret_cast<T4*>(eb + r * 128 + ((c ^ (r & 7)) << 4) + 8 * fh) = v;
        }
#pragma unroll
    for (int j = 0; j < 2 * RT; ++j) {
      const int r = 8 * j + (lane >> 3), c = lane & 7;
      const u32x4 d = *reinterpret_cast<const u32x4*>(eb + r * 128 + ((c ^ (r & 7)) << 4));
      const int orow = out_rows[(TM / 2) * h + r];
      const int col = col0 + 8 * c;
      if (orow >= 0) {
        T* op = O + (int64_t)orow * N + col;
        if (col + 8 <= N) {
          *reinterpret_cast<u32x4*>(op) = d;
        } else {
          typedef T T8 __attribute__((ext_vector_type(8)));
          const T8 e8 = __builtin_bit_cast(T8, d);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < N) op[e] = e8[e];
        }
      }
    }
  }
}

#define NVFP4_FAST_ARGS                                                                        \
  const void* __restrict__ a_base, int64_t a_rows, const uint8_t* __restrict__ wc,             \
      const uint8_t* __restrict__ ws, const float* __restrict__ gw, int M, int N, int K,       \
      void* __restrict__ out, const int32_t* __restrict__ offsets,                             \
      const int32_t* __restrict__ perm, int top_k, int E, int tiles_m,                          \
      const int32_t* __restrict__ amap, int seg
#define NVFP4_FAST_PASS a_base, a_rows, wc, ws, gw, M, N, K, out, offsets, perm, top_k, E, tiles_m, amap, seg

// 256-row tiles: one workgroup (four waves, 256 accumulators each) per CU
template <int DT, bool GATHER, bool PACKED>
__global__ void __launch_bounds__(kGemmThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_gemm_fast_kernel(NVFP4_FAST_ARGS) {
  mfma_gemm_fast_body<DT, GATHER, PACKED, 8>(NVFP4_FAST_PASS);
}

// 128-row tiles: two workgroups per CU (two waves of 128 accumulators per SIMD)
template <int DT, bool GATHER, bool PACKED>
__global__ void __launch_bounds__(kGemmThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_gemm_fast2_kernel(NVFP4_FAST_ARGS) {
  mfma_gemm_fast_body<DT, GATHER, PACKED, 4>(NVFP4_FAST_PASS);
}

// 64-row tiles: the remainders of at most 128 routed rows per expert that
// gather_qmm leaves after its 256-row tiles (a 128-row tile for a remainder
// of a few dozen rows would multiply mostly padding)
template <int DT, bool GATHER, bool PACKED>
__global__ void __launch_bounds__(kGemmThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_gemm_fast4_kernel(NVFP4_FAST_ARGS) {
  mfma_gemm_fast_body<DT, GATHER, PACKED, 2>(NVFP4_FAST_PASS);
}

// the same two tilings for gather_qmm on row-major mxfp4 weights
template <int DT>
__global__ void __launch_bounds__(kGemmThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_gemm_mx4_kernel(NVFP4_FAST_ARGS) {
  mfma_gemm_fast_body<DT, true, false, 8, kWfMx4>(NVFP4_FAST_PASS);
}
template <int DT>
__global__ void __launch_bounds__(kGemmThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
mfma_gemm_mx4_2_kernel(NVFP4_FAST_ARGS) {
  mfma_gemm_fast_body<DT, true, false, 4, kWfMx4>(NVFP4_FAST_PASS);
}

// ------------------------------------------------------------------ packed weight layout
//
// The fast path reads, per k-step, 16 code bytes and one scale dword for each
// of its columns; in the row-major layout those lie in 32 different rows per
// load instruction.  The packed layout puts them in MFMA lane order, once per
// weight: for column tile T (columns 32 T .. 32 T + 31) and k-step s (64 k),
//   codes  block (T, s) of 1 KB: bytes 16 l .. 16 l + 15 = the codes of
//          column 32 T + l % 32, groups 4 s + 2 h and 4 s + 2 h + 1
//          (h = l / 32) -- i.e. row-major bytes 32 s + 16 h .. + 15 of that row;
//   scales block (T, s) of 128 bytes: dword c = the 4 scales of column 32 T + c
//          for step s -- row-major bytes 4 s .. 4 s + 3 of that row;
// blocks ordered by T, then s; columns past the row count are zero.  Several
// experts stack as consecutive row ranges (their row count a multiple of 32).
// One thread per 16-byte code piece; threads of lanes 0..31 also move the
// scale dword of their column.
__global__ void __launch_bounds__(256)
mfma_pack_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t rows,
                 int K, uint8_t* __restrict__ pc, uint8_t* __restrict__ ps, int64_t pieces) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= pieces) return;
  const int KT = K / BK;
  const int l = (int)(i & 63);
  const int64_t blk = i >> 6;  // T * KT + s
  const int64_t T = blk / KT;
  const int st = (int)(blk - T * KT);
  const int64_t col = 32 * T + (l & 31);
  u32x4 c = {0u, 0u, 0u, 0u};
  uint32_t sc = 0u;
  if (col < rows) {
    c = *reinterpret_cast<const u32x4*>(codes + col * (K / 2) + 32 * st + 16 * (l >> 5));
    sc = *reinterpret_cast<const uint32_t*>(scales + col * (K / 16) + 4 * st);
  }
  *reinterpret_cast<u32x4*>(pc + blk * kPackCodeBlock + 16 * l) = c;
  if (l < 32) *reinterpret_cast<uint32_t*>(ps + blk * kPackScaleBlock + 4 * l) = sc;
}

// ------------------------------------------------------------------ float32 path

constexpr int FT = 64, FK = 16;

// out tile 64 x 64, 256 threads with 4 x 4 outputs each; the weight tile is
// decoded to float32 e2m1(q) * (e4m3(s) * g/2688) while staged in LDS.
// TRANS: each expert's weight is [K, N] quantized along N (gather_qmm with
// transpose = False, out = x @ w): element (n, k) is row k, column n.  WF: the
// weight format (mx weights: code value times 2^(s - 127), [N, K] only).
template <bool GATHER, bool TRANS = false, int WF = kWfNv>
__global__ void __launch_bounds__(256)
f32_gemm_kernel(const float* __restrict__ A, const uint8_t* __restrict__ wc,
                const uint8_t* __restrict__ ws, const float* __restrict__ gw, int M, int N, int K,
                float* __restrict__ out, const int32_t* __restrict__ offsets,
                const int32_t* __restrict__ perm, int top_k, int E,
                const int32_t* __restrict__ amap) {
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
        arow[tid] = amap ? amap[row_lo + r] : p / top_k;
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
      if constexpr (WF != kWfNv) {
        static_assert(!TRANS, "mx weights are [N, K]");
        if (n < N && k < K) {
          const int64_t row = wbase + n;
          float cv;
          if constexpr (WF == kWfMx4) {
            const uint32_t byte = wc[row * (K >> 1) + (k >> 1)];
            cv = e2m1_decode((k & 1) ? (byte >> 4) : (byte & 15u));
          } else {
            cv = e4m3_decode(wc[row * K + k]);
          }
          wv = cv * e8m0_value(ws[row * (K >> 5) + (k >> 5)]);
        }
      } else if (n < N && k < K) {
        uint32_t code, sbyte;
        if constexpr (TRANS) {
          const int64_t row = (int64_t)expert * K + k;
          const uint32_t byte = wc[row * (N >> 1) + (n >> 1)];
          code = (n & 1) ? (byte >> 4) : (byte & 15u);
          sbyte = ws[row * (N >> 4) + (n >> 4)];
        } else {
          const int64_t row = wbase + n;
          const uint32_t byte = wc[row * (K >> 1) + (k >> 1)];
          code = (k & 1) ? (byte >> 4) : (byte & 15u);
          sbyte = ws[row * (K >> 4) + (k >> 4)];
        }
        float se;
        {
#pragma clang fp contract(off)
          se = e4m3_decode(sbyte) * dec_w;
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
//
// Routing sorts the routed rows by expert, stably (ascending row id within an
// expert): row q of the entries * mr rows goes to expert idx[q / mr].  It is a
// counting sort over chunks of rows (a multiple of 1024 rows, at most
// kRouteMaxChunks chunks), in three launches or, for small count tables, two:
//   count    one workgroup per chunk: the chunk's per-expert counts;
//   scan     one workgroup: offsets[x], the exclusive prefix of the experts'
//            totals, and each chunk's first slot per expert (for small count
//            tables every scatter workgroup does this itself);
//   scatter  one workgroup per chunk, in steps of 1024 rows: a row's slot is
//            its expert's running slot, plus the same-expert rows of earlier
//            waves of the step, plus its rank among the same-expert lanes of
//            its wave.
// A row whose expert lies outside [0, E) goes to a last bucket: perm[offsets[E]
// .. rows) holds those rows in ascending order, and when an output is given
// the scatter writes zeros to their output rows (no product touches them).

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteMaxE = 1024;
constexpr int kRouteMaxChunks = 256;

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

// the bucket of routed row q: its expert, or E when that lies outside [0, E)
__device__ __forceinline__ int route_bucket(const int32_t* __restrict__ idx, int q, int mr, int E) {
  const int x = idx[q / mr];
  return (x >= 0 && x < E) ? x : E;
}

__global__ void __launch_bounds__(kRouteThreads)
route_count_kernel(const int32_t* __restrict__ idx, int rows, int mr, int E, int chunk,
                   int32_t* __restrict__ counts) {
  __shared__ int hist[kRouteMaxE + 1];
  const int tid = threadIdx.x;
  for (int x = tid; x <= E; x += kRouteThreads) hist[x] = 0;
  __syncthreads();
  const int q0 = blockIdx.x * chunk;
  const int q1 = min(rows, q0 + chunk);
  for (int qb = q0; qb < q1; qb += kRouteThreads) {
    const int q = qb + tid;
    const bool have = q < q1;
    const int b = have ? route_bucket(idx, q, mr, E) : -1;
    match_experts(b, have, [&](int le, int cnt) { atomicAdd(&hist[le], cnt); });
  }
  __syncthreads();
  for (int x = tid; x <= E; x += kRouteThreads) counts[blockIdx.x * (E + 1) + x] = hist[x];
}

// Exclusive prefix over buckets 0 .. E, in place: tot[x] (the buckets'
// totals, zero past E) becomes the first slot of bucket x.  Thread t holds
// buckets 2t and 2t + 1; part is scratch.  Every thread of the workgroup calls
// it.
__device__ __forceinline__ void route_bucket_prefix(int* tot, int* part) {
  const int tid = threadIdx.x;
  const int mine = tot[2 * tid] + tot[2 * tid + 1];
  part[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kRouteThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const int excl = part[tid] - mine;
  const int o0 = excl, o1 = excl + tot[2 * tid];
  __syncthreads();
  tot[2 * tid] = o0;
  tot[2 * tid + 1] = o1;
  __syncthreads();
}

// counts [chunks][E + 1] in, each chunk's first slot per bucket out
__global__ void __launch_bounds__(kRouteThreads)
route_scan_kernel(int32_t* __restrict__ counts, int chunks, int E, int32_t* __restrict__ offsets) {
  __shared__ int tot[2 * kRouteThreads];
  __shared__ int part[kRouteThreads];
  const int tid = threadIdx.x;
  for (int x = tid; x < 2 * kRouteThreads; x += kRouteThreads) {
    int run = 0;
    if (x <= E) {
      for (int c = 0; c < chunks; ++c) {
        const int v = counts[c * (E + 1) + x];
        counts[c * (E + 1) + x] = run;  // the chunk's first slot, relative to the bucket
        run += v;
      }
    }
    tot[x] = run;
  }
  __syncthreads();
  route_bucket_prefix(tot, part);
  for (int x = tid; x <= E; x += kRouteThreads) offsets[x] = tot[x];
  for (int i = tid; i < chunks * (E + 1); i += kRouteThreads) counts[i] += tot[i % (E + 1)];
}

// The chunk's rows in steps of 1024: a row's slot is its bucket's running
// slot base[b], plus the same-bucket rows of earlier waves of the step, plus
// its rank among the same-bucket lanes of its wave.
__device__ __forceinline__ void route_scatter_chunk(const int32_t* __restrict__ idx, int rows, int mr,
                                                    int E, int chunk, int* base, int* wcnt,
                                                    int32_t* __restrict__ perm,
                                                    uint8_t* __restrict__ zero_out, int64_t row_bytes) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q0 = blockIdx.x * chunk;
  const int q1 = min(rows, q0 + chunk);
  for (int qb = q0; qb < q1; qb += kRouteThreads) {
    for (int i = tid; i < kRouteWaves * (E + 1); i += kRouteThreads) wcnt[i] = 0;
    __syncthreads();
    const int q = qb + tid;
    const bool have = q < q1;
    const int b = have ? route_bucket(idx, q, mr, E) : -1;
    const uint64_t same =
        match_experts(b, have, [&](int le, int cnt) { wcnt[wave * (E + 1) + le] = cnt; });
    __syncthreads();
    if (have) {
      int pos = base[b] + __builtin_popcountll(same & ((1ull << lane) - 1ull));
      for (int w = 0; w < wave; ++w) pos += wcnt[w * (E + 1) + b];
      perm[pos] = q;
    }
    if (zero_out) {
      uint64_t bad = __ballot(have && b == E);
      while (bad) {
        const int l = __builtin_ctzll(bad);
        zero_row_wave(zero_out, (int64_t)(qb + wave * 64 + l), row_bytes);
        bad &= bad - 1ull;
      }
    }
    __syncthreads();
    for (int x = tid; x <= E; x += kRouteThreads) {
      int add = 0;
      for (int w = 0; w < kRouteWaves; ++w) add += wcnt[w * (E + 1) + x];
      base[x] += add;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kRouteThreads)
route_scatter_kernel(const int32_t* __restrict__ idx, int rows, int mr, int E, int chunk,
                     const int32_t* __restrict__ starts, int32_t* __restrict__ perm,
                     uint8_t* __restrict__ zero_out, int64_t row_bytes) {
  __shared__ int base[kRouteMaxE + 1];
  __shared__ int wcnt[kRouteWaves * (kRouteMaxE + 1)];
  for (int x = threadIdx.x; x <= E; x += kRouteThreads) base[x] = starts[blockIdx.x * (E + 1) + x];
  route_scatter_chunk(idx, rows, mr, E, chunk, base, wcnt, perm, zero_out, row_bytes);
}

// The scan folded into the scatter, for small count tables (chunks x (E + 1)
// at most kRouteFusedCounts): every workgroup reads the whole table, takes
// the buckets' totals and its chunk's share of the rows before it, and runs
// the bucket prefix itself; workgroup 0 writes offsets.  Same slots as the
// scan kernel, one launch fewer.
constexpr int kRouteFusedCounts = 4096;

__global__ void __launch_bounds__(kRouteThreads)
route_scan_scatter_kernel(const int32_t* __restrict__ idx, int rows, int mr, int E, int chunk,
                          const int32_t* __restrict__ counts, int chunks,
                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                          uint8_t* __restrict__ zero_out, int64_t row_bytes) {
  __shared__ int tot[2 * kRouteThreads];
  __shared__ int part[kRouteThreads];
  __shared__ int base[kRouteMaxE + 1];
  __shared__ int wcnt[kRouteWaves * (kRouteMaxE + 1)];
  const int tid = threadIdx.x;
  for (int x = tid; x < 2 * kRouteThreads; x += kRouteThreads) {
    int run = 0, before = 0;
    if (x <= E) {
      for (int c = 0; c < chunks; ++c) {
        if (c == (int)blockIdx.x) before = run;
        run += counts[c * (E + 1) + x];
      }
      base[x] = before;
    }
    tot[x] = run;
  }
  __syncthreads();
  route_bucket_prefix(tot, part);
  for (int x = tid; x <= E; x += kRouteThreads) {
    base[x] += tot[x];
    if (blockIdx.x == 0) offsets[x] = tot[x];
  }
  route_scatter_chunk(idx, rows, mr, E, chunk, base, wcnt, perm, zero_out, row_bytes);
}

int64_t route_chunk_rows(int64_t rows) {
  int64_t c = (rows + kRouteMaxChunks - 1) / kRouteMaxChunks;
  c = (c + kRouteThreads - 1) / kRouteThreads * kRouteThreads;
  return c < kRouteThreads ? kRouteThreads : c;
}

}  // namespace

// ------------------------------------------------------------------ launchers

template <bool GATHER, bool PACKED, int RT, int WF = kWfNv>
hipError_t launch_fast_rt(int dt, const void* a, int64_t a_rows, const uint8_t* wc, const uint8_t* ws,
                          const float* gw, int64_t rows, int64_t n, int64_t k, void* out,
                          const int32_t* offsets, const int32_t* perm, int64_t top_k, int64_t e,
                          const int32_t* amap, int seg, hipStream_t s_stream) {
  constexpr int TM = 32 * RT;
  // tile rows: an upper bound for the gather (per-expert counts live on the
  // device; surplus workgroups return at once)
  const int64_t tiles_m = seg == 1 ? rows / 256 + std::min<int64_t>(e, rows / 129)
                        : seg == 2 ? e * ((128 + TM - 1) / TM)
                                   : (rows + TM - 1) / TM + (GATHER ? e : 0);
  const int64_t blocks = tiles_m * ((n + BN - 1) / BN);
#define NVFP4_LAUNCH(KER, D)                                                                     \
  KER<D, GATHER, PACKED><<<(int)blocks, kGemmThreads, 0, s_stream>>>(                              \
      a, a_rows, wc, ws, gw, (int)rows, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e,    \
      (int)tiles_m, amap, seg)
#define NVFP4_LAUNCH_MX(KER, D)                                                                  \
  KER<D><<<(int)blocks, kGemmThreads, 0, s_stream>>>(                                              \
      a, a_rows, wc, ws, gw, (int)rows, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e,    \
      (int)tiles_m, amap, seg)
  if constexpr (WF == kWfMx4) {
    static_assert(GATHER && !PACKED, "mxfp4 weights: gather_qmm, row-major");
    if constexpr (RT == 8) {
      if (dt == kF16)
        NVFP4_LAUNCH_MX(mfma_gemm_mx4_kernel, kF16);
      else
        NVFP4_LAUNCH_MX(mfma_gemm_mx4_kernel, kBF16);
    } else {
      if (dt == kF16)
        NVFP4_LAUNCH_MX(mfma_gemm_mx4_2_kernel, kF16);
      else
        NVFP4_LAUNCH_MX(mfma_gemm_mx4_2_kernel, kBF16);
    }
  } else if constexpr (RT == 8) {
    if (dt == kF16)
      NVFP4_LAUNCH(mfma_gemm_fast_kernel, kF16);
    else
      NVFP4_LAUNCH(mfma_gemm_fast_kernel, kBF16);
  } else if constexpr (RT == 2) {
    if (dt == kF16)
      NVFP4_LAUNCH(mfma_gemm_fast4_kernel, kF16);
    else
      NVFP4_LAUNCH(mfma_gemm_fast4_kernel, kBF16);
  } else {
    if (dt == kF16)
      NVFP4_LAUNCH(mfma_gemm_fast2_kernel, kF16);
    else
      NVFP4_LAUNCH(mfma_gemm_fast2_kernel, kBF16);
  }
#undef NVFP4_LAUNCH
#undef NVFP4_LAUNCH_MX
  return hipGetLastError();
}

template <bool GATHER, bool PACKED, int WF = kWfNv>
hipError_t launch_fast(int dt, const void* a, int64_t a_rows, const uint8_t* wc, const uint8_t* ws,
                       const float* gw, int64_t rows, int64_t n, int64_t k, void* out,
                       const int32_t* offsets, const int32_t* perm, int64_t top_k, int64_t e,
                       const int32_t* amap, hipStream_t s) {
  // up to 128 rows (routed pairs) the 128-row tiles skip the half of a
  // 256-row tile that would multiply padding; above that the 256-row tiles
  // are faster (each weight element is decoded for twice as many rows),
  // unless they are too few to give every CU a tile (a long k and few output
  // columns, as in the backward's dx): then the 128-row tiles double the
  // tile count.  Both compute every output element in the same order.
  const int64_t tiles8 = ((rows + 255) / 256) * ((n + BN - 1) / BN);
  if (rows <= 128 || (!GATHER && tiles8 < device_cu_count()))
    return launch_fast_rt<GATHER, PACKED, 4, WF>(dt, a, a_rows, wc, ws, gw, rows, n, k, out, offsets,
                                                 perm, top_k, e, amap, 0, s);
  if constexpr (GATHER) {
    // each expert's whole 256-row tiles and any remainder of more than 128
    // rows on 256-row tiles, then the remainders of at most 128 rows on
    // 128-row tiles: a nearly empty 256-row tile per expert would cost a
    // whole tile, while a remainder above 128 rows costs the same MFMA work
    // either way and, in the first launch, fills the last round of tiles
    // (same summation order for every output either way)
    // (NVFP4 weights: the remainders on 64-row tiles, one or two per expert;
    // at the MoE shape they are a few dozen rows for some experts and the
    // 128-row tiles left this launch mostly multiplying padding)
    if (hipError_t err = launch_fast_rt<GATHER, PACKED, 8, WF>(dt, a, a_rows, wc, ws, gw, rows, n, k,
                                                               out, offsets, perm, top_k, e, amap, 1, s))
      return err;
    constexpr int kTailRT = WF == kWfNv ? 2 : 4;
    return launch_fast_rt<GATHER, PACKED, kTailRT, WF>(dt, a, a_rows, wc, ws, gw, rows, n, k, out,
                                                       offsets, perm, top_k, e, amap, 2, s);
  }
  return launch_fast_rt<GATHER, PACKED, 8, WF>(dt, a, a_rows, wc, ws, gw, rows, n, k, out, offsets, perm,
                                           top_k, e, amap, 0, s);
}

hipError_t launch_mfma_pack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                            uint8_t* pc, uint8_t* ps, hipStream_t s) {
  const int64_t pieces = ((rows + 31) / 32) * (k / BK) * 64;
  if (pieces == 0) return hipSuccess;
  mfma_pack_kernel<<<(int)((pieces + 255) / 256), 256, 0, s>>>(codes, scales, rows, (int)k, pc, ps, pieces);
  return hipGetLastError();
}

hipError_t launch_qqmm_gemm_packed(const void* xhat, int dt, const uint8_t* pc, const uint8_t* ps,
                                   const float* gw, int64_t m, int64_t n, int64_t k, void* out,
                                   hipStream_t s) {
  return launch_fast<false, true>(dt, xhat, m, pc, ps, gw, m, n, k, out, nullptr, nullptr, 1, 1,
                                  nullptr, s);
}

hipError_t launch_gather_gemm_packed(const void* x, int dt, const uint8_t* pc, const uint8_t* ps,
                                     const float* gw, const int32_t* offsets, const int32_t* perm,
                                     int64_t x_rows, int64_t rows, int64_t top_k, const int32_t* amap,
                                     int64_t e, int64_t n, int64_t k, void* out, hipStream_t s) {
  return launch_fast<true, true>(dt, x, x_rows, pc, ps, gw, rows, n, k, out, offsets, perm, top_k, e,
                                 amap, s);
}

hipError_t launch_qqmm_gemm(const void* xhat, int dt, const uint8_t* wc, const uint8_t* ws,
                            const float* gw, int64_t m, int64_t n, int64_t k, void* out,
                            hipStream_t s) {
  if (dt == kF32) {
    int64_t blocks = ((m + FT - 1) / FT) * ((n + FT - 1) / FT);
    f32_gemm_kernel<false><<<(int)blocks, 256, 0, s>>>(
        reinterpret_cast<const float*>(xhat), wc, ws, gw, (int)m, (int)n, (int)k,
        reinterpret_cast<float*>(out), nullptr, nullptr, 1, 1, nullptr);
    return hipGetLastError();
  }
  int64_t blocks = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  if (k % BK == 0 && n % 4 == 0)
    return launch_fast<false, false>(dt, xhat, m, wc, ws, gw, m, n, k, out, nullptr, nullptr, 1, 1,
                                     nullptr, s);
  if (dt == kF16)
    mfma_gemm_kernel<kF16, false><<<(int)blocks, kGemmThreads, 0, s>>>(
        xhat, wc, ws, gw, (int)m, (int)n, (int)k, out, nullptr, nullptr, 1, 1, nullptr);
  else
    mfma_gemm_kernel<kBF16, false><<<(int)blocks, kGemmThreads, 0, s>>>(
        xhat, wc, ws, gw, (int)m, (int)n, (int)k, out, nullptr, nullptr, 1, 1, nullptr);
  return hipGetLastError();
}

size_t route_scratch_bytes(int64_t rows, int64_t e) {
  if (rows <= 0 || e <= 0) return 0;
  const int64_t chunks = (rows + route_chunk_rows(rows) - 1) / route_chunk_rows(rows);
  return (size_t)chunks * (size_t)(e + 1) * sizeof(int32_t);
}

hipError_t launch_moe_route(const int32_t* idx, int64_t entries, int64_t rows_per_entry, int64_t e,
                            int32_t* offsets, int32_t* perm, int32_t* scratch, void* zero_out,
                            int64_t row_bytes, hipStream_t s) {
  const int64_t rows = entries * rows_per_entry;
  const int64_t chunk = route_chunk_rows(rows);
  const int chunks = (int)((rows + chunk - 1) / chunk);
  route_count_kernel<<<chunks, kRouteThreads, 0, s>>>(idx, (int)rows, (int)rows_per_entry, (int)e,
                                                      (int)chunk, scratch);
  if ((int64_t)chunks * (e + 1) <= kRouteFusedCounts) {
    route_scan_scatter_kernel<<<chunks, kRouteThreads, 0, s>>>(
        idx, (int)rows, (int)rows_per_entry, (int)e, (int)chunk, scratch, chunks, offsets, perm,
        reinterpret_cast<uint8_t*>(zero_out), row_bytes);
    return hipGetLastError();
  }
  route_scan_kernel<<<1, kRouteThreads, 0, s>>>(scratch, chunks, (int)e, offsets);
  route_scatter_kernel<<<chunks, kRouteThreads, 0, s>>>(idx, (int)rows, (int)rows_per_entry, (int)e,
                                                        (int)chunk, scratch, perm,
                                                        reinterpret_cast<uint8_t*>(zero_out), row_bytes);
  return hipGetLastError();
}

hipError_t launch_gather_gemm_t_f32(const float* x, const uint8_t* wc, const uint8_t* ws,
                                   const float* gw, const int32_t* offsets, const int32_t* perm,
                                   int64_t rows, int64_t top_k, const int32_t* amap, int64_t e,
                                   int64_t n, int64_t k, float* out, hipStream_t s) {
  const int64_t mt = (rows + FT - 1) / FT + e;
  const int64_t blocks = mt * ((n + FT - 1) / FT);
  f32_gemm_kernel<true, true><<<(int)blocks, 256, 0, s>>>(x, wc, ws, gw, (int)rows, (int)n, (int)k, out,
                                                        offsets, perm, (int)top_k, (int)e, amap);
  return hipGetLastError();
}

hipError_t launch_gather_gemm(const void* x, int dt, const uint8_t* wc, const uint8_t* ws,
                              const float* gw, const int32_t* offsets, const int32_t* perm,
                              int64_t x_rows, int64_t rows, int64_t top_k, const int32_t* amap,
                              int64_t e, int64_t n, int64_t k, void* out, hipStream_t s) {
  if (dt == kF32) {
    int64_t mt = (rows + FT - 1) / FT + e;
    int64_t blocks = mt * ((n + FT - 1) / FT);
    f32_gemm_kernel<true><<<(int)blocks, 256, 0, s>>>(
        reinterpret_cast<const float*>(x), wc, ws, gw, (int)rows, (int)n, (int)k,
        reinterpret_cast<float*>(out), offsets, perm, (int)top_k, (int)e, amap);
    return hipGetLastError();
  }
  int64_t mt = (rows + BM - 1) / BM + e;
  int64_t blocks = mt * ((n + BN - 1) / BN);
  if (k % BK == 0 && n % 4 == 0)
    return launch_fast<true, false>(dt, x, x_rows, wc, ws, gw, rows, n, k, out, offsets, perm, top_k, e,
                                    amap, s);
  if (dt == kF16)
    mfma_gemm_kernel<kF16, true><<<(int)blocks, kGemmThreads, 0, s>>>(
        x, wc, ws, gw, (int)rows, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e, amap);
  else
    mfma_gemm_kernel<kBF16, true><<<(int)blocks, kGemmThreads, 0, s>>>(
        x, wc, ws, gw, (int)rows, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e, amap);
  return hipGetLastError();
}

namespace {

template <int WF>
hipError_t launch_mx_gather_wf(const void* x, int dt, const uint8_t* wc, const uint8_t* ws,
                               const int32_t* offsets, const int32_t* perm, int64_t x_rows,
                               int64_t rows, int64_t top_k, int64_t e, int64_t n, int64_t k,
                               void* out, hipStream_t s) {
  if (dt == kF32) {
    const int64_t blocks = ((rows + FT - 1) / FT + e) * ((n + FT - 1) / FT);
    f32_gemm_kernel<true, false, WF><<<(int)blocks, 256, 0, s>>>(
        reinterpret_cast<const float*>(x), wc, ws, nullptr, (int)rows, (int)n, (int)k,
        reinterpret_cast<float*>(out), offsets, perm, (int)top_k, (int)e, nullptr);
    return hipGetLastError();
  }
  if constexpr (WF == kWfMx4) {
    if (k % BK == 0 && n % 4 == 0)
      return launch_fast<true, false, kWfMx4>(dt, x, x_rows, wc, ws, nullptr, rows, n, k, out, offsets,
                                              perm, top_k, e, nullptr, s);
  }
  const int64_t blocks = ((rows + BM - 1) / BM + e) * ((n + BN - 1) / BN);
  if (dt == kF16)
    mfma_gemm_kernel<kF16, true, WF><<<(int)blocks, kGemmThreads, 0, s>>>(
        x, wc, ws, nullptr, (int)rows, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e, nullptr);
  else
    mfma_gemm_kernel<kBF16, true, WF><<<(int)blocks, kGemmThreads, 0, s>>>(
        x, wc, ws, nullptr, (int)rows, (int)n, (int)k, out, offsets, perm, (int)top_k, (int)e, nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_gather_gemm(const void* x, int dt, int mode, const uint8_t* wc, const uint8_t* ws,
                                 const int32_t* offsets, const int32_t* perm, int64_t x_rows,
                                 int64_t rows, int64_t top_k, int64_t e, int64_t n, int64_t k,
                                 void* out, hipStream_t s) {
  if (mode == 8)
    return launch_mx_gather_wf<kWfMx8>(x, dt, wc, ws, offsets, perm, x_rows, rows, top_k, e, n, k, out, s);
  return launch_mx_gather_wf<kWfMx4>(x, dt, wc, ws, offsets, perm, x_rows, rows, top_k, e, n, k, out, s);
}

}  // namespace nvfp4
