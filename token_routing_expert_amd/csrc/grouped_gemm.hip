// Grouped SwiGLU expert MLP over ragged expert segments of packed rows.
//
// "Token permutation and grouped GEMMs" (zerotofrontier.app, "Expert
// parallelism"): one kernel receives the list of problem sizes (the expert
// segments given by offsets) and schedules the output tiles of all of them
// across the GPU in one launch -- no padding beyond the tile, nothing dropped.
// A SwiGLU expert is three d x ffn matrices, 6 d ffn FLOPs per row
// ("A worked example at DeepSeek-V3's shape").
//
// Two launches per call:
//   GEMM1  h[p, n] = SiLU(sum_k a[p,k] Wg[n,k]) * (sum_k a[p,k] Wu[n,k])
//   GEMM2  y[p, n] = sum_k h[p,k] Wd[n,k]
// Both operands are K-contiguous, so row tiles and weight tiles stage through
// LDS the same way: 128-byte K slices per row (64 bf16 or 32 fp32), stored with
// the 16-byte chunk index XOR-swizzled by the row so that the MFMA operand
// reads (32 rows, one chunk) hit distinct banks.  Each wave runs 32x32 MFMA
// blocks: v_mfma_f32_32x32x16_bf16 for bf16, four v_mfma_f32_32x32x2f32 per
// 16-byte chunk for fp32.  Accumulation is fp32.
#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16 bytes as a native vector (HIP's uint4 struct defeats register promotion
// of small arrays).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Mma;

template <>
struct Mma<true> {
  static __device__ __forceinline__ void run(const u32x4 &a, const u32x4 &b, f32x16 &c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// The four fp32 values of a lane's chunk are four K positions; A and B use
// the same assignment, so the sum over K is unchanged.
template <>
struct Mma<false> {
  static __device__ __forceinline__ void run(const u32x4 &a, const u32x4 &b, f32x16 &c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[0]), __uint_as_float(b[0]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[1]), __uint_as_float(b[1]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[2]), __uint_as_float(b[2]), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[3]), __uint_as_float(b[3]), c, 0, 0, 0);
  }
};

// LDS index (in 16-byte chunks) of chunk cc of tile row r.
__device__ __forceinline__ int swz(int r, int cc) { return r * 8 + (cc ^ (r & 7)); }

__device__ __forceinline__ int clamp_row(int v, int M) { return v < 0 ? 0 : (v > M ? M : v); }

struct Tile {
  int expert, lo, hi, m0, n_tile;
};

// Which expert and which (m, n) tile block L computes.  Tiles are numbered
// expert by expert; inside an expert n-tile major and m-tile minor, so the
// m-tiles that share one weight tile are adjacent.  Every wave of the block
// computes the same answer.  Returns false past the last real tile.
template <int BM>
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int G, int M,
                                          int ntiles, int L, Tile &t) {
  const int lane = lane_id();
  int running = 0;
  for (int eb = 0; eb < G; eb += kWave) {
    const int e = eb + lane;
    int a = 0, b = 0, tiles = 0;
    if (e < G) {
      a = clamp_row(offsets[e], M);
      b = clamp_row(offsets[e + 1], M);
      const int n = b > a ? b - a : 0;
      tiles = ((n + BM - 1) / BM) * ntiles;
    }
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int excl = running + incl - tiles;
    const uint64_t hit = __ballot(tiles > 0 && L >= excl && L < excl + tiles);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      t.expert = eb + src;
      t.lo = uniform(__shfl(a, src));
      t.hi = uniform(__shfl(b, src));
      const int local = L - uniform(__shfl(excl, src));
      const int mtiles = (t.hi - t.lo + BM - 1) / BM;
      t.m0 = t.lo + (local % mtiles) * BM;
      t.n_tile = local / mtiles;
      return true;
    }
    running += __shfl(incl, kWave - 1);
  }
  return false;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Block tile BM x BN of the output (BN output columns of h or y), WM x WN
// waves, each wave (BM/WM) x (BN/WN).  For SWIGLU the weight tile holds the
// BN gate rows and then the BN matching up rows, and each wave keeps a gate
// and an up accumulator per MFMA block.
//
//   A       [M, K] rows, kvec = K * elem / 16 chunks per row
//   B       expert weights; expert g's first row at chunk g * b_expert_vec,
//           up rows (SWIGLU) b_up_vec chunks after the gate rows
//   C       [M, N] output, dtype of A
template <bool BF16, int BM, int BN, int WM, int WN, bool SWIGLU>
__global__ __launch_bounds__(WM *WN * 64) void k_grouped_gemm(
    const u32x4 *__restrict__ A, int M, int kvec, const int32_t *__restrict__ offsets, int G,
    const u32x4 *__restrict__ B, int64_t b_expert_vec, int64_t b_up_vec, int ntiles, int N,
    void *__restrict__ C) {
  constexpr int NT = WM * WN * 64;
  constexpr int BR = SWIGLU ? 2 * BN : BN;      // weight rows per tile
  constexpr int A_PER = BM * 8 / NT;            // 16-byte chunks per thread per k-step
  constexpr int B_PER = BR * 8 / NT;
  constexpr int WMR = BM / WM, WNR = BN / WN;   // wave tile
  constexpr int FM = WMR / 32, FN = WNR / 32;   // 32x32 MFMA blocks per wave
  constexpr int NB = SWIGLU ? 2 * FN : FN;      // B fragments (gate, then up) per k-group
  static_assert(A_PER * NT == BM * 8 && B_PER * NT == BR * 8, "tile / thread mismatch");
  static_assert(FM >= 1 && FN >= 1, "wave tile too small");

  __shared__ u32x4 As[BM * 8];
  __shared__ u32x4 Bs[BR * 8];

  Tile tile;
  if (!find_tile<BM>(offsets, G, M, ntiles, blockIdx.x, tile)) return;
  const int m0 = tile.m0, hi = tile.hi, n0 = tile.n_tile * BN;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = uniform(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int cc_ld = tid & 7;
  const int row_ld = tid >> 3;

  // Global chunk pointers for k-step 0.  Rows past the segment end re-read its
  // last row (their results are never stored).
  const u32x4 *pa[A_PER];
#pragma unroll
  for (int r = 0; r < A_PER; ++r) {
    int row = m0 + row_ld + r * (NT / 8);
    row = row < hi ? row : hi - 1;
    pa[r] = A + (int64_t)row * kvec + cc_ld;
  }
  const u32x4 *bexp = B + (int64_t)tile.expert * b_expert_vec;
  const u32x4 *pb[B_PER];
#pragma unroll
  for (int r = 0; r < B_PER; ++r) {
    const int brow = row_ld + r * (NT / 8);
    const u32x4 *base = bexp;
    int n = n0 + brow;
    if (SWIGLU && brow >= BN) {
      base += b_up_vec;
      n = n0 + brow - BN;
    }
    pb[r] = base + (int64_t)n * kvec + cc_ld;
  }

  // 32-row blocks of this wave that hold at least one live row.
  const int wrow0 = m0 + wm * WMR;
  int live = (hi - wrow0 + 31) / 32;
  live = live < 0 ? 0 : (live > FM ? FM : live);

  f32x16 acc[FM][NB];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  u32x4 ra[A_PER], rb[B_PER];
#pragma unroll
  for (int r = 0; r < A_PER; ++r) ra[r] = pa[r][0];
#pragma unroll
  for (int r = 0; r < B_PER; ++r) rb[r] = pb[r][0];

  const int KT = kvec / 8;
  for (int kt = 0; kt < KT; ++kt) {
    if (kt > 0) __syncthreads();
#pragma unroll
    for (int r = 0; r < A_PER; ++r) As[swz(row_ld + r * (NT / 8), cc_ld)] = ra[r];
#pragma unroll
    for (int r = 0; r < B_PER; ++r) Bs[swz(row_ld + r * (NT / 8), cc_ld)] = rb[r];
    __syncthreads();
    if (kt + 1 < KT) {
      const int off = (kt + 1) * 8;
#pragma unroll
      for (int r = 0; r < A_PER; ++r) ra[r] = pa[r][off];
#pragma unroll
      for (int r = 0; r < B_PER; ++r) rb[r] = pb[r][off];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = 2 * q + (lane >> 5);
      u32x4 fa[FM], fb[NB];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = As[swz(wm * WMR + i * 32 + (lane & 31), cc)];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        fb[j] = Bs[swz(wn * WNR + j * 32 + (lane & 31), cc)];
        if (SWIGLU) fb[FN + j] = Bs[swz(BN + wn * WNR + j * 32 + (lane & 31), cc)];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i < live) {
#pragma unroll
          for (int j = 0; j < NB; ++j) Mma<BF16>::run(fa[i], fb[j], acc[i][j]);
        }
      }
    }
  }

  // Epilogue.  MFMA 32x32 output layout: lane l holds column l % 32 and, in
  // register v, row 8 (v / 4) + 4 (l / 32) + v % 4.
  const int col_l = lane & 31, row_l = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (i >= live) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WNR + j * 32 + col_l;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wrow0 + i * 32 + 8 * (v >> 2) + row_l + (v & 3);
        if (row < hi) {
          const float val = SWIGLU ? silu(acc[i][j][v]) * acc[i][FN + j][v] : acc[i][j][v];
          const int64_t idx = (int64_t)row * N + col;
          if (BF16)
            static_cast<uint16_t *>(C)[idx] = (uint16_t)f32_to_bf16_rne(val);
          else
            static_cast<float *>(C)[idx] = val;
        }
      }
    }
  }
}

template <bool BF16, int BM, int BN, int WM, int WN>
moe_status launch_pair(const void *a, int M, int d, int ffn, const int32_t *offsets, int G,
                       const void *w13, const void *w2, void *h, void *y, hipStream_t stream) {
  const int elem = BF16 ? 2 : 4;
  const int mtiles_max = (M + BM - 1) / BM + G;
  const dim3 block(WM * WN * 64);
  // GEMM1: K = d, N = ffn, weights w13 [G, 2, ffn, d]
  {
    const int kvec = d * elem / 16;
    const int ntiles = ffn / BN;
    const int64_t b_expert = (int64_t)2 * ffn * kvec, b_up = (int64_t)ffn * kvec;
    k_grouped_gemm<BF16, BM, BN, WM, WN, true><<<dim3(mtiles_max * ntiles), block, 0, stream>>>(
        static_cast<const u32x4 *>(a), M, kvec, offsets, G, static_cast<const u32x4 *>(w13),
        b_expert, b_up, ntiles, ffn, h);
  }
  // GEMM2: K = ffn, N = d, weights w2 [G, d, ffn]
  {
    const int kvec = ffn * elem / 16;
    const int ntiles = d / BN;
    const int64_t b_expert = (int64_t)d * kvec;
    k_grouped_gemm<BF16, BM, BN, WM, WN, false><<<dim3(mtiles_max * ntiles), block, 0, stream>>>(
        static_cast<const u32x4 *>(h), M, kvec, offsets, G, static_cast<const u32x4 *>(w2),
        b_expert, 0, ntiles, d, y);
  }
  return launch_status();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_grouped_swiglu(const void *a, moe_dtype dt, int M, int d, int ffn,
                                         const int32_t *offsets, int G, const void *w13,
                                         const void *w2, void *h, void *y, hipStream_t stream) {
  if (M < 0 || G < 1 || d < 1 || ffn < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d % 128 != 0 || ffn % 128 != 0 || G > 4096) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (!a || !offsets || !w13 || !w2 || !h || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w13) || !aligned16(w2) || !aligned16(h) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  // Few rows per expert (decode): 32-row tiles, the weights stream past once.
  const bool small = (int64_t)M < (int64_t)96 * G;
  if (dt == MOE_BF16)
    return small ? launch_pair<true, 32, 128, 1, 4>(a, M, d, ffn, offsets, G, w13, w2, h, y, stream)
                 : launch_pair<true, 128, 128, 2, 2>(a, M, d, ffn, offsets, G, w13, w2, h, y, stream);
  return small ? launch_pair<false, 32, 128, 1, 4>(a, M, d, ffn, offsets, G, w13, w2, h, y, stream)
               : launch_pair<false, 128, 128, 2, 2>(a, M, d, ffn, offsets, G, w13, w2, h, y, stream);
}
