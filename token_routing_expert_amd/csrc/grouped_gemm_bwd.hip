// Backward products of the grouped SwiGLU expert MLP.
//
// The backward pass costs twice the forward's products, 12 d d_e FLOPs per
// assignment ("Expert parallelism", section "A worked example at
// DeepSeek-V3's shape"): for each of the three matrices one product for the
// input gradient and one for the weight gradient.  Per expert e, with the
// rows of its segment (offsets[e] .. offsets[e+1]) stacked:
//
//   dgrad   dh  = dY  Wd_e          [n, d] x [d, ffn]    -> SwiGLU backward -> dGU [n, 2 ffn]
//           dX  = dGU W13_e         [n, 2 ffn] x [2 ffn, d]
//   wgrad   dWd_e  = dY^T  H        [d, n] x [n, ffn]
//           dW13_e = dGU^T X        [2 ffn, n] x [n, d]
//
// The forward products read both operands K-contiguous.  Here the weights of
// a dgrad product are N-contiguous ([K, N] row-major), and both operands of a
// wgrad product are contiguous along the output dimension (the reduction
// runs down the rows).  MFMA wants every lane's 8 bf16 consecutive in K, so
// such operands are staged in LDS as they lie in memory and read back with
// gfx950's transposing LDS read (ds_read_b64_tr_b16), which hands each lane
// four K-consecutive values of one column.
//
// One kernel serves all three shapes: 2 WM waves, (64 WM) x 128 output
// tiles, each wave a 64 x 64 part (2 x 2 MFMA 32x32x16 blocks), K staged 64
// at a time through an S-stage ring filled by direct global-to-LDS buffer
// loads.  Accumulation is fp32; outputs are bf16, rounded to nearest even.
#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"

namespace moe {
namespace {


constexpr int kBN = 128;             // tile columns
constexpr int kMaxG = 1024;          // experts per call (their offsets are staged in LDS)

enum Mode { kDgradStore = 0, kDgradSwiglu = 1, kWgrad = 2 };

struct BwdParams {
  const void *a;            // dgrad: [R, K] rows; wgrad: [R, Mdim] rows
  const void *b;            // dgrad: [G, K, N] expert matrices; wgrad: [b_rows, N] rows
  void *c;                  // dgrad: [R, N] (SwiGLU: dGU [R, 2 N]); wgrad: [G, Mdim, N]
  const void *gu;           // SwiGLU: forward pre-activations [R, 2 N] (gate, then up)
  const int32_t *offsets;   // [G + 1] row segments
  const int32_t *gather;    // wgrad: B row of packed row p is gather[p] / gk (NULL: p)
  int G, R, K, Mdim, N, gk, b_rows;
};

// ---- LDS layouts of one K slice ------------------------------------------
//
// K-contiguous tile (the dgrad's dY or dGU rows): 128 rows x 64 K = 8
// chunks of 16 bytes per row, chunk cc of row r in slot cc ^ key(r) so an
// operand read (32 rows at one chunk) spreads over all banks.
// A row of a slice is CPR chunks: 8 (128 bytes: 64 bf16 or 32 fp32 of K) or
// 4 (64 bytes), where the key is (r / 4) % 4 so that 16 consecutive rows read
// at one chunk cover all 16 bank positions of 256 bytes.
template <int CPR>
__device__ __forceinline__ int kc_key(int r) {
  if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return (r >> 2) & 3;
}
template <int CPR>
__device__ __forceinline__ int kc_slot(int r, int cc) { return r * CPR + (cc ^ kc_key<CPR>(r)); }

// ---- operand fragments ---------------------------------------------------

// MFMA operand of 32 rows (row block rb) at k-group q from a K-contiguous
// tile: lane l gives row l % 32 and the 16-byte chunk 2 q + l / 32 (8 bf16
// or 4 fp32 K values).
template <int CPR>
__device__ __forceinline__ u32x4 frag_kc(const u32x4 *stage, int rb, int q, int lane) {
  return stage[kc_slot<CPR>(rb * 32 + (lane & 31), 2 * q + (lane >> 5))];
}

// fp32: the same operand for 32 columns (block cb) of a column-contiguous
// tile of W fp32 columns (4 W bytes per K-row, the segment swizzle of
// cc_byte): lane l gives column l % 32 at the K rows of its chunk,
// 4 (2 q + l / 32) + i for i = 0..3, read one 4-byte value at a time.
template <int W>
__device__ __forceinline__ u32x4 frag_col32(const char *stage, int cb, int q, int lane) {
  const int col = cb * 32 + (lane & 31);
  const int sg = col >> 4, in_seg = (col & 15) * 4;
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (2 * q + (lane >> 5)) + i;
    out[i] = *reinterpret_cast<const uint32_t *>(stage + r * (4 * W) + ((sg ^ (r & 3)) << 6) + in_seg);
  }
  return out;
}

// c += a b^T over one 16-byte chunk per lane: one bf16 MFMA, or four fp32
// MFMAs whose K positions are the chunk's four values (the same assignment
// on both operands, so the sum over K is unchanged).
template <bool BF16>
__device__ __forceinline__ void mma(const u32x4 &a, const u32x4 &b, f32x16 &c) {
  if constexpr (BF16) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
  }
}

// One output tile.
struct TileB {
  int e, lo, hi, m0, n0, KT;
};

// The kernel is persistent: a workgroup walks its band of tiles and its
// S-stage ring streams K slices continuously across tile boundaries, so the
// next tile's first slices load while this tile finishes and stores.  The
// expert offsets are copied to LDS first, so the tile lookups in the stream
// read LDS and never wait behind loads in flight.
template <int MODE, int WM, int S, int KS, bool GATHER, bool BF16>
__global__ __launch_bounds__(WM * 128) void k_grouped_gemm_bwd(const BwdParams p) {
  constexpr bool WGRAD = MODE == kWgrad;
  constexpr int ES = BF16 ? 2 : 4;                    // element bytes
  constexpr int kKS = BF16 ? KS : KS / 2;             // K per slice: the same bytes per row
  constexpr int CPR = kKS * ES / 16;                  // chunks per K-contiguous row
  constexpr int NW = 2 * WM, BM = 64 * WM;
  constexpr int A_BYTES = BM * kKS * ES, B_BYTES = kKS * kBN * ES, STAGE = A_BYTES + B_BYTES;
  constexpr int A_PW = A_BYTES / 1024 / NW, B_PW = B_BYTES / 1024 / NW;   // DMA groups per wave
  constexpr int LPS = A_PW + B_PW;                                       // loads per slice per wave
  static_assert(A_PW * NW * 1024 == A_BYTES && B_PW * NW * 1024 == B_BYTES, "DMA split");
  __shared__ __attribute__((aligned(16))) char smem[S * STAGE];
  __shared__ int32_t s_off[kMaxG + 1];

  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  for (int i = threadIdx.x; i <= p.G; i += NW * 64) s_off[i] = clamp_row(p.offsets[i], p.R);
  __syncthreads();

  const int ntn = p.N / kBN;
  const int mtn = WGRAD ? p.Mdim / BM : 1;
  // XCD x (workgroups x, x + 8, ...) takes a contiguous band of tiles, so
  // tiles that share operands run on one L2 at the same time.
  const int64_t total = WGRAD ? (int64_t)p.G * mtn * ntn : (int64_t)count_tiles<BM>(s_off, p.G, p.R, ntn);
  const int xcd = blockIdx.x % kXcds, nj = gridDim.x / kXcds;
  const int L0 = (int)(total * xcd / kXcds) + (int)(blockIdx.x / kXcds);
  const int band_end = (int)(total * (xcd + 1) / kXcds);

  auto tile_at = [&](int L, int &e0, int &base) {
    TileB t;
    if constexpr (WGRAD) {
      const int per_e = mtn * ntn;
      t.e = L / per_e;
      const int rem = L - t.e * per_e;
      t.m0 = (rem / ntn) * BM;
      t.n0 = (rem % ntn) * kBN;
      t.lo = s_off[t.e];
      t.hi = s_off[t.e + 1] > t.lo ? s_off[t.e + 1] : t.lo;
      t.KT = (t.hi - t.lo + kKS - 1) / kKS;
    } else {
      Tile x;
      find_tile<BM>(s_off, p.G, p.R, ntn, L, x, e0, base);
      t.e = x.expert;
      t.lo = x.lo;
      t.hi = x.hi;
      t.m0 = x.m0;
      t.n0 = x.n_tile * kBN;
      t.KT = p.K / kKS;
    }
    return t;
  };

  // ---- issue cursor: the next K slice to load -----------------------------
  int Li = L0, kti = 0, issued = 0, ie0 = 0, ibase = 0;
  TileB ti{};
  if (Li < band_end) ti = tile_at(Li, ie0, ibase);
  auto settle = [&]() {   // skip to the next tile with a slice left
    while (Li < band_end && kti >= ti.KT) {
      Li += nj;
      kti = 0;
      if (Li < band_end) ti = tile_at(Li, ie0, ibase);
    }
  };
  settle();

  // Row operand.  dgrad: 8 rows x 128 bytes (K-contiguous) per group, rows
  // past the segment end re-read its last row (never stored).  wgrad: A's
  // K-rows lo + k at columns m0 .., zero past the segment end (the buffer
  // ends there, and its bounds check covers the per-lane offset only, so the
  // whole offset is per lane), which zeroes their products.
  // Column operand: expert e's [K, N] matrix (dgrad) or B's rows of the
  // segment, clamped to it (wgrad).
  auto issue = [&]() {
    char *stage = smem + (issued % S) * STAGE;
    u32x4 *sa = reinterpret_cast<u32x4 *>(stage);
    u32x4 *sb = reinterpret_cast<u32x4 *>(stage + A_BYTES);
    const int kt = kti;
#pragma unroll
    for (int r = 0; r < A_PW; ++r) {
      const int g = wave + NW * r;
      if constexpr (WGRAD) {
        // Column-contiguous stage of BM columns: cc_lane in 2-byte units of
        // BM ES / 2 columns, so the element column is col 2 / ES.
        int krow, col;
        cc_lane<BM * ES / 2>(g, lane, krow, col);
        col = col * 2 / ES;
        const uint32_t off = ((uint32_t)(kt * kKS + krow) * (uint32_t)p.Mdim + (uint32_t)(ti.m0 + col)) * (uint32_t)ES;
        buffer_load_lds16(static_cast<const char *>(p.a) + (int64_t)ti.lo * p.Mdim * ES,
                          (uint32_t)((int64_t)(ti.hi - ti.lo) * p.Mdim * ES), sa + g * 64, off, 0);
      } else {
        // One group: 1024 / (16 CPR) rows; lane l fills row l / CPR of it at
        // slot l % CPR, which holds chunk (l % CPR) ^ key(row).
        constexpr int RPG = 64 / CPR;
        const int lr = g * RPG + lane / CPR;
        int row = ti.m0 + lr;
        row = row < ti.hi ? row : ti.hi - 1;
        const uint32_t chunk = (uint32_t)(lane % CPR) ^ (uint32_t)kc_key<CPR>(lr);
        const uint32_t off = (uint32_t)row * (uint32_t)p.K * (uint32_t)ES + (chunk << 4);
        buffer_load_lds16(p.a, (uint32_t)((int64_t)p.R * p.K * ES), sa + g * 64, off,
                          (uint32_t)kt * kKS * (uint32_t)ES);
      }
    }
#pragma unroll
    for (int r = 0; r < B_PW; ++r) {
      const int g = wave + NW * r;
      int krow, col;
      cc_lane<kBN * ES / 2>(g, lane, krow, col);
      col = col * 2 / ES;
      if constexpr (WGRAD) {
        int row = ti.lo + kt * kKS + krow;
        row = row < ti.hi ? row : ti.hi - 1;
        uint32_t src = (uint32_t)row;
        if constexpr (GATHER) {
          src = (uint32_t)p.gather[row] / (uint32_t)p.gk;
          src = src < (uint32_t)p.b_rows ? src : (uint32_t)p.b_rows - 1u;
        }
        buffer_load_lds16(p.b, (uint32_t)((int64_t)p.b_rows * p.N * ES), sb + g * 64,
                          (src * (uint32_t)p.N + (uint32_t)(ti.n0 + col)) * (uint32_t)ES, 0);
      } else {
        // The expert's weights stream past once per column tile: read them
        // non-temporally (decode-shaped input gradients 1.5-2% faster).
        buffer_load_lds16<kNonTemporal>(
            static_cast<const char *>(p.b) + (int64_t)ti.e * p.K * p.N * ES,
            (uint32_t)((int64_t)p.K * p.N * ES), sb + g * 64,
            ((uint32_t)(kt * kKS + krow) * (uint32_t)p.N + (uint32_t)(ti.n0 + col)) * (uint32_t)ES, 0);
      }
    }
    ++issued;
    ++kti;
    settle();
  };

  // ---- consume cursor: the tile being computed ----------------------------
  int Lc = L0, ktc = 0, consumed = 0, ce0 = 0, cbase = 0;
  TileB tc{};
  if (Lc < band_end) tc = tile_at(Lc, ce0, cbase);

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (Li < band_end) issue();

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const bool odd = lane & 1;
  const int row_l = 4 * (lane >> 5);
  while (Lc < band_end) {
    if (ktc < tc.KT) {
      // This wave's loads of the slice are done once no more than its loads
      // of the slices issued after it remain in flight; one barrier then
      // makes the slice visible and frees the stage the next issue reuses
      // (read in the previous step).
      asm volatile("" ::: "memory");
      wait_vmcnt((issued - consumed - 1) * LPS);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const char *stage = smem + (consumed % S) * STAGE;
      const u32x4 *sa = reinterpret_cast<const u32x4 *>(stage);
      const char *sb = stage + A_BYTES;
      u32x4 fa[2][2], fb[2][2];
      auto fetch = [&](int q, int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if constexpr (WGRAD)
            fa[buf][i] = BF16 ? frag_tr<BM>(stage, 2 * wm + i, q, lane)
                              : frag_col32<BM>(stage, 2 * wm + i, q, lane);
          else
            fa[buf][i] = frag_kc<CPR>(sa, 2 * wm + i, q, lane);
          fb[buf][i] = BF16 ? frag_tr<kBN>(sb, 2 * wn + i, q, lane)
                            : frag_col32<kBN>(sb, 2 * wn + i, q, lane);
        }
      };
      constexpr int NQ = kKS * ES / 32;   // k-groups (one 16-byte chunk per lane) per slice
      fetch(0, 0);
      if (Li < band_end) issue();
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (q < NQ - 1) fetch(q + 1, (q + 1) & 1);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) mma<BF16>(fa[q & 1][i], fb[q & 1][j], acc[i][j]);
      }
      ++consumed;
      ++ktc;
    }
    if (ktc < tc.KT) continue;

    // ---- epilogue of tile tc ----------------------------------------------
    // MFMA 32x32 output layout: lane l holds column l % 32 and, in register
    // v, row 8 (v / 4) + 4 (l / 32) + v % 4.  Adjacent lanes trade values so
    // each holds two adjacent columns of one row (even lanes rows v % 4 =
    // 0, 2, odd lanes 1, 3) and moves them with one 4-byte access.
    const int row_hi = WGRAD ? tc.m0 + BM : tc.hi;
    if constexpr (!BF16) {
      // fp32: every lane stores its own values.
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rblk = tc.m0 + (2 * wm + i) * 32;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = tc.n0 + (2 * wn + j) * 32 + (lane & 31);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = rblk + 8 * (v >> 2) + row_l + (v & 3);
            if (row < row_hi) {
              const float x = acc[i][j][v];
              if constexpr (MODE == kDgradSwiglu) {
                const int64_t base = (int64_t)row * 2 * p.N + col;
                const float g = static_cast<const float *>(p.gu)[base];
                const float u = static_cast<const float *>(p.gu)[base + p.N];
                const float s = sigmoid_f(g);
                static_cast<float *>(p.c)[base] = x * u * (s * (1.0f + g * (1.0f - s)));
                static_cast<float *>(p.c)[base + p.N] = x * (g * s);
              } else {
                const int64_t base =
                    WGRAD ? ((int64_t)tc.e * p.Mdim + row) * p.N + col : (int64_t)row * p.N + col;
                static_cast<float *>(p.c)[base] = x;
              }
            }
            acc[i][j][v] = 0.0f;
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < (BF16 ? 2 : 0); ++i) {
      const int rblk = tc.m0 + (2 * wm + i) * 32;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c0 = (tc.n0 + (2 * wn + j) * 32 + (lane & 31)) & ~1;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float mine = odd ? acc[i][j][v + 1] : acc[i][j][v];
          const float give = odd ? acc[i][j][v] : acc[i][j][v + 1];
          const float got =
              __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0xB1, 0xF, 0xF, false));
          const float x0 = odd ? got : mine, x1 = odd ? mine : got;   // columns c0, c0 + 1
          const int row = rblk + 8 * (v >> 2) + row_l + (v & 3) + (odd ? 1 : 0);
          if (row >= row_hi) continue;
          if constexpr (MODE == kDgradSwiglu) {
            // dh -> (dgate, dup) through h = SiLU(g) u:
            //   dgate = dh u SiLU'(g), dup = dh SiLU(g),
            //   SiLU'(g) = s (1 + g (1 - s)), s = 1 / (1 + e^-g).
            const int64_t base = (int64_t)row * 2 * p.N + c0;
            const uint16_t *gu = static_cast<const uint16_t *>(p.gu);
            const uint32_t gg = *reinterpret_cast<const uint32_t *>(gu + base);
            const uint32_t uu = *reinterpret_cast<const uint32_t *>(gu + base + p.N);
            const float g[2] = {bf16_lo(gg), bf16_hi(gg)}, u[2] = {bf16_lo(uu), bf16_hi(uu)};
            const float dh[2] = {x0, x1};
            float dg[2], du[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const float s = sigmoid_f(g[c]);
              dg[c] = dh[c] * u[c] * (s * (1.0f + g[c] * (1.0f - s)));
              du[c] = dh[c] * (g[c] * s);
            }
            uint16_t *out = static_cast<uint16_t *>(p.c);
            *reinterpret_cast<uint32_t *>(out + base) = pack_bf16x2(dg[0], dg[1]);
            *reinterpret_cast<uint32_t *>(out + base + p.N) = pack_bf16x2(du[0], du[1]);
          } else {
            const int64_t base =
                WGRAD ? ((int64_t)tc.e * p.Mdim + row) * p.N + c0 : (int64_t)row * p.N + c0;
            *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(p.c) + base) = pack_bf16x2(x0, x1);
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
      }
    }
    Lc += nj;
    ktc = 0;
    if (Lc < band_end) tc = tile_at(Lc, ce0, cbase);
  }
}

constexpr int kBwdWM = 2;       // waves along M: 2 -> 128-row tiles
constexpr int kBwdStages = 2;
constexpr int kKS = 64;         // K per ring stage

constexpr int kTileM = 64 * kBwdWM;

template <int MODE, bool GATHER, bool BF16>
void launch_t(const BwdParams &prm, hipStream_t stream, int64_t tiles) {
  constexpr int WM = kBwdWM, S = kBwdStages;
  auto kern = k_grouped_gemm_bwd<MODE, WM, S, kKS, GATHER, BF16>;
  static DeviceCache occ;
  const int grid = persistent_grid((const void *)kern, WM * 128, occ, tiles);
  kern<<<dim3(grid), dim3(WM * 128), 0, stream>>>(prm);
}

template <int MODE, bool GATHER = false>
void launch(const BwdParams &prm, hipStream_t stream, int64_t tiles, bool bf16) {
  if (bf16)
    launch_t<MODE, GATHER, true>(prm, stream, tiles);
  else
    launch_t<MODE, GATHER, false>(prm, stream, tiles);
}

// Shape checks common to the entry points.  The kernels index their
// operands with 32-bit byte offsets.
moe_status check_bwd(moe_dtype dt, int M, int d, int ffn, int G) {
  if (M < 0 || G < 1 || d < 1 || ffn < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d % kBN != 0 || ffn % kBN != 0 || G > kMaxG) return MOE_ERR_UNSUPPORTED;
  const int64_t big = (int64_t)1 << 32, es = dt == MOE_F32 ? 4 : 2;
  if ((int64_t)M * 2 * ffn * es >= big || (int64_t)M * d * es >= big || (int64_t)2 * ffn * d * es >= big)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_grouped_down_backward(const void *dy_perm, moe_dtype dt, int M, int d,
                                                int ffn, const int32_t *offsets, int G,
                                                const void *w2, const void *gu, void *dgu,
                                                hipStream_t stream) {
  const moe_status st = check_bwd(dt, M, d, ffn, G);
  if (st != MOE_OK || M == 0) return st;
  if (!dy_perm || !offsets || !w2 || !gu || !dgu) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dy_perm) || !aligned16(w2) || !aligned16(gu) || !aligned16(dgu))
    return MOE_ERR_INVALID_ARG;
  // dh = dY Wd_e: K = d, N = ffn; Wd_e is [d, ffn], N-contiguous.
  const bool bf16 = dt == MOE_BF16;
  if (bf16 && launch_dgrad_pp(2, dy_perm, M, d, ffn, offsets, G, w2, dgu, gu, stream))
    return launch_status();
  BwdParams prm{dy_perm, w2, dgu, gu, offsets, nullptr, G, M, d, 0, ffn, 1, 0};
  launch<kDgradSwiglu>(prm, stream, ((int64_t)M + kTileM - 1) / kTileM * (ffn / kBN) + (int64_t)G * (ffn / kBN),
                       bf16);
  return launch_status();
}

extern "C" moe_status moe_grouped_gate_up_backward(const void *dgu, moe_dtype dt, int M, int d,
                                                   int ffn, const int32_t *offsets, int G,
                                                   const void *w13, void *dx_perm,
                                                   hipStream_t stream) {
  const moe_status st = check_bwd(dt, M, d, ffn, G);
  if (st != MOE_OK || M == 0) return st;
  if (!dgu || !offsets || !w13 || !dx_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dgu) || !aligned16(w13) || !aligned16(dx_perm)) return MOE_ERR_INVALID_ARG;
  // dX = dGU W13_e: K = 2 ffn (gate rows, then up rows), N = d.
  const bool bf16 = dt == MOE_BF16;
  if (bf16 && launch_dgrad_pp(1, dgu, M, 2 * ffn, d, offsets, G, w13, dx_perm, nullptr, stream))
    return launch_status();
  BwdParams prm{dgu, w13, dx_perm, nullptr, offsets, nullptr, G, M, 2 * ffn, 0, d, 1, 0};
  launch<kDgradStore>(prm, stream, ((int64_t)M + kTileM - 1) / kTileM * (d / kBN) + (int64_t)G * (d / kBN),
                      bf16);
  return launch_status();
}

extern "C" moe_status moe_grouped_weight_grad(const void *a, const void *b, moe_dtype dt, int M,
                                              int m_dim, int n_dim, const int32_t *offsets, int G,
                                              const int32_t *b_order, int b_k, int b_rows,
                                              void *c, hipStream_t stream) {
  if (M < 0 || G < 1 || m_dim < 1 || n_dim < 1 || b_k < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (m_dim % kTileM != 0 || n_dim % kBN != 0 || G > kMaxG) return MOE_ERR_UNSUPPORTED;
  if (!b_order) b_rows = M;
  if (b_rows < 1 && M > 0) return MOE_ERR_INVALID_ARG;
  const int64_t big = (int64_t)1 << 32, es = dt == MOE_F32 ? 4 : 2;
  if ((int64_t)(M + kKS) * m_dim * es >= big || (int64_t)b_rows * n_dim * es >= big ||
      (int64_t)G * m_dim * n_dim >= ((int64_t)1 << 40))
    return MOE_ERR_UNSUPPORTED;
  // With no rows the operands are never read (every expert's gradient is 0).
  if (!offsets || !c || (M > 0 && (!a || !b))) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return MOE_ERR_INVALID_ARG;
  const bool bf16 = dt == MOE_BF16;
  if (bf16 && !b_order && launch_weight_grad(a, b, M, m_dim, n_dim, offsets, G, c, stream))
    return launch_status();
  BwdParams prm{a, b, c, nullptr, offsets, b_order, G, M, 0, m_dim, n_dim, b_k, b_rows};
  if (b_order)
    launch<kWgrad, true>(prm, stream, (int64_t)G * (m_dim / kTileM) * (n_dim / kBN), bf16);
  else
    launch<kWgrad>(prm, stream, (int64_t)G * (m_dim / kTileM) * (n_dim / kBN), bf16);
  return launch_status();
}
