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
// One kernel serves all three shapes: 4 waves, 128 x 128 output tiles, each
// wave a 64 x 64 quarter (2 x 2 MFMA 32x32x16 blocks), K staged 64 at a
// time through an S-stage ring filled by direct global-to-LDS buffer loads.
// Accumulation is fp32; outputs are bf16, rounded to nearest even.
#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"

namespace moe {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128, kBN = 128, kKS = 64;   // tile rows, tile columns, K per slice
constexpr int kThreads = 256;

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
__device__ __forceinline__ int kc_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int kc_slot(int r, int cc) { return r * 8 + (cc ^ kc_key(r)); }

// Column-contiguous tile: 64 K-rows x 128 columns = 256 bytes per K-row,
// four 64-byte segments (32 columns each).  Segment sg of K-row r is stored
// at position sg ^ (r & 3): a transposing read takes 64 bytes from each of
// four K-rows r .. r + 3 per half wave, which then land in four different
// quarters of the 256-byte bank row.
__device__ __forceinline__ int cc_byte(int r, int sg, int byte_in_seg) {
  return r * 256 + ((sg ^ (r & 3)) << 6) + byte_in_seg;
}

// ---- operand fragments ---------------------------------------------------

// MFMA 32x32x16 operand of 32 rows (row block rb) at k-group q from a
// K-contiguous tile: lane l gives row l % 32, K 8 (l / 32) .. + 7.
__device__ __forceinline__ u32x4 frag_kc(const u32x4 *stage, int rb, int q, int lane) {
  return stage[kc_slot(rb * 32 + (lane & 31), 2 * q + (lane >> 5))];
}

// The same operand for 32 columns (column block cb) from a column-contiguous
// tile.  ds_read_b64_tr_b16 works on groups of 16 lanes: if lane 4 i + a of
// a group addresses four consecutive 16-bit values, lane 4 a + b receives
// value b of lanes a, 4 + a, 8 + a, 12 + a.  So lane s addresses K-row
// 16 q + 8 (s / 32) + 4 h + (s % 16) / 4 at columns 16 ((s / 16) % 2) +
// 4 (s % 4) of the block, and lane l receives column l % 32 at K-rows
// 8 (l / 32) + 4 h .. + 3: half h = 0 gives the lane's K 0..3, h = 1 K 4..7.
__device__ __forceinline__ u32x4 frag_tr(const char *stage, int cb, int q, int lane) {
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * q + 8 * (lane >> 5) + 4 * h + ((lane & 15) >> 2);
    const int byte = cc_byte(r, cb, (((lane >> 4) & 1) << 5) + ((lane & 3) << 3));
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(stage + byte));
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    out[2 * h] = w[0];
    out[2 * h + 1] = w[1];
  }
  return out;
}

__device__ __forceinline__ void mma(const u32x4 &a, const u32x4 &b, f32x16 &c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                              __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_at(const uint16_t *p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

template <int MODE, int S>
__global__ __launch_bounds__(kThreads) void k_grouped_gemm_bwd(const BwdParams p) {
  constexpr bool WGRAD = MODE == kWgrad;
  constexpr int STAGE = kBM * kKS * 2 + kKS * kBN * 2;   // bytes: row operand, column operand
  __shared__ __attribute__((aligned(16))) char smem[S * STAGE];

  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  int e, lo, hi, m0, n0;
  const int ntn = p.N / kBN;
  // XCD x (workgroups x, x + 8, ...) takes a contiguous band of tiles, so
  // tiles that share operands run on one L2.  wgrad: the grid has a
  // workgroup per tile; dgrad: a persistent grid walks the band.
  int cur_e = 0, cur_base = 0;
  const int xcd = blockIdx.x % kXcds, nj = gridDim.x / kXcds;
  const int64_t total = WGRAD ? (int64_t)p.G * (p.Mdim / kBM) * ntn
                              : (int64_t)count_tiles<kBM>(p.offsets, p.G, p.R, ntn);
  int L = (int)(total * xcd / kXcds) + (int)(blockIdx.x / kXcds);
  const int band_end = (int)(total * (xcd + 1) / kXcds);

  for (; L < band_end; L += nj) {
    if constexpr (WGRAD) {
      const int per_e = (p.Mdim / kBM) * ntn;
      e = L / per_e;
      const int rem = L - e * per_e;
      m0 = (rem / ntn) * kBM;
      n0 = (rem % ntn) * kBN;
      lo = clamp_row(p.offsets[e], p.R);
      hi = clamp_row(p.offsets[e + 1], p.R);
      if (hi < lo) hi = lo;
    } else {
      Tile t;
      find_tile<kBM>(p.offsets, p.G, p.R, ntn, L, t, cur_e, cur_base);
      e = t.expert;
      lo = t.lo;
      hi = t.hi;
      m0 = t.m0;
      n0 = t.n_tile * kBN;
    }
    const int KT = WGRAD ? (hi - lo + kKS - 1) / kKS : p.K / kKS;

    // ---- loads: every wave fills 4 of the 16 DMA groups of each operand --
    // Row operand.  dgrad: 16 groups of 8 rows x 128 bytes (K-contiguous),
    // rows past the segment end re-read its last row (never stored).  wgrad:
    // 16 groups of 4 K-rows x 256 bytes of A[lo + k, m0 ..], zero past the
    // segment end (the buffer ends there), which zeroes their products.
    // Column operand: 16 groups of 4 K-rows x 256 bytes.  dgrad: rows k of
    // expert e's [K, N] matrix; wgrad: B rows of the segment (clamped to it).
    const int kc_row = lane >> 3, kc_chunk = lane & 7;          // K-contiguous DMA lane map
    const int cc_row = lane >> 4, cc_seg = (lane >> 2) & 3, cc_w = lane & 3;
    const int cc_col = ((cc_seg ^ cc_row) << 5) + cc_w * 8;     // column of this lane's 16 bytes

    // (The buffer's bounds check leaves out the scalar offset, so the wgrad
    // row operand keeps its whole offset, slice included, per lane.)
    const char *a_base;
    uint32_t a_bytes;
    uint32_t a_off[4];
    if constexpr (WGRAD) {
      a_base = static_cast<const char *>(p.a) + (int64_t)lo * p.Mdim * 2;
      a_bytes = (uint32_t)((int64_t)(hi - lo) * p.Mdim * 2);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        a_off[r] = (uint32_t)(((wave + 4 * r) * 4 + cc_row) * p.Mdim + m0 + cc_col) * 2u;
    } else {
      a_base = static_cast<const char *>(p.a);
      a_bytes = (uint32_t)((int64_t)p.R * p.K * 2);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int g = wave + 4 * r;
        int row = m0 + g * 8 + kc_row;
        row = row < hi ? row : hi - 1;
        const uint32_t key = kc_row ^ (g & 1);   // kc_key(8 g + kc_row)
        a_off[r] = (uint32_t)row * (uint32_t)p.K * 2u + (((uint32_t)kc_chunk ^ key) << 4);
      }
    }
    const char *b_base;
    uint32_t b_bytes;
    if constexpr (WGRAD) {
      b_base = static_cast<const char *>(p.b);
      b_bytes = (uint32_t)((int64_t)p.b_rows * p.N * 2);
    } else {
      b_base = static_cast<const char *>(p.b) + (int64_t)e * p.K * p.N * 2;
      b_bytes = (uint32_t)((int64_t)p.K * p.N * 2);
    }
    auto issue = [&](int kt) {
      char *stage = smem + (kt % S) * STAGE;
      u32x4 *sa = reinterpret_cast<u32x4 *>(stage);
      u32x4 *sb = reinterpret_cast<u32x4 *>(stage + kBM * kKS * 2);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int g = wave + 4 * r;
        if constexpr (WGRAD)
          buffer_load_lds16(a_base, a_bytes, sa + g * 64, a_off[r] + (uint32_t)kt * kKS * (uint32_t)p.Mdim * 2u, 0);
        else
          buffer_load_lds16(a_base, a_bytes, sa + g * 64, a_off[r], (uint32_t)kt * kKS * 2u);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int g = wave + 4 * r;
        const int krow = kt * kKS + g * 4 + cc_row;
        uint32_t off;
        if constexpr (WGRAD) {
          int row = lo + krow;
          row = row < hi ? row : hi - 1;
          uint32_t src = (uint32_t)row;
          if (p.gather) {
            src = (uint32_t)p.gather[row] / (uint32_t)p.gk;
            src = src < (uint32_t)p.b_rows ? src : (uint32_t)p.b_rows - 1u;
          }
          off = (src * (uint32_t)p.N + (uint32_t)(n0 + cc_col)) * 2u;
        } else {
          off = ((uint32_t)krow * (uint32_t)p.N + (uint32_t)(n0 + cc_col)) * 2u;
        }
        buffer_load_lds16(b_base, b_bytes, sb + g * 64, off, 0);
      }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < KT) issue(s);

    for (int kt = 0; kt < KT; ++kt) {
      // This wave's 8 loads of slice kt are done once no more than its loads
      // of the later slices already issued remain in flight; then one
      // barrier makes the slice visible and frees the stage slice
      // kt + S - 1 reuses (read in step kt - 1).
      asm volatile("" ::: "memory");
      wait_vmcnt(((kt + S - 2 < KT - 1 ? kt + S - 2 : KT - 1) - kt) * 8);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const char *stage = smem + (kt % S) * STAGE;
      const u32x4 *sa = reinterpret_cast<const u32x4 *>(stage);
      const char *sa_bytes = stage;
      const char *sb = stage + kBM * kKS * 2;
      u32x4 fa[2][2], fb[2][2];
      auto fetch = [&](int q, int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if constexpr (WGRAD)
            fa[buf][i] = frag_tr(sa_bytes, 2 * wm + i, q, lane);
          else
            fa[buf][i] = frag_kc(sa, 2 * wm + i, q, lane);
          fb[buf][i] = frag_tr(sb, 2 * wn + i, q, lane);
        }
      };
      fetch(0, 0);
      if (kt + S - 1 < KT) issue(kt + S - 1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q < 3) fetch(q + 1, (q + 1) & 1);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) mma(fa[q & 1][i], fb[q & 1][j], acc[i][j]);
      }
    }
    // Every wave is done with LDS before the next tile's loads land there.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // ---- epilogue ----------------------------------------------------
    // MFMA 32x32 output layout: lane l holds column l % 32 and, in register
    // v, row 8 (v / 4) + 4 (l / 32) + v % 4.  Adjacent lanes trade values so
    // each holds two adjacent columns of one row (even lanes rows v % 4 =
    // 0, 2, odd lanes 1, 3) and moves them with one 4-byte access.
    const bool odd = lane & 1;
    const int row_l = 4 * (lane >> 5);
    const int row_hi = WGRAD ? m0 + kBM : hi;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rblk = m0 + (2 * wm + i) * 32;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c0 = (n0 + (2 * wn + j) * 32 + (lane & 31)) & ~1;
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
              const float s = 1.0f / (1.0f + __expf(-g[c]));
              const float silu_g = g[c] * s;
              dg[c] = dh[c] * u[c] * (s * (1.0f + g[c] * (1.0f - s)));
              du[c] = dh[c] * silu_g;
            }
            uint16_t *out = static_cast<uint16_t *>(p.c);
            *reinterpret_cast<uint32_t *>(out + base) = pack_bf16x2(dg[0], dg[1]);
            *reinterpret_cast<uint32_t *>(out + base + p.N) = pack_bf16x2(du[0], du[1]);
          } else {
            const int64_t base = WGRAD ? ((int64_t)e * p.Mdim + row) * p.N + c0 : (int64_t)row * p.N + c0;
            *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(p.c) + base) = pack_bf16x2(x0, x1);
          }
        }
      }
    }
  }
}

constexpr int kStages = 2;

template <int MODE>
void launch(const BwdParams &prm, hipStream_t stream, int64_t tiles) {
  auto kern = k_grouped_gemm_bwd<MODE, kStages>;
  int grid;
  if (MODE == kWgrad) {
    grid = (int)((tiles + kXcds - 1) / kXcds * kXcds);
  } else {
    static int per_cu = 0;
    grid = persistent_grid((const void *)kern, kThreads, per_cu, tiles);
  }
  kern<<<dim3(grid), dim3(kThreads), 0, stream>>>(prm);
}

// Shape checks common to the entry points.  The kernels index their
// operands with 32-bit byte offsets.
moe_status check_bwd(moe_dtype dt, int M, int d, int ffn, int G) {
  if (M < 0 || G < 1 || d < 1 || ffn < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d % kBN != 0 || ffn % kBN != 0 || G > 4096) return MOE_ERR_UNSUPPORTED;
  const int64_t big = (int64_t)1 << 32;
  if ((int64_t)M * 2 * ffn * 2 >= big || (int64_t)M * d * 2 >= big || (int64_t)2 * ffn * d * 2 >= big)
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
  BwdParams prm{dy_perm, w2, dgu, gu, offsets, nullptr, G, M, d, 0, ffn, 1, 0};
  launch<kDgradSwiglu>(prm, stream, ((int64_t)M + kBM - 1) / kBM * (ffn / kBN) + (int64_t)G * (ffn / kBN));
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
  BwdParams prm{dgu, w13, dx_perm, nullptr, offsets, nullptr, G, M, 2 * ffn, 0, d, 1, 0};
  launch<kDgradStore>(prm, stream, ((int64_t)M + kBM - 1) / kBM * (d / kBN) + (int64_t)G * (d / kBN));
  return launch_status();
}

extern "C" moe_status moe_grouped_weight_grad(const void *a, const void *b, moe_dtype dt, int M,
                                              int m_dim, int n_dim, const int32_t *offsets, int G,
                                              const int32_t *b_order, int b_k, int b_rows,
                                              void *c, hipStream_t stream) {
  if (M < 0 || G < 1 || m_dim < 1 || n_dim < 1 || b_k < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (m_dim % kBM != 0 || n_dim % kBN != 0 || G > 4096) return MOE_ERR_UNSUPPORTED;
  if (!b_order) b_rows = M;
  if (b_rows < 1 && M > 0) return MOE_ERR_INVALID_ARG;
  const int64_t big = (int64_t)1 << 32;
  if ((int64_t)(M + kKS) * m_dim * 2 >= big || (int64_t)b_rows * n_dim * 2 >= big ||
      (int64_t)G * m_dim * n_dim >= ((int64_t)1 << 40))
    return MOE_ERR_UNSUPPORTED;
  // With no rows the operands are never read (every expert's gradient is 0).
  if (!offsets || !c || (M > 0 && (!a || !b))) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return MOE_ERR_INVALID_ARG;
  BwdParams prm{a, b, c, nullptr, offsets, b_order, G, M, 0, m_dim, n_dim, b_k, b_rows};
  launch<kWgrad>(prm, stream, (int64_t)G * (m_dim / kBM) * (n_dim / kBN));
  return launch_status();
}
