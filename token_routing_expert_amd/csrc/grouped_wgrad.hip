// Weight gradients of the grouped expert products: for every expert e,
//   C[e] = A[seg e]^T B[seg e]      ([Mdim, N], bf16, fp32 accumulation)
// where seg e is the expert's segment of packed rows, A is [M, Mdim] and B is
// [M, N] (both row-major).  dW_down,e = dY^T H and dW13,e = dGU^T X are this
// product.
//
// "Expert parallelism" (zerotofrontier.app), "A worked example at
// DeepSeek-V3's shape": the backward costs twice the forward's FLOPs, and a
// third of the backward is these products.  Their reduction is only an
// expert's rows (about 256 at DeepSeek-V3's prefill), while their outputs
// are whole weight matrices: at that shape the dW13 launch writes 15 GB for
// 3.85 TFLOP, so every 256 x 256 output tile is eight 32-row K slices of
// MFMA work followed by 128 KB of stores.  Issued at the end of the tile and
// waited for before the next tile's first loads (a wave's vector memory
// counter also counts its stores), those stores took 40% of the launch.
//
// This kernel keeps the two-group ping-pong schedule of the forward products
// (8 waves; group 0 loads the A slices, group 1 the B slices, each group's
// MFMAs overlap the other's LDS reads) and removes the tile boundary from
// the pipeline:
//   1. a workgroup's tiles are one stream of K slices: each group keeps
//      issuing the slice a fixed distance ahead of the one it reads, across
//      tile boundaries, so a tile's first slices are already in LDS when its
//      predecessor ends;
//   2. a group's epilogue is one more phase of the ping-pong: it runs while
//      the other group computes (or reads), and writes the group's 128 x 64
//      part per wave through 4 KB of LDS (a ring stage no slice occupies at
//      that point), storing 16-byte lanes that cover whole 128-byte lines:
//      16 nontemporal stores per wave;
//   3. every wait for a slice counts the stores issued after it, so a wave
//      waits for its stores only when it needs a slice issued after them,
//      while they drain under its MFMAs.
// Both operands are column-contiguous for MFMA (the reduction runs along
// their rows), so they are staged as they lie in memory and read back with
// the transposing LDS read (frag_tr).
#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"

namespace moe {
namespace {

constexpr int kWgTile = 256;                 // output rows and columns of a tile
constexpr int kWgSlice = 32;                 // K-rows (segment rows) per slice
constexpr int kWgStage = kWgTile * kWgSlice * 2 / 16;   // 16-byte chunks per operand stage (16 KB)
constexpr int kWgLoads = kWgStage / 64 / 4;  // 1 KB loads per wave per slice: 4
constexpr int kWgStores = 16;                // 16-byte stores per wave per tile
constexpr int kWgRowBlocks = 4;              // 32-row blocks per wave
constexpr int kWgColBlocks = 2;              // 32-column blocks per wave

template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) { static_for_impl<0, N>(f); }

struct WgTile {
  int e, m0, n0;   // expert, first output row and column
  int lo, hi;      // the expert's segment of packed rows
  int kt;          // K slices
};

// Tile order within an expert: BM = 0 walks m tiles, n fastest; BM > 0 walks
// bands of BM m tiles, n tile by n tile, m fastest inside the band (a band
// of all m tiles is m fastest).
template <int BM>
__device__ __forceinline__ WgTile wg_tile_of(int L, int mt, int nt, int lo_raw, int hi_raw, int M) {
  WgTile t;
  t.e = L / (mt * nt);
  const int rem = L - t.e * (mt * nt);
  if constexpr (BM == 0) {
    t.m0 = (rem / nt) * kWgTile;
    t.n0 = (rem % nt) * kWgTile;
  } else {
    const int bm = BM < mt ? BM : mt;            // m tiles per full band
    const int band = rem / (bm * nt), r2 = rem - band * (bm * nt);
    const int bmc = mt - band * bm < bm ? mt - band * bm : bm;   // m tiles of this band
    t.m0 = (band * bm + r2 % bmc) * kWgTile;
    t.n0 = (r2 / bmc) * kWgTile;
  }
  t.lo = clamp_row(lo_raw, M);
  const int hi = clamp_row(hi_raw, M);
  t.hi = hi > t.lo ? hi : t.lo;
  t.kt = (t.hi - t.lo + kWgSlice - 1) / kWgSlice;
  return t;
}
template <int BM>
__device__ __forceinline__ WgTile wg_tile(int L, int mt, int nt, const int32_t *__restrict__ offsets,
                                          int M) {
  const int e = L / (mt * nt);
  return wg_tile_of<BM>(L, mt, nt, offsets[e], offsets[e + 1], M);
}

// s_waitcnt vmcnt(a kWgLoads + b) for a in [0, A) and b in {0, kWgStores}:
// the counts a wave's slice waits can take, each an immediate.
// Any other a waits for everything (never needed; a safe default).
template <int A>
__device__ __forceinline__ void wait_vmcnt_of(int a, int b) {
  static_assert((A - 1) * kWgLoads + kWgStores < 64, "vmcnt");
  if (a < 0 || a >= A) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  } else if (b == 0) {
    static_for<A>([&](auto i) {
      constexpr int n = decltype(i)::value * kWgLoads;
      if (a == decltype(i)::value) __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    });
  } else {
    static_for<A>([&](auto i) {
      constexpr int n = decltype(i)::value * kWgLoads + kWgStores;
      if (a == decltype(i)::value) __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    });
  }
}

// The slice stream of one wave of group GRP (0 loads the A slices, 1 the B
// slices) over the tiles L0, L0 + Lstep, ... below band_end.  The group is a
// template argument so that the fragment addresses (which depend on it) fold
// into constant offsets.
// SA / SB: stages of the A and B rings; DA / DB: slices of A / B in flight
// ahead of the one being read.  A ring keeps one stage beyond those free at
// every tile end for the epilogue's staging.  NT: nontemporal output stores;
// BM: tile order (wg_tile).
template <int GRP, int SA, int SB, int DA, int DB, bool NT, int BM>
__device__ __forceinline__ void wg_run(const u32x4 *__restrict__ A, const u32x4 *__restrict__ B, int M,
                                       int Mdim, int N, const int32_t *__restrict__ offsets,
                                       uint16_t *__restrict__ C, u32x4 *smem, int L0, int band_end,
                                       int Lstep, int wq, int lane) {
  static_assert(SA >= DA + 2 && SB >= DB + 2, "a free ring stage at each tile end");
  constexpr int S = GRP == 0 ? SA : SB;             // stages of this wave's ring
  constexpr int AHEAD = GRP == 0 ? DA : DB;         // slices issued ahead of the one read
  u32x4 *const a_ring = smem;
  u32x4 *const b_ring = smem + SA * kWgStage;
  u32x4 *const ring = GRP == 0 ? a_ring : b_ring;
  const int mt = Mdim / kWgTile, nt = N / kWgTile;

  // ---- issue side: the next slice of the stream this wave loads ----------
  // A lane's byte offset holds the whole position (K-row of the slice,
  // column), so the buffer's bounds check -- the buffer ends at the segment
  // end -- turns the K-rows of a last partial slice into zeros.
  const int ld = GRP == 0 ? Mdim : N;               // elements per operand row
  const u32x4 *const opnd = GRP == 0 ? A : B;
  const uint32_t kstep = (uint32_t)kWgSlice * (uint32_t)ld * 2u;   // bytes per slice
  uint32_t off[kWgLoads];
  const u32x4 *base = opnd;
  uint32_t bytes = 0;
  int Li = L0, kti = 0, KTi = 0;   // tile, slice within it, its slices
  bool idone = false;              // every slice of the stream issued
  int ji = 0;                      // stream position of the next slice issued
  auto setup = [&](const WgTile &t) {
    base = opnd + (int64_t)t.lo * (ld / 8);
    bytes = (uint32_t)((int64_t)(t.hi - t.lo) * ld * 2);
    const int c0 = GRP == 0 ? t.m0 : t.n0;
#pragma unroll
    for (int r = 0; r < kWgLoads; ++r) {
      int krow, col;
      cc_lane<kWgTile>(wq + 4 * r, lane, krow, col);
      off[r] = ((uint32_t)krow * (uint32_t)ld + (uint32_t)(c0 + col)) * 2u;
    }
  };
  // Move the cursor past a finished tile, and past tiles of empty experts,
  // which have no slices.  In the loop this runs right after a compute
  // phase's MFMAs are issued: every LDS read of the phase has landed, so the
  // wait for the segment bounds' scalar loads waits for nothing else, and it
  // overlaps the MFMAs still executing.
  auto advance = [&]() {
    while (!idone && kti == KTi) {
      Li += Lstep;
      if (Li >= band_end) {
        idone = true;
        break;
      }
      const WgTile t = wg_tile<BM>(Li, mt, nt, offsets, M);
      setup(t);
      kti = 0;
      KTi = t.kt;
    }
  };
  // Issue the cursor's slice; advance() has run since the previous issue.
  auto issue_next = [&]() {
    if (idone) return;
    u32x4 *stage = ring + (ji % S) * kWgStage;
    // The buffer's base and size are wave-uniform by construction; stating
    // it keeps the compiler from looping over lanes around each load.
    const uint64_t b64 = reinterpret_cast<uint64_t>(base);
    const u32x4 *ub = reinterpret_cast<const u32x4 *>(
        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b64 >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b64));
    const uint32_t ubytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);
#pragma unroll
    for (int r = 0; r < kWgLoads; ++r)
      buffer_load_lds16(ub, ubytes, stage + (wq + 4 * r) * 64, off[r] + (uint32_t)kti * kstep, 0);
    ++ji;
    ++kti;
  };
  // Wait until stream slice j (already issued) has landed.  In flight after
  // it may stay: the slices issued after it and, if the last epilogue's
  // stores came after it, those stores.  (Should an earlier epilogue's
  // stores also have come after it, the wait is stricter than needed.)
  int last_epi_ji = 0;   // ji when the last epilogue's stores were issued
  auto wait_for = [&](int j) {
    wait_vmcnt_of<AHEAD>(ji - 1 - j, j < last_epi_ji ? kWgStores : 0);
  };

  // ---- compute side ------------------------------------------------------
  // Output of this wave: row blocks GRP + 2 i (32 rows each) and column
  // blocks 2 wq, 2 wq + 1 of the tile.

  {
    const WgTile t0 = wg_tile<BM>(L0, mt, nt, offsets, M);
    setup(t0);
    KTi = t0.kt;
    advance();
  }
#pragma unroll
  for (int s = 0; s < AHEAD; ++s) {
    issue_next();
    advance();
  }
  asm volatile("" ::: "memory");
  if (ji > 0) wait_for(0);
  asm volatile("" ::: "memory");
  phase_barrier();
  asm volatile("" ::: "memory");

  int jc = 0;   // stream position of the next slice read
  for (int L = L0;;) {
    const WgTile t = wg_tile<BM>(L, mt, nt, offsets, M);
    if (GRP == 1) phase_barrier();   // group 1 runs one phase behind group 0
    asm volatile("" ::: "memory");
    f32x16 acc[kWgRowBlocks][kWgColBlocks];
#pragma unroll
    for (int i = 0; i < kWgRowBlocks; ++i)
#pragma unroll
      for (int j = 0; j < kWgColBlocks; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

#pragma unroll 1
    for (int kt = 0; kt < t.kt; ++kt, ++jc) {
      // Memory phase: this wave's fragments of slice jc, then the next load.
      const char *As = reinterpret_cast<const char *>(a_ring + (jc % SA) * kWgStage);
      const char *Bs = reinterpret_cast<const char *>(b_ring + (jc % SB) * kWgStage);
      u32x4 fa[2][kWgRowBlocks], fb[2][kWgColBlocks];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int j = 0; j < kWgColBlocks; ++j) fb[q][j] = frag_tr<kWgTile>(Bs, 2 * wq + j, q, lane);
#pragma unroll
        for (int i = 0; i < kWgRowBlocks; ++i) fa[q][i] = frag_tr<kWgTile>(As, GRP + 2 * i, q, lane);
      }
      issue_next();
      asm volatile("" ::: "memory");
      // Group 0 reads slice jc + 1 at its next memory phase, right after the
      // next barrier but one.
      if (GRP == 1 && jc + 1 < ji) wait_for(jc + 1);
      asm volatile("" ::: "memory");
      phase_barrier();
      asm volatile("" ::: "memory");
      // Compute phase.
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < kWgRowBlocks; ++i)
#pragma unroll
          for (int j = 0; j < kWgColBlocks; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fb[q][j]),
                                                                __builtin_bit_cast(bf16x8, fa[q][i]),
                                                                acc[i][j], 0, 0, 0);
      asm volatile("" ::: "memory");
      advance();
      asm volatile("" ::: "memory");
      if (GRP == 0 && jc + 1 < ji) wait_for(jc + 1);
      asm volatile("" ::: "memory");
      phase_barrier();
      asm volatile("" ::: "memory");
    }

    if (GRP == 0) phase_barrier();   // wait out group 1's last compute phase
    asm volatile("" ::: "memory");
    // Epilogue phase (the other group computes or reads meanwhile).  The
    // staging block is in the stage of stream slice jc + AHEAD: the slices
    // in flight or unread are jc .. jc + AHEAD - 1, and this wave refills
    // that stage only at its next memory phase.
    // The MFMAs take the B fragment as their first operand, so each 32 x 32
    // block holds the transpose: lane l holds output row l % 32 and, in
    // register v, output column 8 (v / 4) + 4 (l / 32) + v % 4 -- registers
    // 4 a .. 4 a + 3 are four consecutive columns of one row, one 8-byte bf16
    // word.  A 32-row block goes to the staging block row-major in bf16
    // (32 rows x 128 bytes): 16-byte chunk c of row r sits at c ^ (r % 8),
    // its two 8-byte halves swapped when bit 3 of r is set.  LDS writes are
    // served 16 lanes (128 bytes) per cycle with banks repeating every 128
    // bytes, and the 16 lanes of a write here are 16 rows of one half-chunk:
    // the rotation gives them 16 different 8-byte slots.  (A rotation by
    // r / 2 measured 2-way conflicts on every write.)  Each lane then reads 16
    // bytes of one row (8 lanes per row, so 16 lanes cover two whole rows),
    // swaps the halves back in rows 8..15 and 24..31, and stores them:
    // every store instruction writes 8 whole 128-byte rows.  The buffer
    // store's scalar offset carries the row step, so the stores need no
    // address arithmetic.
    char *const stg = reinterpret_cast<char *>(ring + ((jc + AHEAD) % S) * kWgStage) + wq * 4096;
    const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        C + (int64_t)t.e * Mdim * N, (short)0, 0x7FFFFFFF, kBufferFlags);
    const int wrow = lane & 31, whalf = lane >> 5;   // write side: row, 8-byte half of a chunk
    const int rrow = lane >> 3, rch = lane & 7;      // read side: row (of 8), chunk
    const uint32_t vout = ((uint32_t)(t.m0 + 32 * GRP + rrow) * (uint32_t)N +
                           (uint32_t)(t.n0 + 64 * wq + 8 * rch)) * 2u;
#pragma unroll
    for (int i = 0; i < kWgRowBlocks; ++i) {
#pragma unroll
      for (int j = 0; j < kWgColBlocks; ++j)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 pk = {(__bf16)acc[i][j][4 * a], (__bf16)acc[i][j][4 * a + 1],
                             (__bf16)acc[i][j][4 * a + 2], (__bf16)acc[i][j][4 * a + 3]};
          const int chunk = (4 * j + a) ^ (wrow & 7);
          const int half = whalf ^ ((wrow >> 3) & 1);
          *reinterpret_cast<u32x2 *>(stg + wrow * 128 + chunk * 16 + half * 8) = __builtin_bit_cast(u32x2, pk);
        }
      u32x4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 8 * u + rrow;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + r * 128 + ((rch ^ (r & 7)) << 4));
        q[u] = (u & 1) == 0 ? v : u32x4{v[2], v[3], v[0], v[1]};   // rows with bit 3 set (u odd)
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // Rows 64 i + 8 u of this wave's row blocks (block GRP + 2 i).
        const uint32_t soff = (uint32_t)(64 * i + 8 * u) * (uint32_t)N * 2u;
        __builtin_amdgcn_raw_buffer_store_b128(q[u], out_rsrc, vout, soff, NT ? 2 : 0);
      }
    }
    last_epi_ji = ji;
    asm volatile("" ::: "memory");
    phase_barrier();
    asm volatile("" ::: "memory");
    L += Lstep;
    if (L >= band_end) break;
  }
}

template <int SA, int SB, int DA, int DB, bool NT, int BM>
__global__ __launch_bounds__(512) void k_weight_grad(const u32x4 *__restrict__ A, const u32x4 *__restrict__ B,
                                                     int M, int Mdim, int N,
                                                     const int32_t *__restrict__ offsets, int G,
                                                     uint16_t *__restrict__ C) {
  static_assert(DA >= 1 && DB >= 1, "rings");
  static_assert((SA + SB) * kWgStage * 16 <= 160 * 1024, "LDS");
  __shared__ u32x4 smem[(SA + SB) * kWgStage];

  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int total = G * (Mdim / kWgTile) * (N / kWgTile);

  // Persistent walk.  Workgroup i runs on XCD i mod 8.  With many balanced
  // experts each XCD takes a contiguous band of the tile list, so the tiles
  // sharing an expert's rows run together on one L2.  With few experts, or
  // one expert far above the mean rows, the walk is round-robin over all
  // XCDs instead, which keeps them evenly loaded.
  int mx = 0;
  for (int e = lane; e < G; e += kWave) {
    const int n = clamp_row(offsets[e + 1], M) - clamp_row(offsets[e], M);
    mx = n > mx ? n : mx;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int o = __shfl_xor(mx, off);
    mx = o > mx ? o : mx;
  }
  const bool rr = G <= 16 || (int64_t)uniform(mx) * G > 2 * (int64_t)M;
  const int xcd = blockIdx.x % kXcds, nj = gridDim.x / kXcds;
  const int band_end = rr ? total : (int)((int64_t)total * (xcd + 1) / kXcds);
  const int L0 = rr ? (int)blockIdx.x : (int)((int64_t)total * xcd / kXcds) + (int)(blockIdx.x / kXcds);
  const int Lstep = rr ? (int)gridDim.x : nj;
  if (L0 >= band_end) return;
  if (wave < 4)
    wg_run<0, SA, SB, DA, DB, NT, BM>(A, B, M, Mdim, N, offsets, C, smem, L0, band_end, Lstep, wave, lane);
  else
    wg_run<1, SA, SB, DA, DB, NT, BM>(A, B, M, Mdim, N, offsets, C, smem, L0, band_end, Lstep, wave - 4, lane);
}

}  // namespace

// [G, m_dim, n_dim] weight gradients; false (nothing launched) when m_dim or
// n_dim is not a multiple of 256 or an operand is too large for 32-bit
// offsets.
bool launch_weight_grad(const void *a, const void *b, int M, int m_dim, int n_dim,
                        const int32_t *offsets, int G, void *out, hipStream_t stream) {
  if (m_dim % kWgTile != 0 || n_dim % kWgTile != 0) return false;
  // Lane byte offsets are 32-bit and reach up to a slice past the last row.
  const int64_t widest = m_dim > n_dim ? m_dim : n_dim;
  if ((int64_t)(M + kWgSlice) * widest * 2 >= ((int64_t)1 << 32)) return false;
  const int64_t tiles = (int64_t)G * (m_dim / kWgTile) * (n_dim / kWgTile);
  auto kern = k_weight_grad<5, 5, 3, 3, true, 4>;
  static DeviceCache occ;
  const int grid = persistent_grid((const void *)kern, 512, occ, tiles);
  kern<<<dim3(grid), dim3(512), 0, stream>>>(static_cast<const u32x4 *>(a), static_cast<const u32x4 *>(b),
                                            M, m_dim, n_dim, offsets, G, static_cast<uint16_t *>(out));
  return true;
}

}  // namespace moe
