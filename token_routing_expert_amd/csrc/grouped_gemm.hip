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
#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"

namespace moe {
namespace {

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

// LDS layout of a staged tile: row r holds 8 16-byte chunks (one K slice of
// 128 bytes: 64 bf16 or 32 fp32).  Chunk cc of row r is stored in slot
// cc ^ key(r).  The key makes any 16 consecutive rows read at one logical
// chunk -- an MFMA operand fetch reads 32 rows at one chunk -- cover every
// bank of a 256-byte LDS bank row exactly once.
__device__ __forceinline__ int swz_key(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int cc) { return r * 8 + (cc ^ swz_key(r)); }

// Block tile: up to BM rows x BN output columns (of h or y), WM x WN waves.
// Wave (wm, wn) owns row blocks wm, wm + WM, wm + 2 WM, ... (32 rows each,
// interleaved so a short tile still spreads over all waves) and BN / WN
// columns.  For SWIGLU the weight tile holds the BN gate rows and then the BN
// matching up rows, and each wave keeps a gate and an up accumulator per MFMA
// block.
//
//   A       [M, K] rows, kvec = K * elem / 16 chunks per row
//   B       expert weights; expert g's first row at chunk g * b_expert_vec,
//           up rows (SWIGLU) b_up_vec chunks after the gate rows
//   C       [M, N] output, dtype of A
//
// Persistent: the grid is a multiple of 8 workgroups sized to the resident
// capacity; workgroup i serves XCD i % 8's band of tiles, so the tiles that
// share operands run on one L2 at the same time.
//
// K loop: 128-byte K slices of the row tile and of the weight tile stream into
// LDS with direct global-to-LDS loads (global_load_lds_dwordx4) that never
// pass through registers.  The two operands have separate rings: the row
// tile (shared by the workgroups of an expert, so mostly an L2 hit) SA
// stages, SA - 1 slices ahead; the weight tile (read once from HBM) SB
// stages, SB - 1 slices ahead.  One wave instruction fills 8 tile rows (1 KB of LDS,
// contiguous); each lane fetches the global chunk that the swizzle puts at
// its LDS slot.  Row groups wholly past the segment end are not loaded.  Each
// wave waits (vmcnt) only for its own loads of the slice about to be used,
// then one barrier makes the whole slice visible.
template <bool BF16, int BM, int BN, int WM, int WN, bool SWIGLU, int SA, int SB, bool SAVE = false>
__global__ __launch_bounds__(WM *WN * 64) void k_grouped_gemm(
    const u32x4 *__restrict__ A, int M, int kvec, const int32_t *__restrict__ offsets, int G,
    const u32x4 *__restrict__ B, int64_t b_expert_vec, int64_t b_up_vec, int ntiles, int N,
    void *__restrict__ C, const int32_t *__restrict__ gather, int gk, int a_rows,
    void *__restrict__ GU) {
  constexpr int NW = WM * WN;
  constexpr int BR = SWIGLU ? 2 * BN : BN;      // weight rows per tile
  // Row-tile loaders, weight-tile loaders.  A 32-row tile is 4 loads per
  // slice, which one wave issues; the other waves then share the weight
  // stream (decode's gate/up product: 2.44 -> 2.19 ms with 3 weight loaders
  // instead of 2).
  constexpr int NWA = BM <= 32 ? 1 : NW / 2, NWB = NW - NWA;
  constexpr int A_TOT = BM / 8, B_TOT = BR / 8;  // 8-row groups per slice
  constexpr int A_PW = (A_TOT + NWA - 1) / NWA, B_PW = (B_TOT + NWB - 1) / NWB;
  constexpr int MAXLD = A_PW > B_PW ? A_PW : B_PW;
  constexpr int FM = BM / 32 / WM;              // row blocks per wave
  constexpr int WNR = BN / WN, FN = WNR / 32;   // columns, column blocks per wave
  constexpr int NB = SWIGLU ? 2 * FN : FN;      // B fragments (gate, then up) per k-group
  constexpr int ASTAGE = BM * 8, BSTAGE = BR * 8;   // 16-byte chunks per stage
  static_assert(NWA >= 1 && NWB >= 1 && BM % 8 == 0 && BR % 8 == 0, "tile / wave mismatch");
  static_assert(FM * WM * 32 == BM && FN >= 1, "wave tile");
  static_assert(SA >= 2 && SB >= 2 && (SA - 2) * A_PW < 64 && (SB - 2) * B_PW < 64, "rings");

  __shared__ u32x4 smem[SA * ASTAGE + SB * BSTAGE];
  u32x4 *const a_ring = smem;
  u32x4 *const b_ring = smem + SA * ASTAGE;

  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  // DMA lane mapping: lane l fills row l / 8 of its 8-row group, LDS slot
  // l % 8, which holds global chunk (l % 8) ^ key(row).
  const int ld_row = lane >> 3;
  const int ld_slot = lane & 7;
  const int KT = kvec / 8;
  const bool a_loader = wave < NWA;
  const int lw = a_loader ? wave : wave - NWA;
  const int lstride = a_loader ? NWA : NWB;
  const int S = a_loader ? SA : SB;   // stages of this wave's ring

  const int xcd = blockIdx.x % kXcds, nj = gridDim.x / kXcds;
  const int total = count_tiles<BM>(offsets, G, M, ntiles);
  const int band_end = (int)((int64_t)total * (xcd + 1) / kXcds);

  int cur_e = 0, cur_base = 0;   // search cursor of find_tile
  for (int L = (int)((int64_t)total * xcd / kXcds) + (int)(blockIdx.x / kXcds); L < band_end;
       L += nj) {
    Tile tile;
    find_tile<BM>(offsets, G, M, ntiles, L, tile, cur_e, cur_base);
    const int m0 = tile.m0, hi = tile.hi, n0 = tile.n_tile * BN;
    const int rows = hi - m0 < BM ? hi - m0 : BM;   // live rows of this tile

    // DMA roles: waves 0 .. NWA-1 load the row tile, the other waves the
    // weight tile, so each wave's vmcnt queue holds one operand's loads only
    // and a weight slice issued SB - 1 steps ahead never holds up a row slice.
    // Loader lw of an operand fills its 8-row groups lw, lw + stride, ...; a
    // row group is loaded only if its first row is live, and its rows past
    // the segment end re-read the last row (their results are never stored).
    const int ngroups = a_loader ? ((rows + 7) / 8 < A_TOT ? (rows + 7) / 8 : A_TOT) : B_TOT;
    const int nld = ngroups > lw ? (ngroups - lw + lstride - 1) / lstride : 0;
    // Uniform base pointer plus a 32-bit per-lane chunk offset (the host
    // checks that every offset fits), so the loads use the scalar-base form.
    const u32x4 *lbase = a_loader ? A : B + (int64_t)tile.expert * b_expert_vec;
    // Row loaders: the source row of each of their groups, found once per
    // tile (with gather, packed row p is row gather[p] / gk of A, clamped to
    // A's a_rows rows).
    uint32_t arow[A_PW];
    if (a_loader) {
#pragma unroll
      for (int r = 0; r < A_PW; ++r) {
        int row = m0 + (lw + r * lstride) * 8 + ld_row;
        row = row < hi ? row : hi - 1;
        arow[r] = gather ? gather_row(gather, row, gk, a_rows) : (uint32_t)row;
      }
    }
    auto issue = [&](int kt) {
      u32x4 *stage = a_loader ? a_ring + (kt % SA) * ASTAGE : b_ring + (kt % SB) * BSTAGE;
      if (a_loader) {
#pragma unroll
        for (int r = 0; r < A_PW; ++r) {
          if (r < nld) {
            const int g = lw + r * lstride;
            const uint32_t key = ld_row ^ (g & 1);   // swz_key(8 g + ld_row)
            const uint32_t off = arow[r] * (uint32_t)kvec + (uint32_t)kt * 8u + ((uint32_t)ld_slot ^ key);
            __builtin_amdgcn_global_load_lds(
                (const void *)(lbase + off),
                (__attribute__((address_space(3))) void *)(stage + g * 64), 16, 0, 0);
          }
        }
        return;
      }
      // A rolled loop: unrolled, the per-instruction offsets would be hoisted
      // out of the K loop and held in registers the MFMA blocks need.
#pragma unroll 1
      for (int r = 0; r < nld; ++r) {
        const int g = lw + r * lstride;
        const uint32_t key = ld_row ^ (g & 1);   // swz_key(8 g + ld_row)
        const int brow = g * 8 + ld_row;
        uint32_t off = SWIGLU && brow >= BN ? (uint32_t)b_up_vec + (uint32_t)(n0 + brow - BN) * kvec
                                            : (uint32_t)(n0 + brow) * (uint32_t)kvec;
        off += (uint32_t)kt * 8u + ((uint32_t)ld_slot ^ key);
        // Non-temporal: few rows per expert stream each weight byte past once
        // (decode's down product: 1.27 -> 1.16 ms at 128 tokens x top-8).
        __builtin_amdgcn_global_load_lds(
            (const void *)(lbase + off),
            (__attribute__((address_space(3))) void *)(stage + g * 64), 16, 0, kNonTemporal);
      }
    };

    // Row blocks of this wave that hold at least one live row: blocks
    // wm, wm + WM, ... below ceil(rows / 32).
    const int nblk = (rows + 31) / 32;
    int live = (nblk - wm + WM - 1) / WM;
    live = live < 0 ? 0 : (live > FM ? FM : live);

    f32x16 acc[FM][NB];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // Prologue: each loader issues slices 0 .. S-2 of its ring; step j then
    // issues slice j + S - 1.  At step kt the slices after kt that are
    // already issued (up to S - 2 of them) may stay in flight.
#pragma unroll
    for (int s = 0; s < (SA > SB ? SA : SB) - 1; ++s)
      if (s < S - 1 && s < KT) issue(s);

    // The K loop, instantiated twice: FULL (every row block of this wave is
    // live, the common case) issues all MFMAs unconditionally; the other
    // variant skips dead blocks.  Fragments of k-group q + 1 are read from
    // LDS while the MFMAs of k-group q run.
    auto kloop = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      for (int kt = 0; kt < KT; ++kt) {
        // This wave's loads of slice kt are done once no more than its loads
        // of later slices remain in flight.
        asm volatile("" ::: "memory");
        wait_vmcnt(((kt + S - 2 < KT - 1 ? kt + S - 2 : KT - 1) - kt) * nld);
        // Every wave's part of slice kt has landed, and every wave is done
        // with the stages that row slice kt + SA - 1 and weight slice
        // kt + SB - 1 overwrite (both were read in step kt - 1).
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");

        const u32x4 *As = a_ring + (kt % SA) * ASTAGE;
        const u32x4 *Bs = b_ring + (kt % SB) * BSTAGE;
        u32x4 fa[2][FM], fb[2][NB];
        auto fetch = [&](int q, int buf) {
          const int cc = 2 * q + (lane >> 5);
#pragma unroll
          for (int i = 0; i < FM; ++i)
            if (FULL || i < live) fa[buf][i] = As[swz((wm + i * WM) * 32 + (lane & 31), cc)];
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            fb[buf][j] = Bs[swz(wn * WNR + j * 32 + (lane & 31), cc)];
            if (SWIGLU) fb[buf][FN + j] = Bs[swz(BN + wn * WNR + j * 32 + (lane & 31), cc)];
          }
        };
        fetch(0, 0);
        if (kt + S - 1 < KT) issue(kt + S - 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < 3) fetch(q + 1, (q + 1) & 1);
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            if (FULL || i < live) {
#pragma unroll
              for (int j = 0; j < NB; ++j) Mma<BF16>::run(fa[q & 1][i], fb[q & 1][j], acc[i][j]);
            }
          }
        }
      }
    };
    if (live == FM)
      kloop(std::true_type{});
    else
      kloop(std::false_type{});

    // All waves are done reading LDS before the next tile's loads land in it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // Epilogue.  MFMA 32x32 output layout: lane l holds column l % 32 and, in
    // register v, row 8 (v / 4) + 4 (l / 32) + v % 4.
    const int col_l = lane & 31, row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= live) continue;
      const int rblk = m0 + (wm + i * WM) * 32;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WNR + j * 32 + col_l;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = rblk + 8 * (v >> 2) + row_l + (v & 3);
          if (row < hi) {
            const float val = SWIGLU ? silu(acc[i][j][v]) * acc[i][FN + j][v] : acc[i][j][v];
            const int64_t idx = (int64_t)row * N + col;
            if (BF16)
              static_cast<uint16_t *>(C)[idx] = (uint16_t)f32_to_bf16_rne(val);
            else
              static_cast<float *>(C)[idx] = val;
            if constexpr (SAVE && SWIGLU) {
              // Pre-activations for the backward: gate at column col, up at
              // N + col of a [M, 2 N] row.
              const int64_t g = (int64_t)row * 2 * N + col;
              if (BF16) {
                static_cast<uint16_t *>(GU)[g] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
                static_cast<uint16_t *>(GU)[g + N] = (uint16_t)f32_to_bf16_rne(acc[i][FN + j][v]);
              } else {
                static_cast<float *>(GU)[g] = acc[i][j][v];
                static_cast<float *>(GU)[g + N] = acc[i][FN + j][v];
              }
            }
          }
        }
      }
    }
  }
}

// Ping-pong variant for tiles with many rows: 8 waves, two per SIMD, in two
// groups of 4.  The tile is up to BM rows x BR weight rows (SWIGLU: BR/2 gate
// rows then the matching BR/2 up rows, i.e. BR/2 columns of h; otherwise BR
// output columns).  Inside a group, wave (wm, wn) of WMG x WNG owns weight
// rows [64 wn, 64 wn + 64) -- for SWIGLU 32 gate rows and their 32 up rows --
// and the row blocks (32 rows each) g + 2 (wm + WMG i) of its group g.
//
// The two groups run the same program half a phase apart: every two k-groups
// (64 bytes of K) are a memory phase (LDS -> registers and issuing loads) and
// a compute phase (MFMAs from registers), each closed by a barrier.  Group 1
// starts one barrier late, so while one group issues MFMAs the other works
// on memory, and the matrix cores of each SIMD stay busy.  A memory phase
// need not wait for its LDS reads: they finish under the wave's next compute
// phase while the other group's reads already queue, which keeps the LDS
// busy across the barrier.
//
// K is staged in slices of 16 CPR bytes per row (CPR = 8: 128 bytes, two
// phase pairs per slice; CPR = 4: 64 bytes, one).  Narrow slices make the
// ring stages small, so more of them fit: the weight tile, streamed from HBM,
// can then be requested several phases before it is read.  Direct
// global-to-LDS loads (one wave instruction = 1 KB = 64 / CPR rows); group 0
// loads the row tile into a ring of SA stages, DA slices ahead, group 1
// the weight tile into a ring of SB stages, SB - 1 slices ahead, so each
// wave's vmcnt queue holds one operand.  A slice is visible to every wave
// after the first barrier that follows all its loaders' waits: group 0 waits
// for row slice k + 1 at the end of its last compute phase of slice k, group
// 1 for weight slice k + 1 at the end of its last memory phase of slice k --
// both right before the barrier after which group 0 reads slice k + 1.  A
// stage is refilled only after both groups' last reads of it.

template <int CPR>
__device__ __forceinline__ int swz_c(int r, int cc) {
  if constexpr (CPR == 8)
    return swz(r, cc);
  else
    return r * 4 + (cc ^ ((r >> 2) & 3));   // 16 consecutive rows at one chunk: all banks once
}

// VAR selects the product: 0 the forward's (weights K-contiguous, [N, K]
// per expert); 1 and 2 a backward input-gradient product, whose weights are
// [K, N] per expert (N-contiguous) and are staged as column-contiguous tiles
// read back transposed -- 1 stores the product, 2 is the down product's
// backward, whose epilogue applies the SwiGLU backward with the forward's
// pre-activations GU ([M, 2 N]) and writes dgu ([M, 2 N]) to C.  4 is 1
// adding the product to C.  (The weight gradients run on their own kernel,
// grouped_wgrad.hip.)
template <bool BF16, int BM, int BR, int SA, int SB, int CPR, int DA, bool SWIGLU, bool SPLIT,
          bool SAVE = false, int VAR = 0>
__global__ __launch_bounds__(512) void k_grouped_gemm_pp(
    const u32x4 *__restrict__ A, int M, int kvec, const int32_t *__restrict__ offsets, int G,
    const u32x4 *__restrict__ B, int64_t b_expert_vec, int64_t b_up_vec, int ntiles, int N,
    void *__restrict__ C, const int32_t *__restrict__ gather, int gk, int a_rows,
    void *__restrict__ GU) {
  constexpr int BN = SWIGLU ? BR / 2 : BR;       // output columns per tile
  constexpr int WNG = BR / 64, WMG = 4 / WNG;    // waves of a group across N and M
  constexpr int FM = (BM / 64 + WMG - 1) / WMG;  // row blocks per wave
  constexpr int NB = 2;                          // B fragments per k-group
  constexpr int NH = CPR / 4;                    // phase pairs per slice
  constexpr int RPI = 64 / CPR;                  // rows per DMA instruction
  constexpr int ASTAGE = BM * CPR, BSTAGE = BR * CPR;   // 16-byte chunks per stage
  constexpr int A_TOT = BM / RPI, B_TOT = BR / RPI;     // DMA groups per slice
  constexpr int NLB = B_TOT / 4;                 // weight loads per group-1 wave per slice
  static_assert(CPR == 4 || CPR == 8, "slice width");
  static_assert(BM % 64 == 0 && BM % RPI == 0 && (BR == 128 || BR == 256) && B_TOT % 4 == 0, "tile");
  static_assert(SA >= 2 && SB >= 2 && DA >= 1 && DA <= SA - 1, "rings");
  static_assert((SA * ASTAGE + SB * BSTAGE) * 16 <= 160 * 1024, "LDS");
  static_assert(NLB * (SB - 2) < 64 && ((A_TOT + 3) / 4) * (DA - 1) < 64, "vmcnt");
  // A memory phase ends with its LDS reads still in flight (they complete
  // under the next compute phase) unless a stage they read may be refilled
  // in the very next phase: group 0 refills the row stage of slice
  // kt + DA - SA at its first memory phase of slice kt, one phase after
  // group 1's last read of slice kt - 1.  With DA = SA - 1 that is the same
  // stage, so group 1 drains its reads at its last memory phase of a slice.
  // Every other refill targets a stage whose last reads were consumed by
  // MFMAs at least one phase earlier.
  constexpr bool kDrainLast = DA == SA - 1;
  static_assert(FM <= 5, "row blocks per wave");
  static_assert(VAR == 0 || (BF16 && !SWIGLU && !SAVE), "backward products: bf16, plain tiles");
  constexpr bool BT = VAR != 0;                  // B [K, N]: column-contiguous stages
  // The forward's plain product (the down product, bf16) stores through
  // LDS as whole 128-byte lines (STG); its MFMAs take the weight fragment
  // first, so each 32 x 32 block holds the transposed output.
  constexpr bool STG = BF16 && VAR == 0 && !SAVE && !SWIGLU;
  constexpr bool kStoreNT = true;
  // The forward's SwiGLU product (bf16) stores h, and with SAVE the
  // pre-activations, through LDS too (STGH), as 64-byte row segments.
  constexpr bool STGH = BF16 && VAR == 0 && SWIGLU;

  __shared__ u32x4 smem[SA * ASTAGE + SB * BSTAGE];
  u32x4 *const a_ring = smem;
  u32x4 *const b_ring = smem + SA * ASTAGE;

  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int grp = wave >> 2, wq = wave & 3;
  const int wn = wq % WNG, wm = wq / WNG;
  // DMA lane mapping: lane l fills row l / CPR of its group, LDS slot l % CPR,
  // which holds global chunk (l % CPR) ^ key(row); the key of a group's rows
  // depends on the group only through its parity (CPR = 8) or not at all.
  const int ld_row = lane / CPR, ld_slot = lane % CPR;
  const int KT_all = kvec / CPR;   // slices per tile (forward and input-gradient products)

  const int xcd = blockIdx.x % kXcds, nj = gridDim.x / kXcds;
  const int total = count_tiles<BM>(offsets, G, M, ntiles);
  const int band_end = (int)((int64_t)total * (xcd + 1) / kXcds);
  const int L0 = (int)((int64_t)total * xcd / kXcds) + (int)(blockIdx.x / kXcds);
  const int Lstep = nj;

  int cur_e = 0, cur_base = 0;   // search cursor of find_tile
  for (int L = L0; L < band_end;
       L += Lstep) {
    Tile tile;
    find_tile<BM>(offsets, G, M, ntiles, L, tile, cur_e, cur_base);
    const int m0 = tile.m0, hi = tile.hi, n0 = tile.n_tile * BN;
    const int rows = hi - m0 < BM ? hi - m0 : BM;
    const int KT = KT_all;
    const int nblk = (rows + 31) / 32;
    // Row blocks g + 2 (wm + WMG i) below nblk.
    int live = (nblk - grp - 2 * wm + 2 * WMG - 1) / (2 * WMG);
    live = live < 0 ? 0 : (live > FM ? FM : live);

    // Group 0: row groups wq, wq + 4, ... whose first row is live (rows past
    // the segment end re-read its last row; their results are never stored);
    // na of them per slice.  Group 1: weight groups wq, wq + 4, ...
    const int a_groups = (rows + RPI - 1) / RPI < A_TOT ? (rows + RPI - 1) / RPI : A_TOT;
    const int na = a_groups > wq ? (a_groups - wq + 3) / 4 : 0;
    auto key_of = [&](int g) -> uint32_t {
      return CPR == 8 ? (uint32_t)(ld_row ^ (g & 1)) : (uint32_t)((ld_row >> 2) & 3);
    };
    // Buffer-to-LDS loads: a resource per operand tile (the row tile from row
    // m0, the expert's weights), a per-lane 32-bit byte offset fixed for the
    // tile, and the K position as the scalar offset -- a K step costs no
    // address arithmetic.
    constexpr int NLA = (A_TOT + 3) / 4;           // row loads per group-0 wave per slice, at most
    // Without gather the resource starts at the tile's first row; with
    // gather (packed row p is row gather[p] / gk of A) it spans A's a_rows rows.
    const u32x4 *a_base = gather ? A : A + (int64_t)m0 * kvec;
    const uint32_t a_bytes = (uint32_t)((int64_t)(gather ? a_rows : rows) * kvec * 16);
    const u32x4 *b_base = B + (int64_t)tile.expert * b_expert_vec;
    const uint32_t b_bytes = (uint32_t)(b_expert_vec * 16);
    auto a_offsets = [&](uint32_t (&off)[NLA]) {
#pragma unroll
      for (int r = 0; r < NLA; ++r) {
        const int g = wq + 4 * r;
        int row = g * RPI + ld_row;
        row = row < rows ? row : rows - 1;
        const uint32_t src = gather ? gather_row(gather, m0 + row, gk, a_rows) : (uint32_t)row;
        off[r] = (src * (uint32_t)kvec + ((uint32_t)ld_slot ^ key_of(g))) * 16u;
      }
    };
    auto b_offsets = [&](uint32_t (&off)[NLB]) {
#pragma unroll
      for (int r = 0; r < NLB; ++r) {
        const int g = wq + 4 * r;
        if constexpr (BT) {
          // K-row krow of the slice, columns n0 + col .. + 7 of the [K, N]
          // matrix; the slice's K position is the scalar offset.
          int krow, col;
          cc_lane<BR>(g, lane, krow, col);
          off[r] = ((uint32_t)krow * (uint32_t)N + (uint32_t)(n0 + col)) * 2u;
        } else {
          const int brow = g * RPI + ld_row;
          off[r] = ((SWIGLU && brow >= BN ? (uint32_t)b_up_vec + (uint32_t)(n0 + brow - BN) * kvec
                                          : (uint32_t)(n0 + brow) * (uint32_t)kvec) +
                    ((uint32_t)ld_slot ^ key_of(g))) * 16u;
        }
      }
    };
    // Bytes from one K slice to the next in the weight tile.
    const uint32_t b_step = BT ? (uint32_t)(CPR * 8) * (uint32_t)N * 2u : (uint32_t)CPR * 16u;
    auto issue_a = [&](int kt, const uint32_t (&off)[NLA]) {
      u32x4 *stage = a_ring + (kt % SA) * ASTAGE;
#pragma unroll
      for (int r = 0; r < NLA; ++r)
        if (r < na) buffer_load_lds16(a_base, a_bytes, stage + (wq + 4 * r) * 64, off[r], kt * CPR * 16);
    };
    // The input-gradient products read their weights non-temporally (2-3%
    // faster); for the forward products that policy measured 20% slower.
    constexpr int kWeightPolicy = VAR == 0 ? 0 : kNonTemporal;
    auto issue_b = [&](int kt, const uint32_t (&off)[NLB]) {
      u32x4 *stage = b_ring + (kt % SB) * BSTAGE;
#pragma unroll
      for (int r = 0; r < NLB; ++r)
        buffer_load_lds16<kWeightPolicy>(b_base, b_bytes, stage + (wq + 4 * r) * 64, off[r],
                                         (uint32_t)kt * b_step);
    };
    // Waits for slice k of this wave's operand: the slices after it that are
    // already issued (up to k + SB - 2, or k + DA - 1 for the row tile) may
    // stay in flight.
    auto wait_b = [&](int k) {
      constexpr int kSteady = (SB - 2) * NLB;
      if (k + SB - 2 <= KT - 1)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kSteady & 15) | ((kSteady >> 4) << 14));
      else
        wait_vmcnt((KT - 1 - k) * NLB);
    };
    auto wait_a = [&](int k) {
      const int last = k + DA - 1 < KT - 1 ? k + DA - 1 : KT - 1;
      if constexpr (DA > 1 && VAR != 1) {
        // A run-time count becomes a search over the wait's immediate forms,
        // a dozen scalar branches per slice; the usual cases -- a full slice
        // ahead, with all of this wave's row groups (na = NLA) or one fewer --
        // take an immediate.  (Measured: 0.5-2% faster for the forward
        // products and the down product's backward, but 14% slower for the
        // first product's input gradient, which therefore keeps the search.)
        constexpr int kFull = (DA - 1) * NLA, kLess = (DA - 1) * (NLA - 1);
        if (last == k + DA - 1 && na == NLA) {
          __builtin_amdgcn_s_waitcnt(0x0F70 | (kFull & 15) | ((kFull >> 4) << 14));
          return;
        }
        if (last == k + DA - 1 && na == NLA - 1) {
          __builtin_amdgcn_s_waitcnt(0x0F70 | (kLess & 15) | ((kLess >> 4) << 14));
          return;
        }
      }
      wait_vmcnt((last - k) * na);
    };

    // The rest of the tile.  SPLIT: instantiated per number of live row
    // blocks NL of this wave (the waves of a tile may differ), so the MFMA
    // and epilogue code has no per-block branches -- for tiles that are
    // often partly live.  Otherwise one body skips dead blocks at run time.
    auto run_tile = [&](auto nl_tag, auto dyn_tag, auto grp_tag) {
    constexpr int GRP = decltype(grp_tag)::value;   // this wave's group, as a constant
    constexpr int NL = decltype(nl_tag)::value;
    constexpr bool DYN = decltype(dyn_tag)::value;   // NL = FM, blocks below live only
    constexpr int NLM = NL > 0 ? NL : 1;
    f32x16 acc[NLM][NB];
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // Slices 0 .. DA - 1 (row tile) or 0 .. SB - 2 (weight tile) of this
    // wave's operand, wait for slice 0, then group 1 starts one barrier late.
    uint32_t off[GRP == 0 ? NLA : NLB];
    if constexpr (GRP == 0)
      a_offsets(off);
    else
      b_offsets(off);
    asm volatile("" ::: "memory");
    if constexpr (GRP == 0) {
#pragma unroll
      for (int s = 0; s < DA; ++s)
        if (s < KT) issue_a(s, off);
      asm volatile("" ::: "memory");
      wait_a(0);
    } else {
#pragma unroll
      for (int s = 0; s < SB - 1; ++s)
        if (s < KT) issue_b(s, off);
      asm volatile("" ::: "memory");
      wait_b(0);
    }
    asm volatile("" ::: "memory");
    phase_barrier();
    asm volatile("" ::: "memory");
    if (GRP == 1) phase_barrier();
    asm volatile("" ::: "memory");

    // B fragment rows of this wave inside the weight tile.
    const int brow0 = SWIGLU ? wn * 32 : wn * 64;
    const int brow1 = SWIGLU ? BN + wn * 32 : wn * 64 + 32;

    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        // Memory phase.  The weight fragments are read first: the compute
        // phase's first MFMAs need them and one row fragment.  (The compiler
        // orders these loads after the previous phase's MFMAs that read the
        // same registers.)
        const u32x4 *As = a_ring + (kt % SA) * ASTAGE;
        const u32x4 *Bs = b_ring + (kt % SB) * BSTAGE;
        u32x4 fa[2][NLM], fb[2][NB];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int cc = 2 * (2 * h + q) + (lane >> 5);
          if constexpr (BT) {
            const char *bsb = reinterpret_cast<const char *>(Bs);
            fb[q][0] = frag_tr<BR>(bsb, brow0 / 32, 2 * h + q, lane);
            fb[q][1] = frag_tr<BR>(bsb, brow1 / 32, 2 * h + q, lane);
          } else {
            fb[q][0] = Bs[swz_c<CPR>(brow0 + (lane & 31), cc)];
            fb[q][1] = Bs[swz_c<CPR>(brow1 + (lane & 31), cc)];
          }
#pragma unroll
          for (int i = 0; i < NL; ++i)
            if (!DYN || i < live)
              fa[q][i] = As[swz_c<CPR>((GRP + 2 * (wm + WMG * i)) * 32 + (lane & 31), cc)];
        }
        if (h == 0) {
          if constexpr (GRP == 0) {
            if (kt + DA < KT) issue_a(kt + DA, off);
          } else {
            if (kt + SB - 1 < KT) issue_b(kt + SB - 1, off);
          }
        }
        asm volatile("" ::: "memory");
        if (GRP == 1 && kDrainLast && h == NH - 1)
          __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0): reads done before the barrier
        // Group 0 reads slice kt + 1 right after the next barrier but one.
        if (GRP == 1 && h == NH - 1 && kt + 1 < KT) wait_b(kt + 1);
        asm volatile("" ::: "memory");
        phase_barrier();
        asm volatile("" ::: "memory");
        // Compute phase.
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int i = 0; i < NL; ++i)
            if (!DYN || i < live)
#pragma unroll
              for (int j = 0; j < NB; ++j) {
                if constexpr (STG || STGH)
                  Mma<BF16>::run(fb[q][j], fa[q][i], acc[i][j]);
                else
                  Mma<BF16>::run(fa[q][i], fb[q][j], acc[i][j]);
              }
        asm volatile("" ::: "memory");
        if (GRP == 0 && h == NH - 1 && kt + 1 < KT) wait_a(kt + 1);
        asm volatile("" ::: "memory");
        phase_barrier();
        asm volatile("" ::: "memory");
      }
    }
    if (GRP == 0) phase_barrier();   // both groups leave the tile aligned
    asm volatile("" ::: "memory");

    if constexpr (STG) {
      // Epilogue through LDS.  Each block holds the transpose: lane l holds
      // output row l % 32 and, in register v, column 8 (v / 4) + 4 (l / 32) +
      // v % 4 of the block -- registers 4 a .. 4 a + 3 are four consecutive
      // columns of one row, one 8-byte bf16 word.  A 32-row block of the
      // wave (64 columns) goes to 4 KB of staging row-major: 16-byte chunk c
      // of row r at c ^ (r % 8), its 8-byte halves swapped when bit 3 of r
      // is set -- the 16 lanes of a write (16 rows of one half-chunk) then
      // fill 16 different 8-byte bank slots.  Each lane reads 16 bytes of
      // one row back (8 lanes per row), swaps the halves back in rows with
      // bit 3 set, and stores them: 8 whole 128-byte rows per instruction,
      // rows past the segment end left out.  The staging is in row stages
      // DA .. SA - 1: the K loop's reads of them are done at the barrier
      // that closes the tile, the next tile's first loads fill stages below
      // DA, and stage DA is refilled only after the next tile's first
      // barrier, which every wave reaches after its epilogue's reads.
      static_assert((SA - DA) * ASTAGE * 16 >= 8 * 4096, "epilogue staging");
      char *const stg = reinterpret_cast<char *>(a_ring + DA * ASTAGE) + wave * 4096;
      const uint64_t cb = reinterpret_cast<uint64_t>(static_cast<uint16_t *>(C) + (int64_t)m0 * N);
      const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<void *>(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(cb >> 32)) << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)cb)),
          (short)0, 0x7FFFFFFF, kBufferFlags);
      const int wrow = lane & 31, whalf = lane >> 5;   // write side: row, 8-byte half of a chunk
      const int rrow = lane >> 3, rch = lane & 7;      // read side: row (of 8), chunk
      const uint32_t vout = ((uint32_t)rrow * (uint32_t)N + (uint32_t)(n0 + wn * 64 + 8 * rch)) * 2u;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if (DYN && i >= live) continue;
        const int rb = GRP + 2 * (wm + WMG * i);
#pragma unroll
        for (int j = 0; j < NB; ++j)
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
          q[u] = (u & 1) == 0 ? v : u32x4{v[2], v[3], v[0], v[1]};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (m0 + 32 * rb + 8 * u + rrow < hi)
            __builtin_amdgcn_raw_buffer_store_b128(q[u], out_rsrc, vout,
                                                   (uint32_t)(32 * rb + 8 * u) * (uint32_t)N * 2u,
                                                   kStoreNT ? 2 : 0);
      }
      return;
    }

    if constexpr (STGH) {
      // Epilogue through LDS for the SwiGLU product: a wave's 32 output
      // columns of a 32-row block are 64 bytes per row.  As above, lane l
      // holds row l % 32 and registers 4 a .. 4 a + 3 hold columns 8 a +
      // 4 (l / 32) .. + 3.  Staging rows are 64 bytes: 16-byte chunk c of row
      // r sits at c ^ ((r / 2) % 4), its halves swapped when bit 3 of r is
      // set, so the 16 lanes of an 8-byte write (16 rows) fill 16 different
      // 8-byte slots of 128 bytes.  Each lane reads 16 bytes back (4 lanes
      // per row, 16 rows per read: 256 contiguous bytes) and stores them:
      // 16 row segments of 64 bytes per instruction, the other half of each
      // 128-byte line coming from the neighbouring wave, so these are plain
      // stores that meet in the L2.  Same staging place and lifetime as the
      // plain product's.
      static_assert((SA - DA) * ASTAGE * 16 >= 8 * 2048, "epilogue staging");
      char *const stg = reinterpret_cast<char *>(a_ring + DA * ASTAGE) + wave * 2048;
      const int wrow = lane & 31, whalf = lane >> 5;
      const int rrow = lane >> 2, rch = lane & 3;      // read side: row (of 16), logical chunk
      const int pch = rch ^ ((rrow >> 1) & 3);         // its place in the staging row
      const bool rswap = (rrow >> 3) & 1;
      // Buffer resource from row m0 of a row-major [*, ld] bf16 matrix.
      auto rsrc_at = [&](void *base, int64_t ld) {
        const uint64_t cb = reinterpret_cast<uint64_t>(static_cast<uint16_t *>(base) + (int64_t)m0 * ld);
        return __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void *>(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(cb >> 32)) << 32) |
                                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)cb)),
            (short)0, 0x7FFFFFFF, kBufferFlags);
      };
      // One 32 x 32 block of this lane's 16 values to rows 32 rb .. + 31 of
      // the tile, columns col .. col + 31 of a matrix of pitch ld.
      auto put_block = [&](__amdgpu_buffer_rsrc_t rsrc, uint32_t ld, int col, int rb, const float(&val)[16]) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 pk = {(__bf16)val[4 * a], (__bf16)val[4 * a + 1], (__bf16)val[4 * a + 2],
                             (__bf16)val[4 * a + 3]};
          const int chunk = a ^ ((wrow >> 1) & 3);
          const int half = whalf ^ ((wrow >> 3) & 1);
          *reinterpret_cast<u32x2 *>(stg + wrow * 64 + chunk * 16 + half * 8) = __builtin_bit_cast(u32x2, pk);
        }
        u32x4 q[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + (16 * u + rrow) * 64 + pch * 16);
          q[u] = rswap ? u32x4{v[2], v[3], v[0], v[1]} : v;
        }
        const uint32_t vout = ((uint32_t)rrow * ld + (uint32_t)(col + 8 * rch)) * 2u;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (m0 + 32 * rb + 16 * u + rrow < hi)
            __builtin_amdgcn_raw_buffer_store_b128(q[u], rsrc, vout, (uint32_t)(32 * rb + 16 * u) * ld * 2u, 0);
      };
      const __amdgpu_buffer_rsrc_t h_rsrc = rsrc_at(C, N);
      const int col = n0 + wn * 32;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if (DYN && i >= live) continue;
        const int rb = GRP + 2 * (wm + WMG * i);
        float val[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) val[v] = silu(acc[i][0][v]) * acc[i][1][v];
        put_block(h_rsrc, (uint32_t)N, col, rb, val);
        if constexpr (SAVE) {
          // Pre-activations for the backward: gate at column col, up at
          // N + col of a [M, 2 N] row.
          const __amdgpu_buffer_rsrc_t gu_rsrc = rsrc_at(GU, 2 * (int64_t)N);
          float g[16], u[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            g[v] = acc[i][0][v];
            u[v] = acc[i][1][v];
          }
          put_block(gu_rsrc, 2u * (uint32_t)N, col, rb, g);
          put_block(gu_rsrc, 2u * (uint32_t)N, N + col, rb, u);
        }
      }
      return;
    }

    // Epilogue.  MFMA 32x32 output layout: lane l holds column l % 32 and, in
    // register v, row 8 (v / 4) + 4 (l / 32) + v % 4.  bf16 output: adjacent
    // lanes (columns c, c + 1) trade values so each holds two columns of one
    // row, and one 4-byte store writes the pair -- even lanes rows t = 0, 2 of
    // each group of four rows, odd lanes rows t = 1, 3.
    const int col_l = lane & 31, row_l = 4 * (lane >> 5);
    const bool odd = lane & 1;
    // Stores one 32 x 32 block (this lane's 16 values) at column col of the
    // row-major [*, ld] output dst.
    auto put = [&](void *dst, int64_t ld, int rblk, int col, const float(&val)[16]) {
      if constexpr (BF16) {
        uint32_t *out = static_cast<uint32_t *>(dst);
        const int c0 = col & ~1;
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          // Rows t = v % 4 (even lanes keep it) and t + 1 (odd lanes).
          const float mine = odd ? val[v + 1] : val[v];
          const float give = odd ? val[v] : val[v + 1];
          const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0xB1, 0xF, 0xF, false));
          const float lo = odd ? got : mine, hi2 = odd ? mine : got;   // columns c0, c0 + 1
          const int row = rblk + 8 * (v >> 2) + row_l + (v & 3) + (odd ? 1 : 0);
          if (row < hi) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 pk = {(__bf16)lo, (__bf16)hi2};
            out[((int64_t)row * ld + c0) >> 1] = __builtin_bit_cast(uint32_t, pk);
          }
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = rblk + 8 * (v >> 2) + row_l + (v & 3);
          if (row < hi) static_cast<float *>(dst)[(int64_t)row * ld + col] = val[v];
        }
      }
    };
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (DYN && i >= live) continue;
      const int rblk = m0 + (GRP + 2 * (wm + WMG * i)) * 32;
#pragma unroll
      for (int j = 0; j < (SWIGLU ? 1 : 2); ++j) {
        const int col = n0 + (SWIGLU ? wn * 32 : wn * 64 + j * 32) + col_l;
        float val[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) val[v] = SWIGLU ? silu(acc[i][0][v]) * acc[i][1][v] : acc[i][j][v];
        if constexpr (VAR == 2) {
          // dh -> (dgate, dup) through h = SiLU(g) u:
          //   dgate = dh u SiLU'(g), dup = dh SiLU(g),
          //   SiLU'(g) = s (1 + g (1 - s)), s = 1 / (1 + e^-g).
          // Adjacent lanes trade values so each holds two adjacent columns of
          // one row, read as one 4-byte pair of g and of u.
          const int c0 = col & ~1;
          const uint16_t *gu = static_cast<const uint16_t *>(GU);
          uint16_t *out = static_cast<uint16_t *>(C);
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            const float mine = odd ? val[v + 1] : val[v];
            const float give = odd ? val[v] : val[v + 1];
            const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0xB1, 0xF, 0xF, false));
            const float dh[2] = {odd ? got : mine, odd ? mine : got};   // columns c0, c0 + 1
            const int row = rblk + 8 * (v >> 2) + row_l + (v & 3) + (odd ? 1 : 0);
            if (row < hi) {
              const int64_t base = (int64_t)row * 2 * N + c0;
              const uint32_t gg = *reinterpret_cast<const uint32_t *>(gu + base);
              const uint32_t uu = *reinterpret_cast<const uint32_t *>(gu + base + N);
              const float g[2] = {bf16_lo(gg), bf16_hi(gg)}, u[2] = {bf16_lo(uu), bf16_hi(uu)};
              float dg[2], du[2];
#pragma unroll
              for (int c = 0; c < 2; ++c) {
                const float s = sigmoid_f(g[c]);
                dg[c] = dh[c] * u[c] * (s * (1.0f + g[c] * (1.0f - s)));
                du[c] = dh[c] * (g[c] * s);
              }
              *reinterpret_cast<uint32_t *>(out + base) = pack_bf16x2(dg[0], dg[1]);
              *reinterpret_cast<uint32_t *>(out + base + N) = pack_bf16x2(du[0], du[1]);
            }
          }
          continue;
        }
        if constexpr (VAR == 4) {
          // C += product: each lane reads the pair of columns it then writes.
          const int c0 = col & ~1;
          uint32_t *out = static_cast<uint32_t *>(C);
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            const float mine = odd ? val[v + 1] : val[v];
            const float give = odd ? val[v] : val[v + 1];
            const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0xB1, 0xF, 0xF, false));
            const int row = rblk + 8 * (v >> 2) + row_l + (v & 3) + (odd ? 1 : 0);
            if (row < hi) {
              const int64_t at = ((int64_t)row * N + c0) >> 1;
              const uint32_t old = out[at];
              out[at] = pack_bf16x2(bf16_lo(old) + (odd ? got : mine), bf16_hi(old) + (odd ? mine : got));
            }
          }
          continue;
        }
        put(C, N, rblk, col, val);
        if constexpr (SAVE && SWIGLU) {
          // Pre-activations for the backward: gate at column col, up at
          // N + col of a [M, 2 N] row.
          float g[16], u[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            g[v] = acc[i][0][v];
            u[v] = acc[i][1][v];
          }
          put(GU, 2 * (int64_t)N, rblk, col, g);
          put(GU, 2 * (int64_t)N, rblk, N + col, u);
        }
      }
    }
    };
    using Dyn = std::true_type;
    using Fixed = std::false_type;
    auto by_live = [&](auto g) {
      if constexpr (!SPLIT) {
        run_tile(std::integral_constant<int, FM>{}, Dyn{}, g);
      } else {
        switch (live) {
          case 5: if constexpr (FM >= 5) run_tile(std::integral_constant<int, 5>{}, Fixed{}, g); break;
          case 4: if constexpr (FM >= 4) run_tile(std::integral_constant<int, 4>{}, Fixed{}, g); break;
          case 3: if constexpr (FM >= 3) run_tile(std::integral_constant<int, 3>{}, Fixed{}, g); break;
          case 2: if constexpr (FM >= 2) run_tile(std::integral_constant<int, 2>{}, Fixed{}, g); break;
          case 1: run_tile(std::integral_constant<int, 1>{}, Fixed{}, g); break;
          default: run_tile(std::integral_constant<int, 0>{}, Fixed{}, g); break;
        }
      }
    };
    // Each group runs its own copy of the tile code: the loads it issues and
    // the waits it makes are fixed per group, so they need no branches.
    if (grp == 0)
      by_live(std::integral_constant<int, 0>{});
    else
      by_live(std::integral_constant<int, 1>{});
  }
}

// One launch of the grouped GEMM with tile shape Cfg.
template <int BM_, int BN_, int WM_, int WN_, int SA_, int SB_>
struct TileCfg {
  static constexpr bool PP = false;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, SA = SA_, SB = SB_;
};
// Ping-pong kernel: BM-row x BR-weight-row tiles, K slices of 16 CPR bytes,
// SA row-tile and SB weight-tile ring stages; SPLIT: one kernel body per live
// row-block count.
template <int BM_, int BR_, int SA_, int SB_, int CPR_, bool SPLIT_, int DA_>
struct PpCfg {
  static constexpr bool PP = true;
  static constexpr int BM = BM_, BR = BR_, SA = SA_, SB = SB_, CPR = CPR_, DA = DA_;
  static constexpr bool SPLIT = SPLIT_;
};

// gather (optional): packed row p of the product is row gather[p] / gk of a,
// which then has a_rows rows.
// gu (SAVE only): also store the gate and up pre-activations, [M, 2 N].
// grid_rows (optional): the rows the grid is sized for, when the segments
// cover fewer than M rows (one expert of a loop of products).
template <bool BF16, bool SWIGLU, typename Cfg, bool SAVE = false>
void launch_one(const void *a, int M, int K, int N, const int32_t *offsets, int G, const void *w,
                void *out, hipStream_t stream, const int32_t *gather = nullptr, int gk = 1,
                int a_rows = 0, void *gu = nullptr, int grid_rows = -1) {
  const int gm = grid_rows >= 0 ? grid_rows : M;
  const int elem = BF16 ? 2 : 4;
  const int kvec = K * elem / 16;
  // w13 is [G, 2, N, K] (gate rows, then up rows); w2 is [G, N, K].
  const int64_t b_expert = (int64_t)(SWIGLU ? 2 : 1) * N * kvec;
  const int64_t b_up = SWIGLU ? (int64_t)N * kvec : 0;
  if constexpr (Cfg::PP) {
    constexpr int BN = SWIGLU ? Cfg::BR / 2 : Cfg::BR;
    const int ntiles = N / BN;
    const int64_t mtiles_max = (gm + Cfg::BM - 1) / Cfg::BM + G;
    auto kern = k_grouped_gemm_pp<BF16, Cfg::BM, Cfg::BR, Cfg::SA, Cfg::SB, Cfg::CPR, Cfg::DA, SWIGLU,
                                  Cfg::SPLIT, SAVE>;
    static DeviceCache occ;
    const int grid = persistent_grid((const void *)kern, 512, occ, mtiles_max * ntiles);
    kern<<<dim3(grid), dim3(512), 0, stream>>>(static_cast<const u32x4 *>(a), M, kvec, offsets, G,
                                              static_cast<const u32x4 *>(w), b_expert, b_up,
                                              ntiles, N, out, gather, gk, a_rows, gu);
  } else {
    const int ntiles = N / Cfg::BN;
    const int64_t mtiles_max = (gm + Cfg::BM - 1) / Cfg::BM + G;
    auto kern = k_grouped_gemm<BF16, Cfg::BM, Cfg::BN, Cfg::WM, Cfg::WN, SWIGLU, Cfg::SA, Cfg::SB, SAVE>;
    static DeviceCache occ;
    const int threads = Cfg::WM * Cfg::WN * 64;
    const int grid = persistent_grid((const void *)kern, threads, occ, mtiles_max * ntiles);
    kern<<<dim3(grid), dim3(threads), 0, stream>>>(static_cast<const u32x4 *>(a), M, kvec, offsets,
                                                  G, static_cast<const u32x4 *>(w), b_expert,
                                                  b_up, ntiles, N, out, gather, gk, a_rows, gu);
  }
}

// Tile shapes.
//   Small  (a few rows per expert, decode): 32-row tiles of the 4-wave kernel;
//          the weights stream past once, three slices in flight.
//   Medium (up to 320 rows per expert, e.g. 256 experts x 8192 tokens x top-8):
//          ping-pong tiles of 320 rows x 256 weight rows, so one tile covers
//          an expert's rows, each weight byte is read once and the
//          workgroups of an XCD share the expert's rows through L2.  The
//          wide weight tile halves how often the rows are re-read; 64-byte K
//          slices let LDS hold 4 row stages (2 slices ahead, so no memory
//          phase has to drain its LDS reads) and 5 weight stages (4 ahead).
//   Large  (many rows per expert): ping-pong tiles of 256 rows, 128-byte
//          slices, 2 row stages (1 ahead) and 3 weight stages (2 ahead).
using G1Small = TileCfg<32, 128, 1, 4, 2, 4>;
// fp32 rows are twice as long per K element: with two weight stages a
// workgroup takes 73 KB of LDS instead of 139, so two fit per CU (small
// problems then run their tiles in one round).
using G1SmallF32 = TileCfg<32, 128, 1, 4, 2, 2>;
using G2Small = TileCfg<32, 128, 1, 4, 2, 4>;
using G1Medium = PpCfg<320, 256, 4, 5, 4, true, 2>;
using G2Medium = PpCfg<320, 256, 4, 5, 4, true, 2>;
using G1Large = PpCfg<256, 256, 2, 3, 8, true, 1>;
using G2Large = PpCfg<256, 256, 2, 3, 8, true, 1>;

// Which tile family serves a call: by the mean rows per expert.  Both halves
// of an expert MLP use the same family.  The ping-pong tiles are up to 128
// columns of h and 256 columns of y wide.
enum class Family { Small, Medium, Large };
constexpr int kLongK = 8192;   // reduction length from which the down product uses medium tiles
inline Family family_of(int M, int G, int d) {
  const int64_t per_expert = ((int64_t)M + G - 1) / G;
  if (per_expert < 96 || d % 256 != 0) return Family::Small;
  return per_expert <= 320 ? Family::Medium : Family::Large;
}

// The forward products: family_of, except that a problem too small to give
// the ping-pong tiles one tile per compute unit -- counted for the down
// product, which has the fewest (d / 256 column tiles per row tile) -- runs
// on the 32-row tiles, which spread it over several times as many
// workgroups (the small fp32 layer: 8 down tiles become 128).
inline Family forward_family(int M, int G, int d) {
  const Family f = family_of(M, G, d);
  if (f == Family::Small) return f;
  const int64_t per_expert = ((int64_t)M + G - 1) / G;
  const int bm = f == Family::Medium ? 320 : 256;
  const int64_t tiles = (int64_t)G * ((per_expert + bm - 1) / bm) * (d / 256);
  return tiles < device_cus() ? Family::Small : f;
}

// GEMM1: gate/up + SwiGLU, K = d, N = ffn.  With gu, the pre-activations
// are stored too (the forward of a training step).
template <bool BF16>
void launch_gate_up(Family f, const void *a, int M, int d, int ffn, const int32_t *offsets, int G,
                    const void *w13, void *h, hipStream_t stream, const int32_t *gather = nullptr,
                    int gk = 1, int a_rows = 0, void *gu = nullptr, int grid_rows = -1) {
  if (gu) {
    if (f == Family::Small)
      launch_one<BF16, true, std::conditional_t<BF16, G1Small, G1SmallF32>, true>(
          a, M, d, ffn, offsets, G, w13, h, stream, gather, gk, a_rows, gu);
    else if (f == Family::Medium)
      launch_one<BF16, true, G1Medium, true>(a, M, d, ffn, offsets, G, w13, h, stream, gather, gk, a_rows, gu);
    else
      launch_one<BF16, true, G1Large, true>(a, M, d, ffn, offsets, G, w13, h, stream, gather, gk, a_rows, gu);
    return;
  }
  if (f == Family::Small)
    launch_one<BF16, true, std::conditional_t<BF16, G1Small, G1SmallF32>>(
        a, M, d, ffn, offsets, G, w13, h, stream, gather, gk, a_rows, nullptr, grid_rows);
  else if (f == Family::Medium)
    launch_one<BF16, true, G1Medium>(a, M, d, ffn, offsets, G, w13, h, stream, gather, gk, a_rows,
                                     nullptr, grid_rows);
  else
    launch_one<BF16, true, G1Large>(a, M, d, ffn, offsets, G, w13, h, stream, gather, gk, a_rows,
                                    nullptr, grid_rows);
}

// GEMM2: down, K = ffn, N = d.
template <bool BF16>
void launch_down(Family f, const void *h, int M, int ffn, int d, const int32_t *offsets, int G,
                 const void *w2, void *y, hipStream_t stream, int grid_rows = -1) {
  if (f == Family::Small)
    launch_one<BF16, false, G2Small>(h, M, ffn, d, offsets, G, w2, y, stream, nullptr, 1, 0, nullptr,
                                     grid_rows);
  else if (f == Family::Medium || ffn >= kLongK)
    // A long K (wide experts) is better served by the medium tiles' deeper
    // rings of 64-byte slices, also when there are many rows per expert.
    launch_one<BF16, false, G2Medium>(h, M, ffn, d, offsets, G, w2, y, stream, nullptr, 1, 0, nullptr,
                                      grid_rows);
  else
    launch_one<BF16, false, G2Large>(h, M, ffn, d, offsets, G, w2, y, stream, nullptr, 1, 0, nullptr,
                                     grid_rows);
}

// Backward input-gradient products on the ping-pong tiles (bf16).
template <int VAR, typename Cfg>
void launch_dgrad(const void *a, int M, int K, int N, const int32_t *offsets, int G, const void *w,
                  void *out, const void *gu, hipStream_t stream) {
  const int kvec = K * 2 / 16;
  const int64_t b_expert = (int64_t)K * N * 2 / 16;
  const int ntiles = N / Cfg::BR;
  const int64_t mtiles_max = (M + Cfg::BM - 1) / Cfg::BM + G;
  auto kern = k_grouped_gemm_pp<true, Cfg::BM, Cfg::BR, Cfg::SA, Cfg::SB, Cfg::CPR, Cfg::DA, false,
                                Cfg::SPLIT, false, VAR>;
  static DeviceCache occ;
  const int grid = persistent_grid((const void *)kern, 512, occ, mtiles_max * ntiles);
  kern<<<dim3(grid), dim3(512), 0, stream>>>(static_cast<const u32x4 *>(a), M, kvec, offsets, G,
                                            static_cast<const u32x4 *>(w), b_expert, 0, ntiles, N,
                                            out, nullptr, 1, 0, const_cast<void *>(gu));
}

// Argument checks shared by the three entry points (pointers are checked by
// each).  Returns MOE_OK when the call may launch.
moe_status check_shape(moe_dtype dt, int M, int d, int ffn, int G) {
  if (M < 0 || G < 1 || d < 1 || ffn < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d % 128 != 0 || ffn % 128 != 0 || G > 4096) return MOE_ERR_UNSUPPORTED;
  // 16-byte chunk offsets inside the row operands and inside one expert's
  // weights are 32-bit in the kernels.
  const int64_t elem = dt == MOE_F32 ? 4 : 2, big = (int64_t)1 << 31;
  const int64_t krow = (int64_t)(d > ffn ? d : ffn) * elem / 16;
  if ((int64_t)M * krow >= big || (int64_t)2 * ffn * d * elem / 16 >= big) return MOE_ERR_UNSUPPORTED;
  // Byte offsets inside one expert's weights are 32-bit in the ping-pong kernel.
  if ((int64_t)2 * ffn * d * elem >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

// Reduction length from which the first product's input gradient (var 1)
// uses the medium tiles.
constexpr int kDgradLongK = 4096;

bool launch_dgrad_pp(int var, const void *a, int M, int K, int N, const int32_t *offsets, int G,
                     const void *w, void *out, const void *gu, hipStream_t stream) {
  const Family f = family_of(M, G, K);
  if (f == Family::Small || N % 256 != 0 || K % 64 != 0) return false;
  // Like the forward's down product, the first product's input gradient
  // (var 1: N = d wide, K = 2 ffn) runs faster on the medium tiles' deeper
  // rings of narrower slices once K is long; the down product's (var 2, with
  // the SwiGLU epilogue) stays on the large tiles (measured at Mixtral and
  // EP64-share shapes).
  if (f == Family::Medium || (var == 1 && K >= kDgradLongK)) {
    if (var == 2) launch_dgrad<2, G2Medium>(a, M, K, N, offsets, G, w, out, gu, stream);
    else if (var == 4) launch_dgrad<4, G2Medium>(a, M, K, N, offsets, G, w, out, gu, stream);
    else launch_dgrad<1, G2Medium>(a, M, K, N, offsets, G, w, out, gu, stream);
  } else {
    if (var == 2) launch_dgrad<2, G2Large>(a, M, K, N, offsets, G, w, out, gu, stream);
    else if (var == 4) launch_dgrad<4, G2Large>(a, M, K, N, offsets, G, w, out, gu, stream);
    else launch_dgrad<1, G2Large>(a, M, K, N, offsets, G, w, out, gu, stream);
  }
  return true;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_grouped_gate_up(const void *a, moe_dtype dt, int M, int d, int ffn,
                                          const int32_t *offsets, int G, const void *w13, void *h,
                                          hipStream_t stream) {
  const moe_status st = check_shape(dt, M, d, ffn, G);
  if (st != MOE_OK || M == 0) return st;
  if (!a || !offsets || !w13 || !h) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w13) || !aligned16(h)) return MOE_ERR_INVALID_ARG;
  const Family f = forward_family(M, G, d);
  if (dt == MOE_BF16)
    launch_gate_up<true>(f, a, M, d, ffn, offsets, G, w13, h, stream);
  else
    launch_gate_up<false>(f, a, M, d, ffn, offsets, G, w13, h, stream);
  return launch_status();
}

extern "C" moe_status moe_grouped_gate_up_gather(const void *x, moe_dtype dt, int T, int k, int M,
                                                 int d, int ffn, const int32_t *order,
                                                 const int32_t *offsets, int G, const void *w13,
                                                 void *h, hipStream_t stream) {
  if (T < 0 || k < 1 || M < 0) return MOE_ERR_INVALID_ARG;
  const moe_status st = check_shape(dt, M, d, ffn, G);
  if (st != MOE_OK || M == 0) return st;
  // Byte offsets inside x are 32-bit in the kernels.
  const int64_t elem = dt == MOE_F32 ? 4 : 2;
  if ((int64_t)T * d * elem >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  if (!x || !order || !offsets || !w13 || !h) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(h)) return MOE_ERR_INVALID_ARG;
  const Family f = forward_family(M, G, d);
  if (dt == MOE_BF16)
    launch_gate_up<true>(f, x, M, d, ffn, offsets, G, w13, h, stream, order, k, T);
  else
    launch_gate_up<false>(f, x, M, d, ffn, offsets, G, w13, h, stream, order, k, T);
  return launch_status();
}

extern "C" moe_status moe_grouped_gate_up_save(const void *x, moe_dtype dt, int T, int k, int M,
                                               int d, int ffn, const int32_t *order,
                                               const int32_t *offsets, int G, const void *w13,
                                               void *h, void *gu, hipStream_t stream) {
  if (T < 0 || k < 1 || M < 0) return MOE_ERR_INVALID_ARG;
  const moe_status st = check_shape(dt, M, d, ffn, G);
  if (st != MOE_OK || M == 0) return st;
  const int64_t elem = dt == MOE_F32 ? 4 : 2;
  if (order && (int64_t)T * d * elem >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  if (!x || !offsets || !w13 || !h || !gu) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(h) || !aligned16(gu)) return MOE_ERR_INVALID_ARG;
  const Family f = forward_family(M, G, d);
  if (dt == MOE_BF16)
    launch_gate_up<true>(f, x, M, d, ffn, offsets, G, w13, h, stream, order, order ? k : 1, order ? T : M, gu);
  else
    launch_gate_up<false>(f, x, M, d, ffn, offsets, G, w13, h, stream, order, order ? k : 1, order ? T : M, gu);
  return launch_status();
}

extern "C" moe_status moe_grouped_down(const void *h, moe_dtype dt, int M, int ffn, int d,
                                       const int32_t *offsets, int G, const void *w2, void *y,
                                       hipStream_t stream) {
  const moe_status st = check_shape(dt, M, d, ffn, G);
  if (st != MOE_OK || M == 0) return st;
  if (!h || !offsets || !w2 || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w2) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  const Family f = forward_family(M, G, d);
  if (dt == MOE_BF16)
    launch_down<true>(f, h, M, ffn, d, offsets, G, w2, y, stream);
  else
    launch_down<false>(f, h, M, ffn, d, offsets, G, w2, y, stream);
  return launch_status();
}

extern "C" moe_status moe_grouped_swiglu(const void *a, moe_dtype dt, int M, int d, int ffn,
                                         const int32_t *offsets, int G, const void *w13,
                                         const void *w2, void *h, void *y, hipStream_t stream) {
  const moe_status st = check_shape(dt, M, d, ffn, G);
  if (st != MOE_OK || M == 0) return st;
  if (!a || !offsets || !w13 || !w2 || !h || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w13) || !aligned16(w2) || !aligned16(h) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  const Family f = forward_family(M, G, d);
  if (dt == MOE_BF16) {
    launch_gate_up<true>(f, a, M, d, ffn, offsets, G, w13, h, stream);
    launch_down<true>(f, h, M, ffn, d, offsets, G, w2, y, stream);
  } else {
    launch_gate_up<false>(f, a, M, d, ffn, offsets, G, w13, h, stream);
    launch_down<false>(f, h, M, ffn, d, offsets, G, w2, y, stream);
  }
  return launch_status();
}

extern "C" moe_status moe_expert_loop_swiglu(const void *a, moe_dtype dt, int M, int d, int ffn,
                                             const int32_t *offsets, const int32_t *offsets_host,
                                             int G, const void *w13, const void *w2, void *h,
                                             void *y, hipStream_t stream) {
  const moe_status st = check_shape(dt, M, d, ffn, G);
  if (st != MOE_OK) return st;
  if (!offsets_host) return MOE_ERR_INVALID_ARG;
  if (offsets_host[0] < 0 || offsets_host[G] > M) return MOE_ERR_INVALID_ARG;
  for (int e = 0; e < G; ++e)
    if (offsets_host[e + 1] < offsets_host[e]) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (!a || !offsets || !w13 || !w2 || !h || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w13) || !aligned16(w2) || !aligned16(h) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  const int64_t elem = dt == MOE_F32 ? 4 : 2;
  const int64_t w13_bytes = 2 * (int64_t)ffn * d * elem, w2_bytes = (int64_t)d * ffn * elem;
  // One product per expert: the kernels read the segment bounds from
  // offsets + e (a one-expert list) and the grid is sized for its rows.
  for (int e = 0; e < G; ++e) {
    const int n = offsets_host[e + 1] - offsets_host[e];
    if (n == 0) continue;
    const Family f = family_of(n, 1, d);
    const void *we13 = static_cast<const char *>(w13) + e * w13_bytes;
    const void *we2 = static_cast<const char *>(w2) + e * w2_bytes;
    if (dt == MOE_BF16) {
      launch_gate_up<true>(f, a, M, d, ffn, offsets + e, 1, we13, h, stream, nullptr, 1, 0, nullptr, n);
      launch_down<true>(f, h, M, ffn, d, offsets + e, 1, we2, y, stream, n);
    } else {
      launch_gate_up<false>(f, a, M, d, ffn, offsets + e, 1, we13, h, stream, nullptr, 1, 0, nullptr, n);
      launch_down<false>(f, h, M, ffn, d, offsets + e, 1, we2, y, stream, n);
    }
  }
  return launch_status();
}
