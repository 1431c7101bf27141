// Device and host helpers shared by the grouped products of the forward
// (grouped_gemm.hip) and the backward (grouped_gemm_bwd.hip): operand types,
// the tile schedule over ragged expert segments, direct global-to-LDS loads
// and the persistent grid.
#pragma once

#include <atomic>

#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16 bytes as a native vector (HIP's uint4 struct defeats register promotion
// of small arrays).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int clamp_row(int v, int M) { return v < 0 ? 0 : (v > M ? M : v); }

struct Tile {
  int expert, lo, hi, m0, n_tile;
};

// MI355X dispatches workgroup i of a launch to XCD i % 8; each XCD has its own
// L2.  The persistent kernels below give XCD x a contiguous band of tiles so
// the tiles that share operands run on the same L2 at the same time.
constexpr int kXcds = 8;

// Total number of (m, n) tiles over all expert segments.  Every wave
// computes the same value.
template <int BM>
__device__ __forceinline__ int count_tiles(const int32_t *__restrict__ offsets, int G, int M,
                                           int ntiles) {
  const int lane = lane_id();
  int sum = 0;
  for (int eb = 0; eb < G; eb += kWave) {
    const int e = eb + lane;
    if (e < G) {
      const int a = clamp_row(offsets[e], M), b = clamp_row(offsets[e + 1], M);
      const int n = b > a ? b - a : 0;
      sum += ((n + BM - 1) / BM) * ntiles;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  return uniform(sum);
}

constexpr int kMBlock = 4;   // m-tiles of an expert grouped together in the tile order

// Which expert and which (m, n) tile is tile number L.  Tiles are numbered
// expert by expert; inside an expert by blocks of kMBlock m-tiles, each
// block n-tile major and m-tile minor, so the m-tiles that share one weight
// tile are adjacent and the n-tiles that share a block's rows follow each
// other.  Every wave computes the same answer.
// A workgroup asks for increasing L, so the search resumes at the expert
// (e0) and tile number (base) of the previous answer: one 64-expert window
// per call in the usual case instead of a scan from expert 0.
template <int BM>
__device__ __forceinline__ bool find_tile(const int32_t *__restrict__ offsets, int G, int M,
                                          int ntiles, int L, Tile &t, int &e0, int &base) {
  const int lane = lane_id();
  int running = base;
  for (int eb = e0; eb < G; eb += kWave) {
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
      const int first = uniform(__shfl(excl, src));
      const int local = L - first;
      const int mtiles = (t.hi - t.lo + BM - 1) / BM;
      // Inside an expert the m-tiles go in blocks of kMBlock: block by block,
      // n-tile by n-tile, the block's m-tiles adjacent.  Tiles that run at
      // the same time on one XCD then share kMBlock row tiles and a few
      // weight tiles instead of one weight tile and many row tiles.
      const int mb = min(local / (kMBlock * ntiles), (mtiles - 1) / kMBlock);
      const int msize = min(kMBlock, mtiles - mb * kMBlock);
      const int rem = local - mb * kMBlock * ntiles;
      t.m0 = t.lo + (mb * kMBlock + rem % msize) * BM;
      t.n_tile = rem / msize;
      e0 = t.expert;
      base = first;
      return true;
    }
    running += __shfl(incl, kWave - 1);
  }
  return false;
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 63] (the count is an
// immediate, so the value selects one of 64 waits through a branch tree).
template <int LO, int HI>
__device__ __forceinline__ void wait_vmcnt_range(int n) {
  if constexpr (LO == HI) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (LO & 15) | ((LO >> 4) << 14));
  } else {
    constexpr int MID = (LO + HI) / 2;
    if (n <= MID) wait_vmcnt_range<LO, MID>(n);
    else wait_vmcnt_range<MID + 1, HI>(n);
  }
}
__device__ __forceinline__ void wait_vmcnt(int n) { wait_vmcnt_range<0, 63>(n < 63 ? n : 63); }

// The logistic function with the hardware reciprocal (within 1 ulp in fp32)
// instead of a correctly rounded division: the SwiGLU epilogues evaluate it
// for every output, and the division's instruction sequence was a third of
// a gate/up tile's epilogue.  e^-g overflowing to infinity gives 0, as the
// division would.
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu(float g) { return g * sigmoid_f(g); }

// Source row of packed row p under a gather: token gather[p] / gk, clamped to
// [0, a_rows) so a corrupt index can only steer a read inside A.
__device__ __forceinline__ uint32_t gather_row(const int32_t *gather, int p, int gk, int a_rows) {
  const uint32_t src = (uint32_t)gather[p] / (uint32_t)gk;
  return src < (uint32_t)a_rows ? src : (uint32_t)a_rows - 1u;
}


// Fourth word of a raw buffer resource on gfx9-class GPUs: 32-bit data
// format, no swizzle, no stride; accesses at or past the byte count return 0.
constexpr int kBufferFlags = 0x00020000;


// One wave's 16-byte-per-lane buffer load straight into LDS: lane l's data
// lands at lds + 16 l.  base/bytes describe the buffer; voff is the lane's
// byte offset, soff a wave-uniform byte offset added to it.  CPOL is the
// instruction's cache policy (kNonTemporal: the nt bit).
constexpr int kNonTemporal = 2;
template <int CPOL = 0>
__device__ __forceinline__ void buffer_load_lds16(const void *base, uint32_t bytes, u32x4 *lds,
                                                  uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t res =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (__attribute__((address_space(3))) void *)lds, 16,
                                           voff, soff, 0, CPOL);
}

// A workgroup barrier that is also a scheduling fence: without the fences the
// compiler may move MFMAs (register-only instructions) across s_barrier, which
// would pull one group's compute phase into the other group's window.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Per-device caches of launch-shape queries.  Entries are atomics: calls on
// several host threads may fill one at the same time (each stores the same
// value), and a reader sees either 0 (not yet queried) or the value.
constexpr int kMaxDevices = 64;
struct DeviceCache {
  std::atomic<int> v[kMaxDevices];
};

// The current device, or -1 when it cannot be cached.
inline int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

// Compute units of the current device.
inline int device_cus() {
  static DeviceCache cus;   // zero-initialised: static storage
  const int dev = current_device();
  int n = dev >= 0 ? cus.v[dev].load(std::memory_order_relaxed) : 0;
  if (n > 0) return n;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  if (dev >= 0) cus.v[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Persistent grid: resident workgroups (CUs x blocks per CU), no more than
// there can be tiles, rounded to a multiple of the XCD count.  occ caches the
// occupancy query of one kernel instantiation, per device.
inline int persistent_grid(const void *kernel, int threads, DeviceCache &occ, int64_t max_tiles) {
  const int dev = current_device();
  int per_cu = dev >= 0 ? occ.v[dev].load(std::memory_order_relaxed) : 0;
  if (per_cu == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    if (dev >= 0) occ.v[dev].store(per_cu, std::memory_order_relaxed);
  }
  int64_t g = (int64_t)device_cus() * per_cu;
  const int64_t cap = (max_tiles + kXcds - 1) / kXcds * kXcds;
  if (g > cap) g = cap;
  g = g / kXcds * kXcds;
  return (int)(g < kXcds ? kXcds : g);
}

// ---- column-contiguous operand tiles ------------------------------------
// An operand stored along the output dimension ([K, N] row-major weights of
// a backward product, or the rows of a weight gradient's operands) is staged
// in LDS as it lies in memory and read back transposed for MFMA, which wants
// every lane's values consecutive in K.

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Column-contiguous tile: K-rows of W columns (W = 128 or 256), 2 W bytes
// per K-row in 64-byte segments of 32 columns.  Segment sg of K-row r is
// stored at position sg ^ (r & 3): a transposing read takes 64 bytes from
// each of four K-rows r .. r + 3 per half wave, which then land in four
// different quarters of the 256-byte bank row.
template <int W>
__device__ __forceinline__ int cc_byte(int r, int sg, int byte_in_seg) {
  return r * (2 * W) + ((sg ^ (r & 3)) << 6) + byte_in_seg;
}

// A column-contiguous stage of W columns (W = 128 or 256) is filled by
// 1 KB DMA groups of 512 / W K-rows; lane l of group g fills K-row
// g (512 / W) + l / (W / 8) at physical chunk l % (W / 8), which holds the
// 16 bytes at this column of the tile (segment swizzle of cc_byte).
template <int W>
__device__ __forceinline__ void cc_lane(int g, int lane, int &krow, int &col) {
  constexpr int LPR = W / 8;   // lanes per K-row
  krow = g * (512 / W) + lane / LPR;
  const int pc = lane % LPR;
  col = (((pc >> 2) ^ (krow & 3)) << 5) + (pc & 3) * 8;
}

// The same operand for 32 columns (column block cb) from a column-contiguous
// tile.  ds_read_b64_tr_b16 works on groups of 16 lanes: if lane 4 i + a of
// a group addresses four consecutive 16-bit values, lane 4 a + b receives
// value b of lanes a, 4 + a, 8 + a, 12 + a.  So lane s addresses K-row
// 16 q + 8 (s / 32) + 4 h + (s % 16) / 4 at columns 16 ((s / 16) % 2) +
// 4 (s % 4) of the block, and lane l receives column l % 32 at K-rows
// 8 (l / 32) + 4 h .. + 3: half h = 0 gives the lane's K 0..3, h = 1 K 4..7.
template <int W>
__device__ __forceinline__ u32x4 frag_tr(const char *stage, int cb, int q, int lane) {
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * q + 8 * (lane >> 5) + 4 * h + ((lane & 15) >> 2);
    const int byte = cc_byte<W>(r, cb, (((lane >> 4) & 1) << 5) + ((lane & 3) << 3));
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(stage + byte));
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    out[2 * h] = w[0];
    out[2 * h + 1] = w[1];
  }
  return out;
}

}  // namespace
}  // namespace moe

namespace moe {
// The backward input-gradient products on the ping-pong tiles (defined in
// grouped_gemm.hip): var 1 stores out = a W_e ([M, K] x [K, N] per expert
// segment), var 2 applies the SwiGLU backward with the pre-activations gu
// and writes dgu ([M, 2 N]), var 4 adds the product to out.  Returns false, launching nothing, when the
// shape is not one the ping-pong tiles serve (few rows per expert, N not a
// multiple of 256); the caller then uses its own tiles.
bool launch_dgrad_pp(int var, const void *a, int M, int K, int N, const int32_t *offsets, int G,
                     const void *w, void *out, const void *gu, hipStream_t stream);
// Weight gradients out[e] = a[seg e]^T b[seg e] ([G, m_dim, n_dim])
// (grouped_wgrad.hip); false (nothing launched) when m_dim or n_dim is not a
// multiple of 256 or an operand is too large for 32-bit offsets.
bool launch_weight_grad(const void *a, const void *b, int M, int m_dim, int n_dim,
                        const int32_t *offsets, int G, void *out, hipStream_t stream);
}  // namespace moe
