// Device and host helpers shared by the grouped products of the forward
// (grouped_gemm.hip) and the backward (grouped_gemm_bwd.hip): operand types,
// the tile schedule over ragged expert segments, direct global-to-LDS loads
// and the persistent grid.
#pragma once

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

// Which expert and which (m, n) tile is tile number L.  Tiles are numbered
// expert by expert; inside an expert n-tile major and m-tile minor, so the
// m-tiles that share one weight tile are adjacent and the n-tiles that share
// the expert's rows follow each other.  Every wave computes the same answer.
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
      t.m0 = t.lo + (local % mtiles) * BM;
      t.n_tile = local / mtiles;
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

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

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
// byte offset, soff a wave-uniform byte offset added to it.
__device__ __forceinline__ void buffer_load_lds16(const void *base, uint32_t bytes, u32x4 *lds,
                                                  uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t res =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (__attribute__((address_space(3))) void *)lds, 16,
                                           voff, soff, 0, 0);
}

// A workgroup barrier that is also a scheduling fence: without the fences the
// compiler may move MFMAs (register-only instructions) across s_barrier, which
// would pull one group's compute phase into the other group's window.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Compute units of the current device (cached per device id).
inline int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Persistent grid: resident workgroups (CUs x blocks per CU), no more than
// there can be tiles, rounded to a multiple of the XCD count.  per_cu caches
// the occupancy query of one kernel instantiation.
inline int persistent_grid(const void *kernel, int threads, int &per_cu, int64_t max_tiles) {
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  int64_t g = (int64_t)device_cus() * per_cu;
  const int64_t cap = (max_tiles + kXcds - 1) / kXcds * kXcds;
  if (g > cap) g = cap;
  g = g / kXcds * kXcds;
  return (int)(g < kXcds ? kXcds : g);
}

}  // namespace
}  // namespace moe
