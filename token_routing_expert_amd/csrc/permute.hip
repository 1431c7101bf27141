// Permute: per-chunk expert histograms, one exclusive scan, a stable
// wave-ballot multisplit that writes order and inv, and a row scatter that
// reads every token row once and writes its k packed copies.
//
// "Token permutation and grouped GEMMs" (zerotofrontier.app, "Expert
// parallelism"): order is the stable argsort of the expert ids, X[order] puts
// rows in expert order, and inv (inv[order] = arange) undoes it.
#include <math.h>

#include <atomic>
#include <mutex>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kScatterNV = 8;   // 16-byte vectors per lane per round of the row scatter
constexpr int kMaxChunks = 1024;

// Assignments per chunk: at least 2048, and few enough chunks that the scan's
// per-expert walk over chunks stays short.
inline int64_t chunk_size(int64_t M) {
  int64_t c = 2048;
  while ((M + c - 1) / c > kMaxChunks) c *= 2;
  return c;
}

// hist[c][e] = number of assignments in chunk c with expert e.
__global__ __launch_bounds__(kThreads) void k_hist(const int32_t *__restrict__ ids, int64_t M, int E,
                                                   int64_t chunk, int32_t *__restrict__ hist) {
  extern __shared__ int h[];
  for (int e = threadIdx.x; e < E; e += kThreads) h[e] = 0;
  __syncthreads();
  const int64_t a0 = blockIdx.x * chunk;
  const int64_t a1 = min(a0 + chunk, M);
  for (int64_t a = a0 + threadIdx.x; a < a1; a += kThreads) {
    const int e = ids[a];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// One block of 1024 threads, thread e owns expert e (E <= 1024).
// counts[e] = sum over chunks; offsets = exclusive scan of counts;
// hist[c][e] becomes the first packed position of chunk c's expert-e rows.
// The chunk walks read kBatch chunks' counts at a time, so their loads are in
// flight together instead of one L2 round trip per chunk.
__global__ __launch_bounds__(1024) void k_scan(int32_t *__restrict__ hist, int nchunks, int E,
                                               int32_t *__restrict__ counts,
                                               int32_t *__restrict__ offsets) {
  constexpr int kBatch = 8;
  __shared__ int wave_tot[16];
  const int e = threadIdx.x;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  int total = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = c0 + i < nchunks ? hist[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) total += v[i];
    }
    counts[e] = total;
  }
  // Block-wide exclusive scan of total over e.
  int incl = total;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  if (wv == 0) {
    int t = lane < 16 ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(t, off);
      if (lane >= off) t += o;
    }
    if (lane < 16) wave_tot[lane] = t;  // inclusive totals per wave
  }
  __syncthreads();
  const int excl = incl - total + (wv > 0 ? wave_tot[wv - 1] : 0);
  if (e < E) {
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + total;
    int run = excl;
    for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = c0 + i < nchunks ? hist[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (c0 + i < nchunks) hist[(int64_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    }
  }
}

// Stable ranks within a chunk, for a workgroup of NW waves.  The chunk
// [c0, c0 + chunk) is cut into NW contiguous parts, one per wave.  Each wave
// walks its part 64 assignments at a time; lanes with equal expert ids find
// each other with one ballot per id bit, and the rank of a lane is the
// number of equal lanes below it.  Ranks therefore follow assignment order,
// which makes the sort stable.  base(e) is the first packed position of the
// chunk's expert-e assignments; cnt is NW E ints of LDS.
//
// Capacity form (cap >= 0): an assignment's rank inside its expert is its
// packed position minus seg_start[e]; rank r < cap goes to slot e cap + r,
// a higher rank is dropped (inv = -1, no order entry).
template <int NW, typename Base>
__device__ __forceinline__ void stable_ranks(const int32_t *__restrict__ ids, int64_t M, int E, int nbits,
                                             int64_t c0, int64_t chunk, Base base, int *cnt,
                                             int32_t *__restrict__ order, int32_t *__restrict__ inv,
                                             const int32_t *__restrict__ seg_start, int cap) {
  const int wv = uniform(threadIdx.x >> 6), lane = lane_id();
  for (int i = threadIdx.x; i < NW * E; i += NW * kWave) cnt[i] = 0;
  __syncthreads();
  const int64_t part = (chunk + NW - 1) / NW;
  const int64_t q0 = min(c0 + wv * part, min(c0 + chunk, M)), q1 = min(q0 + part, min(c0 + chunk, M));
  int *mine = cnt + wv * E;
  for (int64_t a = q0 + lane; a < q1; a += kWave) {
    const int e = ids[a];
    if (e >= 0 && e < E) atomicAdd(&mine[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += NW * kWave) {
    int run = base(e);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int v = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int64_t s = q0; s < q1; s += kWave) {
    const int64_t a = s + lane;
    const int e = a < q1 ? ids[a] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    int pos = 0;
    if (valid) {
      pos = mine[e] + __popcll(peers & below);
      if (cap < 0) {
        order[pos] = (int32_t)a;
        inv[a] = pos;
      } else {
        const int r = pos - seg_start[e];
        const int slot = r < cap ? e * cap + r : -1;
        if (slot >= 0) order[slot] = (int32_t)a;
        inv[a] = slot;
      }
    }
    // All lanes have read mine[] above; now the lowest lane of each group of
    // equal ids advances that expert's cursor.
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers & below) == 0) mine[e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

// Chunk blockIdx.x of the multi-chunk permute (4 waves); its bases are the
// scanned histogram row.
__global__ __launch_bounds__(kThreads) void k_multisplit(const int32_t *__restrict__ ids, int64_t M,
                                                         int E, int nbits, int64_t chunk,
                                                         const int32_t *__restrict__ base,
                                                         int32_t *__restrict__ order,
                                                         int32_t *__restrict__ inv,
                                                         const int32_t *__restrict__ seg_start = nullptr,
                                                         int cap = -1) {
  extern __shared__ int cnt[];  // [4][E]
  const int32_t *row = base + (int64_t)blockIdx.x * E;
  stable_ranks<kThreads / kWave>(ids, M, E, nbits, (int64_t)blockIdx.x * chunk, chunk,
                                 [row](int e) { return row[e]; }, cnt, order, inv, seg_start, cap);
}

// All assignments in one chunk (M <= 2048): the histogram, the scan and the
// stable ranks in one workgroup of 16 waves -- one launch instead of three.
// Writes counts and offsets (dropless) or counts and seg_start (capacity).
constexpr int kOneThreads = 1024;
constexpr int kOneMaxE = 960;   // 17 E ints of LDS stay within 64 KB
__global__ __launch_bounds__(kOneThreads) void k_permute_one(const int32_t *__restrict__ ids, int64_t M,
                                                            int E, int nbits, int32_t *__restrict__ counts,
                                                            int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ order,
                                                            int32_t *__restrict__ inv, int cap) {
  extern __shared__ int lds[];  // base [E], then cnt [16][E]
  __shared__ int wave_tot[16];
  int *base = lds, *cnt = lds + E;
  const int e = threadIdx.x, lane = lane_id(), wv = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < E; i += kOneThreads) base[i] = 0;
  __syncthreads();
  for (int64_t a = threadIdx.x; a < M; a += kOneThreads) {
    const int x = ids[a];
    if (x >= 0 && x < E) atomicAdd(&base[x], 1);
  }
  __syncthreads();
  // Exclusive scan of the counts over the experts (E <= 1024, thread e owns e).
  const int total = e < E ? base[e] : 0;
  int incl = total;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  if (wv == 0) {
    int t = lane < 16 ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(t, off);
      if (lane >= off) t += o;
    }
    if (lane < 16) wave_tot[lane] = t;
  }
  __syncthreads();
  const int excl = incl - total + (wv > 0 ? wave_tot[wv - 1] : 0);
  if (e < E) {
    counts[e] = total;
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + total;
    base[e] = excl;
  }
  __syncthreads();
  stable_ranks<kOneThreads / kWave>(ids, M, E, nbits, 0, M, [base](int x) { return base[x]; }, cnt, order,
                                    inv, base, cap);
}

// Capacity form: the slots no assignment reached (rank past the expert's
// count) hold -1, and the block offsets are e cap.
__global__ __launch_bounds__(kThreads) void k_capacity_fill(const int32_t *__restrict__ counts, int E,
                                                            int cap, int32_t *__restrict__ order,
                                                            int32_t *__restrict__ offsets) {
  const int64_t s = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (s <= E) offsets[s] = (int32_t)(s * cap);
  if (s >= (int64_t)E * cap) return;
  const int e = (int)(s / cap), r = (int)(s - (int64_t)e * cap);
  if (r >= counts[e]) order[s] = -1;
}

// A store of data that is not read again soon (nontemporal: it does not
// displace cached data on its way to HBM).
__device__ __forceinline__ void store_stream(uint4 *p, const uint4 &v) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u *>(p));
}

// One wave per token: read the row once (16-byte vectors), write k copies.
// Up to 64 NV vectors of the row are loaded into registers before the first
// store, so those loads are in flight at once; the k copies then stream out
// with nontemporal stores.  Longer rows take several rounds.
template <int NV>
__global__ __launch_bounds__(kThreads) void k_row_scatter(const uint4 *__restrict__ x, int T, int k,
                                                          int nvec, const int32_t *__restrict__ inv,
                                                          int64_t M, uint4 *__restrict__ x_perm) {
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const uint4 *src = x + (int64_t)t * nvec;
  int dst[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) dst[j] = j < k ? uniform(inv[(int64_t)t * k + j]) : -1;
  for (int v0 = 0; v0 < nvec; v0 += NV * kWave) {
    uint4 r[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = v0 + u * kWave + lane;
      if (v < nvec) r[u] = src[v];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= k) break;
      const int p = dst[j];
      if (p < 0 || p >= M) continue;
      uint4 *out = x_perm + (int64_t)p * nvec;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int v = v0 + u * kWave + lane;
        if (v < nvec) store_stream(out + v, r[u]);
      }
    }
  }
}

// Capacity form: one wave per slot of the padded batch copies the row of the
// slot's token, or writes zeros into a padding slot.
__global__ __launch_bounds__(kThreads) void k_capacity_rows(const uint4 *__restrict__ x, int T, int k,
                                                            int nvec, const int32_t *__restrict__ order,
                                                            int64_t slots, uint4 *__restrict__ x_cap) {
  const int64_t s = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (s >= slots) return;
  const int a = uniform(order[s]);
  const int64_t t = a >= 0 ? a / k : -1;
  uint4 *out = x_cap + s * nvec;
  if (t < 0 || t >= T) {
    for (int v = lane_id(); v < nvec; v += kWave) store_stream(out + v, make_uint4(0, 0, 0, 0));
    return;
  }
  const uint4 *src = x + t * nvec;
  for (int v0 = 0; v0 < nvec; v0 += kScatterNV * kWave) {
    uint4 r[kScatterNV];
#pragma unroll
    for (int u = 0; u < kScatterNV; ++u) {
      const int v = v0 + u * kWave + lane_id();
      if (v < nvec) r[u] = src[v];
    }
#pragma unroll
    for (int u = 0; u < kScatterNV; ++u) {
      const int v = v0 + u * kWave + lane_id();
      if (v < nvec) store_stream(out + v, r[u]);
    }
  }
}

// Generic k (> 16): the same copy with inv read inside the loop.
__global__ __launch_bounds__(kThreads) void k_row_scatter_anyk(const uint4 *__restrict__ x, int T,
                                                               int k, int nvec,
                                                               const int32_t *__restrict__ inv,
                                                               int64_t M,
                                                               uint4 *__restrict__ x_perm) {
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  for (int v = lane; v < nvec; v += kWave) {
    const uint4 r = x[(int64_t)t * nvec + v];
    for (int j = 0; j < k; ++j) {
      const int p = uniform(inv[(int64_t)t * k + j]);
      if (p >= 0 && p < M) x_perm[(int64_t)p * nvec + v] = r;
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_permute_workspace_bytes(int T, int k, int E) {
  if (T <= 0 || k <= 0 || E <= 0) return 16;
  const int64_t M = (int64_t)T * k;
  const int64_t nchunks = (M + chunk_size(M) - 1) / chunk_size(M);
  return (size_t)nchunks * (size_t)E * sizeof(int32_t);
}

extern "C" moe_status moe_permute(const void *x, moe_dtype dt, int T, int d,
                                  const int32_t *topk_ids, int k, int E, int32_t *counts,
                                  int32_t *offsets, int32_t *order, int32_t *inv, void *x_perm,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1 || d < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (E > 1024 || d % 8 != 0 || (int64_t)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  const int64_t M = (int64_t)T * k;
  // x and x_perm both NULL: index-only mode (counts, offsets, order, inv).
  const bool rows = x || x_perm;
  if (M > 0 && (!topk_ids || !order || !inv || !workspace)) return MOE_ERR_INVALID_ARG;
  if (M > 0 && rows && (!x || !x_perm)) return MOE_ERR_INVALID_ARG;
  if (M > 0 && rows && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe_permute_workspace_bytes(T, k, E)) return MOE_ERR_INVALID_ARG;

  const int64_t chunk = chunk_size(M > 0 ? M : 1);
  const int nchunks = (int)((M + chunk - 1) / chunk);
  int32_t *hist = static_cast<int32_t *>(workspace);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;

  if (nchunks == 1 && E <= kOneMaxE) {
    k_permute_one<<<dim3(1), dim3(kOneThreads), sizeof(int) * 17 * E, stream>>>(
        topk_ids, M, E, nbits, counts, offsets, order, inv, -1);
  } else {
    if (nchunks > 0)
      k_hist<<<dim3(nchunks), dim3(kThreads), sizeof(int) * E, stream>>>(topk_ids, M, E, chunk, hist);
    // The scan also runs for M == 0 so that counts and offsets are written.
    k_scan<<<dim3(1), dim3(1024), 0, stream>>>(hist, nchunks, E, counts, offsets);
    if (M == 0) return launch_status();
    k_multisplit<<<dim3(nchunks), dim3(kThreads), sizeof(int) * 4 * E, stream>>>(
        topk_ids, M, E, nbits, chunk, hist, order, inv);
  }
  if (!rows) return launch_status();
  const int elem = dt == MOE_F32 ? 4 : 2;
  const int nvec = (int)((int64_t)d * elem / 16);
  const dim3 grid((T + 3) / 4);
  if (k <= 16)
    k_row_scatter<kScatterNV><<<grid, dim3(kThreads), 0, stream>>>(
        static_cast<const uint4 *>(x), T, k, nvec, inv, M, static_cast<uint4 *>(x_perm));
  else
    k_row_scatter_anyk<<<grid, dim3(kThreads), 0, stream>>>(static_cast<const uint4 *>(x), T, k,
                                                             nvec, inv, M,
                                                             static_cast<uint4 *>(x_perm));
  return launch_status();
}

// ---- the permute without a caller workspace --------------------------------
// The per-chunk histograms live in this file-scope device array instead.  In
// host code `scratch` names a host-side stand-in: the device address of each
// GPU's copy comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to a kernel.
constexpr size_t kNoAllocScratchBytes = 1u << 20;
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

namespace moe {
namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxScratchDevices];   // zero-initialised: static storage
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up on the first call on
// that device; NULL if the lookup fails.
void *device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();   // clear the error so it does not surface at a later call
    return nullptr;
  }
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}
}  // namespace
}  // namespace moe

extern "C" moe_status moe_permute_noalloc(const void *x, moe_dtype dt, int T, int d,
                                          const int32_t *topk_ids, int k, int E, int32_t *counts,
                                          int32_t *offsets, int32_t *order, int32_t *inv,
                                          void *x_perm, hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1 || d < 1) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_permute_workspace_bytes(T, k, E);
  if (need > kNoAllocScratchBytes) return MOE_ERR_UNSUPPORTED;
  void *ws = device_scratch();
  if (!ws) return MOE_ERR_HIP;
  return moe_permute(x, dt, T, d, topk_ids, k, E, counts, offsets, order, inv, x_perm, ws,
                     kNoAllocScratchBytes, stream);
}

extern "C" int64_t moe_expert_capacity(int64_t M, int E, double cf) {
  if (E < 1 || M < 0 || !(cf > 0.0)) return -1;
  return (int64_t)ceil(cf * (double)M / (double)E);
}

extern "C" size_t moe_permute_capacity_workspace_bytes(int T, int k, int E) {
  if (E <= 0) return 16;
  return moe_permute_workspace_bytes(T, k, E) + (size_t)(E + 1) * sizeof(int32_t);
}

extern "C" moe_status moe_permute_capacity(const void *x, moe_dtype dt, int T, int d,
                                           const int32_t *topk_ids, int k, int E, int cap,
                                           int32_t *counts, int32_t *offsets, int32_t *order,
                                           int32_t *inv, void *x_cap, void *workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1 || d < 1 || cap < 0) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (E > 1024 || d % 8 != 0 || (int64_t)T * k >= (1ll << 31) || (int64_t)E * cap >= (1ll << 31))
    return MOE_ERR_UNSUPPORTED;
  const int64_t M = (int64_t)T * k, slots = (int64_t)E * cap;
  if (!counts || !offsets || !workspace) return MOE_ERR_INVALID_ARG;
  if ((M > 0 && (!topk_ids || !inv)) || (slots > 0 && !order)) return MOE_ERR_INVALID_ARG;
  const bool rows = x || x_cap;   // both NULL: index-only mode
  if (rows && slots > 0 && (!x || !x_cap || !aligned16(x) || !aligned16(x_cap)))
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe_permute_capacity_workspace_bytes(T, k, E)) return MOE_ERR_INVALID_ARG;

  const int64_t chunk = chunk_size(M > 0 ? M : 1);
  const int nchunks = (int)((M + chunk - 1) / chunk);
  int32_t *hist = static_cast<int32_t *>(workspace);
  int32_t *seg_start = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                                   moe_permute_workspace_bytes(T, k, E));
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  if (nchunks == 1 && E <= kOneMaxE) {
    k_permute_one<<<dim3(1), dim3(kOneThreads), sizeof(int) * 17 * E, stream>>>(
        topk_ids, M, E, nbits, counts, seg_start, order, inv, cap);
  } else {
    if (nchunks > 0)
      k_hist<<<dim3(nchunks), dim3(kThreads), sizeof(int) * E, stream>>>(topk_ids, M, E, chunk, hist);
    k_scan<<<dim3(1), dim3(1024), 0, stream>>>(hist, nchunks, E, counts, seg_start);
    if (M > 0)
      k_multisplit<<<dim3(nchunks), dim3(kThreads), sizeof(int) * 4 * E, stream>>>(
          topk_ids, M, E, nbits, chunk, hist, order, inv, seg_start, cap);
  }
  const int64_t fill = (slots > E + 1 ? slots : E + 1);
  k_capacity_fill<<<dim3((unsigned)((fill + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream>>>(
      counts, E, cap, order, offsets);
  if (!rows || slots == 0) return launch_status();
  const int elem = dt == MOE_F32 ? 4 : 2;
  const int nvec = (int)((int64_t)d * elem / 16);
  k_capacity_rows<<<dim3((unsigned)((slots + 3) / 4)), dim3(kThreads), 0, stream>>>(
      static_cast<const uint4 *>(x), T, k, nvec, order, slots, static_cast<uint4 *>(x_cap));
  return launch_status();
}
