// Unpermute and weight: y[t] = sum_j w[t,j] y_perm[inv[t k + j]] (+ y_shared[t]).
// With no gates (w = NULL) every gate is 1: the sum of a token's k rows,
// which is also the backward of the permute (the dispatch's gradient is
// combined back into the token).
//
// "Expert parallelism" (zerotofrontier.app), section "Expert parallelism",
// step 7 of the forward pass: every expert output row returns to the token it
// came from, scaled by that token's gate for the expert, and the k
// contributions add up.  The kernel computes this sum from the token's side:
// one wave per token fetches the token's k packed rows through inv and
// stores the token once.  No two waves write one token, so no atomics are
// needed, and the fp32 additions run in a fixed order (slot 0..k-1, then the
// shared row).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kCombineNV = 2;   // 16-byte vectors per lane per round

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Loads and stores of rows that are touched once: nontemporal, so the
// streams do not displace cached data.
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
  const v4u q = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
  return make_uint4(q[0], q[1], q[2], q[3]);
}
__device__ __forceinline__ void store_stream(uint4 *p, const uint4 &v) {
  __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u *>(p));
}

template <bool BF16>
struct Vec;

// 16 bytes = 8 bf16 values.
template <>
struct Vec<true> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void add(float *acc, float w, const uint4 &v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += w * bf16_lo(u[i]);
      acc[2 * i + 1] += w * bf16_hi(u[i]);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float *acc) {
    return make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                      pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
};

// 16 bytes = 4 fp32 values.
template <>
struct Vec<false> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void add(float *acc, float w, const uint4 &v) {
    acc[0] += w * __uint_as_float(v.x);
    acc[1] += w * __uint_as_float(v.y);
    acc[2] += w * __uint_as_float(v.z);
    acc[3] += w * __uint_as_float(v.w);
  }
  static __device__ __forceinline__ uint4 pack(const float *acc) {
    return make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                      __float_as_uint(acc[3]));
  }
};

// One wave per token.  The token's k slots (packed positions and gates) are
// read once into scalar registers; each lane then handles NV vectors of the
// row per round, issuing the loads of all k rows (and the shared row) for all
// NV vectors before the first add, so a round keeps NV (k + 1) loads in
// flight.  The adds keep the fixed order slot 0 .. k-1, then the shared row.
// The expert rows are read once and the output written once: both stream
// with nontemporal accesses.
template <bool BF16, int KMAX, int NV>
__global__ __launch_bounds__(kThreads) void k_combine(const uint4 *__restrict__ y_perm, int T, int k,
                                                      int nvec, const int32_t *__restrict__ inv,
                                                      const float *__restrict__ w,
                                                      const uint4 *__restrict__ y_sh, int64_t M,
                                                      uint4 *__restrict__ y) {
  using V = Vec<BF16>;
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  int p[KMAX];
  float g[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    p[j] = -1;
    g[j] = 0.0f;
    if (j < k) {
      const int q = uniform(inv[(int64_t)t * k + j]);
      p[j] = q >= 0 && q < M ? q : -1;
      g[j] = w ? __uint_as_float(uniform(__float_as_uint(w[(int64_t)t * k + j]))) : 1.0f;
    }
  }
  for (int v0 = lane; v0 < nvec; v0 += NV * kWave) {
    uint4 r[NV][KMAX + 1];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = v0 + u * kWave;
      if (v < nvec) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (p[j] >= 0) r[u][j] = load_stream(y_perm + (int64_t)p[j] * nvec + v);
        if (y_sh) r[u][KMAX] = y_sh[(int64_t)t * nvec + v];
      }
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int v = v0 + u * kWave;
      if (v < nvec) {
        float acc[V::N];
#pragma unroll
        for (int i = 0; i < V::N; ++i) acc[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (p[j] >= 0) V::add(acc, g[j], r[u][j]);
        if (y_sh) V::add(acc, 1.0f, r[u][KMAX]);
        store_stream(y + (int64_t)t * nvec + v, V::pack(acc));
      }
    }
  }
}

// Any k up to 64: the slots are read inside the loop, four loads at a time.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void k_combine_anyk(const uint4 *__restrict__ y_perm, int T,
                                                           int k, int nvec,
                                                           const int32_t *__restrict__ inv,
                                                           const float *__restrict__ w,
                                                           const uint4 *__restrict__ y_sh, int64_t M,
                                                           uint4 *__restrict__ y) {
  using V = Vec<BF16>;
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  for (int v = lane; v < nvec; v += kWave) {
    float acc[V::N];
#pragma unroll
    for (int i = 0; i < V::N; ++i) acc[i] = 0.0f;
    int j = 0;
    for (; j + 4 <= k; j += 4) {
      uint4 r[4];
      float g[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = uniform(inv[(int64_t)t * k + j + u]);
        g[u] = w ? w[(int64_t)t * k + j + u] : 1.0f;
        ok[u] = p >= 0 && p < M;
        if (ok[u]) r[u] = y_perm[(int64_t)p * nvec + v];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ok[u]) V::add(acc, g[u], r[u]);
    }
    for (; j < k; ++j) {
      const int p = uniform(inv[(int64_t)t * k + j]);
      if (p >= 0 && p < M) V::add(acc, w ? w[(int64_t)t * k + j] : 1.0f, y_perm[(int64_t)p * nvec + v]);
    }
    if (y_sh) V::add(acc, 1.0f, y_sh[(int64_t)t * nvec + v]);
    y[(int64_t)t * nvec + v] = V::pack(acc);
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_unpermute_combine_rows(const void *y_perm, int64_t rows, moe_dtype dt,
                                                 int T, int k, int d, const int32_t *inv,
                                                 const float *topk_w, const void *y_shared, void *y,
                                                 hipStream_t stream) {
  if (T < 0 || k < 1 || d < 1 || rows < 0) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d % 8 != 0 || k > 64 || (int64_t)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if ((rows > 0 && !y_perm) || !inv || !y) return MOE_ERR_INVALID_ARG;   // topk_w NULL: every gate is 1
  if ((y_perm && !aligned16(y_perm)) || !aligned16(y) || (y_shared && !aligned16(y_shared)))
    return MOE_ERR_INVALID_ARG;
  const int elem = dt == MOE_F32 ? 4 : 2;
  const int nvec = (int)((int64_t)d * elem / 16);
  const int64_t M = rows;   // inv entries outside [0, rows) add nothing
  const dim3 grid((T + 3) / 4), block(kThreads);
  const uint4 *yp = static_cast<const uint4 *>(y_perm);
  const uint4 *ys = static_cast<const uint4 *>(y_shared);
  uint4 *out = static_cast<uint4 *>(y);
  constexpr int NV = kCombineNV;
  if (dt == MOE_BF16) {
    if (k == 1)
      k_combine<true, 1, NV><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
    else if (k == 2)
      k_combine<true, 2, NV><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
    else if (k <= 4)
      k_combine<true, 4, NV><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
    else if (k <= 8)   // k + 1 rows per vector already keep enough loads in flight
      k_combine<true, 8, 1><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
    else
      k_combine_anyk<true><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
  } else {
    if (k == 1)
      k_combine<false, 1, NV><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
    else if (k == 2)
      k_combine<false, 2, NV><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
    else if (k <= 4)
      k_combine<false, 4, NV><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
    else if (k <= 8)
      k_combine<false, 8, 1><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
    else
      k_combine_anyk<false><<<grid, block, 0, stream>>>(yp, T, k, nvec, inv, topk_w, ys, M, out);
  }
  return launch_status();
}

extern "C" moe_status moe_unpermute_combine(const void *y_perm, moe_dtype dt, int T, int k, int d,
                                            const int32_t *inv, const float *topk_w,
                                            const void *y_shared, void *y, hipStream_t stream) {
  if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
  if (!y_perm && T > 0) return MOE_ERR_INVALID_ARG;
  return moe_unpermute_combine_rows(y_perm, (int64_t)T * k, dt, T, k, d, inv, topk_w, y_shared, y,
                                    stream);
}
