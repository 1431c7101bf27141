// Backward of the combine and of the gates.
//
// In the backward pass the combine's gradient goes out to the expert rows the
// way the dispatch did ("Expert parallelism", section "How many bytes
// move").  From y[t] = sum_j w[t,j] y_perm[inv[t k + j]] (+ y_shared[t]):
//
//   dy_perm[inv[t k + j]] = w[t,j] dy[t]
//   dgate[t,j]            = dy[t] . y_perm[inv[t k + j]]
//   dy_shared[t]          = dy[t]
//
// and the gate gradient reaches the logits through the gate formula of the
// route (the choice itself is piecewise constant, and the balancing bias is
// outside the gradient: "05 - Expert Parallelism (MoE)", section "Load
// balancing"), and from the logits through the router product,
// logits = x w_router^T, to x and w_router.
#include "common.hpp"
#include "gemm_common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <bool BF16>
struct Row16;

// 16 bytes = 8 bf16.
template <>
struct Row16<true> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4 &v, float *f) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(u[i]);
      f[2 * i + 1] = bf16_hi(u[i]);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float *f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};

// 16 bytes = 4 fp32.
template <>
struct Row16<false> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const uint4 &v, float *f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ uint4 pack(const float *f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

// Sum over the 64 lanes in a fixed butterfly order (the same bits every run).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One wave per token, KMAX slots at a time: the token's gradient row is read
// once per slot group and each of its k packed rows once.  Every lane keeps
// a partial dot product per slot over the 16-byte vectors it handles (in
// order), then the wave adds the partials in a fixed order.
template <bool BF16, int KMAX>
__global__ __launch_bounds__(kThreads) void k_combine_bwd(
    const uint4 *__restrict__ dy, int T, int k, int nvec, const int32_t *__restrict__ inv,
    const float *__restrict__ w, const uint4 *__restrict__ y_perm, int64_t M,
    uint4 *__restrict__ dy_perm, float *__restrict__ dgate, uint4 *__restrict__ dy_sh) {
  using V = Row16<BF16>;
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  for (int j0 = 0; j0 < k; j0 += KMAX) {
    int p[KMAX];
    float g[KMAX], dot[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      p[j] = -1;
      g[j] = 0.0f;
      dot[j] = 0.0f;
      if (j0 + j < k) {
        const int q = uniform(inv[(int64_t)t * k + j0 + j]);
        p[j] = q >= 0 && q < M ? q : -1;
        g[j] = __uint_as_float(uniform(__float_as_uint(w[(int64_t)t * k + j0 + j])));
      }
    }
    for (int v = lane; v < nvec; v += kWave) {
      const uint4 dv = dy[(int64_t)t * nvec + v];
      uint4 yv[KMAX];
      if (dgate) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (p[j] >= 0) yv[j] = y_perm[(int64_t)p[j] * nvec + v];
      }
      float df[V::N];
      V::unpack(dv, df);
      if (dy_sh && j0 == 0) dy_sh[(int64_t)t * nvec + v] = dv;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (p[j] < 0) continue;
        float o[V::N];
#pragma unroll
        for (int i = 0; i < V::N; ++i) o[i] = g[j] * df[i];
        dy_perm[(int64_t)p[j] * nvec + v] = V::pack(o);
        if (dgate) {
          float yf[V::N];
          V::unpack(yv[j], yf);
#pragma unroll
          for (int i = 0; i < V::N; ++i) dot[j] += df[i] * yf[i];
        }
      }
    }
    if (dgate) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        const float s = wave_sum(dot[j]);
        if (lane == 0 && j0 + j < k) dgate[(int64_t)t * k + j0 + j] = s;
      }
    }
  }
}

// One wave per token.  Lane j < k holds slot j: its expert c_j, gate w_j,
// gate gradient dw_j and logit l_j.  Then, with dot = sum_j w_j dw_j:
//   softmax, renormalised:  dl[c_j] = w_j (dw_j - dot)
//   softmax, not renorm.:   dl[e]   = P_e ([e = c_j] dw_j - dot),  P = softmax(l)
//   sigmoid, renormalised:  dl[c_j] = s_j (1 - s_j) (dw_j - dot) / sum_i s_i
//   sigmoid, not renorm.:   dl[c_j] = s_j (1 - s_j) dw_j
// with s_j = 1 / (1 + e^-l_j); every other entry of the row is 0.
__global__ __launch_bounds__(kThreads) void k_gate_bwd(const float *__restrict__ logits,
                                                       const int32_t *__restrict__ ids,
                                                       const float *__restrict__ w,
                                                       const float *__restrict__ dw, int T, int E,
                                                       int k, int gating, int renorm,
                                                       float *__restrict__ dlogits) {
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const float *l = logits + (int64_t)t * E;
  int c = -1;
  float wj = 0.0f, dwj = 0.0f, lj = 0.0f;
  if (lane < k) {
    c = ids[(int64_t)t * k + lane];
    c = c >= 0 && c < E ? c : -1;
    wj = w[(int64_t)t * k + lane];
    dwj = dw[(int64_t)t * k + lane];
    lj = c >= 0 ? l[c] : 0.0f;
  }
  const float dot = wave_sum(wj * dwj);
  const bool softmax = gating == MOE_SOFTMAX;
  float val = 0.0f;   // this slot's entry (softmax not renormalised: its P_c dw part)
  float mx = 0.0f, inv_sum = 0.0f;
  if (softmax && !renorm) {
    float m = -INFINITY;
    for (int e = lane; e < E; e += kWave) m = fmaxf(m, l[e]);
    mx = wave_max(m);
    float s = 0.0f;
    for (int e = lane; e < E; e += kWave) s += __expf(l[e] - mx);
    inv_sum = 1.0f / wave_sum(s);
    val = __expf(lj - mx) * inv_sum * dwj;
  } else if (softmax) {
    val = wj * (dwj - dot);
  } else {
    const float s = 1.0f / (1.0f + __expf(-lj));
    if (renorm) {
      const float ssum = wave_sum(lane < k ? s : 0.0f);
      val = s * (1.0f - s) * (dwj - dot) / ssum;
    } else {
      val = s * (1.0f - s) * dwj;
    }
  }
  float *out = dlogits + (int64_t)t * E;
  for (int e = lane; e < E; e += kWave) {
    float r = softmax && !renorm ? -__expf(l[e] - mx) * inv_sum * dot : 0.0f;
    for (int j = 0; j < k; ++j) {
      const int cj = __shfl(c, j);
      const float vj = __shfl(val, j);
      if (cj == e) r += vj;
    }
    out[e] = r;
  }
}

// The router product's backward starts from a bf16 copy of dlogits (the
// products' operand type); the same launch writes the one-segment offsets
// [0, T] the grouped products take.
__global__ __launch_bounds__(kThreads) void k_dlogits_bf16(const float *__restrict__ dl, int64_t n,
                                                           int T, uint16_t *__restrict__ out,
                                                           int32_t *__restrict__ offsets) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = (uint16_t)f32_to_bf16_rne(dl[i]);
  if (i == 0) {
    offsets[0] = 0;
    offsets[1] = T;
  }
}

inline size_t router_ws_split(int T, int E) {   // bytes of the bf16 copy, rounded up to 256
  return (((size_t)T * E * 2) + 255) / 256 * 256;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_router_backward_workspace_bytes(int T, int E) {
  if (T < 0 || E < 1) return 0;
  return router_ws_split(T, E) + 256;
}

extern "C" moe_status moe_router_backward(const float *dlogits, const void *x, moe_dtype dt, int T,
                                          int d, const void *w_router, int E, void *dx,
                                          void *dw_router, void *workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  if (T < 0 || d < 1 || E < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  // The ping-pong product tiles: 256-wide E and d, at least 96 tokens.
  if (E % 256 != 0 || d % 256 != 0 || (T > 0 && T < 96)) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * d * 2 >= ((int64_t)1 << 32) || (int64_t)T * E * 2 >= ((int64_t)1 << 32))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0 || (!dx && !dw_router)) return MOE_OK;
  if (!dlogits || !x || !w_router || !workspace) return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe_router_backward_workspace_bytes(T, E)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(workspace) || (dx && !aligned16(dx)) ||
      (dw_router && !aligned16(dw_router)))
    return MOE_ERR_INVALID_ARG;
  uint16_t *dl = static_cast<uint16_t *>(workspace);
  int32_t *offsets = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + router_ws_split(T, E));
  const int64_t n = (int64_t)T * E;
  k_dlogits_bf16<<<dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream>>>(
      dlogits, n, T, dl, offsets);
  // dx += dlogits w_router: [T, E] x [E, d] (w_router row-major is [K, N]).
  if (dx && !launch_dgrad_pp(4, dl, T, E, d, offsets, 1, w_router, dx, nullptr, stream))
    return MOE_ERR_UNSUPPORTED;
  // dw_router = dlogits^T x: one segment of T rows, [E, d].
  if (dw_router && !launch_weight_grad(dl, x, T, E, d, offsets, 1, dw_router, stream))
    return MOE_ERR_UNSUPPORTED;
  return launch_status();
}

extern "C" moe_status moe_combine_backward(const void *dy, moe_dtype dt, int T, int k, int d,
                                           const int32_t *inv, const float *topk_w,
                                           const void *y_perm, void *dy_perm, float *dgate,
                                           void *dy_shared, hipStream_t stream) {
  if (T < 0 || k < 1 || d < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d % 8 != 0 || k > 64 || (int64_t)T * k >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!dy || !inv || !topk_w || !dy_perm) return MOE_ERR_INVALID_ARG;
  if ((dgate == nullptr) != (y_perm == nullptr)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(dy) || !aligned16(dy_perm) || (y_perm && !aligned16(y_perm)) ||
      (dy_shared && !aligned16(dy_shared)))
    return MOE_ERR_INVALID_ARG;
  const int elem = dt == MOE_F32 ? 4 : 2;
  const int nvec = (int)((int64_t)d * elem / 16);
  const int64_t M = (int64_t)T * k;
  const dim3 grid((T + 3) / 4), block(kThreads);
  const uint4 *dyv = static_cast<const uint4 *>(dy);
  const uint4 *yp = static_cast<const uint4 *>(y_perm);
  uint4 *dyp = static_cast<uint4 *>(dy_perm);
  uint4 *dys = static_cast<uint4 *>(dy_shared);
#define MOE_COMBINE_BWD(B, KM) \
  k_combine_bwd<B, KM><<<grid, block, 0, stream>>>(dyv, T, k, nvec, inv, topk_w, yp, M, dyp, dgate, dys)
  if (dt == MOE_BF16) {
    if (k == 1) MOE_COMBINE_BWD(true, 1);
    else if (k == 2) MOE_COMBINE_BWD(true, 2);
    else if (k <= 4) MOE_COMBINE_BWD(true, 4);
    else MOE_COMBINE_BWD(true, 8);
  } else {
    if (k == 1) MOE_COMBINE_BWD(false, 1);
    else if (k == 2) MOE_COMBINE_BWD(false, 2);
    else if (k <= 4) MOE_COMBINE_BWD(false, 4);
    else MOE_COMBINE_BWD(false, 8);
  }
#undef MOE_COMBINE_BWD
  return launch_status();
}

extern "C" moe_status moe_gate_backward(const float *logits, const int32_t *topk_ids,
                                        const float *topk_w, const float *dgate, int T, int E,
                                        int k, moe_gating gating, int renormalize, float *dlogits,
                                        hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (gating != MOE_SOFTMAX && gating != MOE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (k > 64 || E > 4096) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w || !dgate || !dlogits) return MOE_ERR_INVALID_ARG;
  k_gate_bwd<<<dim3((T + 3) / 4), dim3(kThreads), 0, stream>>>(logits, topk_ids, topk_w, dgate, T,
                                                               E, k, (int)gating, renormalize ? 1 : 0,
                                                               dlogits);
  return launch_status();
}
