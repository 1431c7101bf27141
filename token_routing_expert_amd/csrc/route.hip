// Route (top-k gating, optionally group-limited), the pinned sigmoid, and the
// send-count matrix.  Compiled with -ffp-contract=off: the pinned sigmoid must
// be exactly the operation sequence written here.
//
// Step 1 of the forward pass in "Expert parallelism" (zerotofrontier.app),
// with DeepSeek-V3's node-limited selection from its section "What DeepSeek-V3
// did about it"; the send-count matrix is the one of its section "A dispatch
// you can check by hand".
#include <float.h>
#include <math.h>

#include "common.hpp"

namespace moe {
namespace {

// exp(y) for y <= 0: Cody & Waite reduction y = n ln2 + r with ln2 split into
// a 12-significant-bit head (n * head is exact) and a tail, the degree-7
// Taylor polynomial of exp(r) with coefficients fl(1/i!) in Horner form, and
// an exact scaling by 2^n.  Inputs below -87 (results below the normal
// range) give 0.  Each line is one correctly rounded fp32 operation.
__device__ __forceinline__ float pinned_exp_nonpos(float y) {
  constexpr float kLog2e = (float)1.4426950408889634074;
  constexpr float kLn2Hi = 2839.0f / 4096.0f;
  constexpr float kLn2Lo = (float)(0.69314718055994530942 - 2839.0 / 4096.0);
  constexpr float c2 = (float)(1.0 / 2), c3 = (float)(1.0 / 6), c4 = (float)(1.0 / 24);
  constexpr float c5 = (float)(1.0 / 120), c6 = (float)(1.0 / 720), c7 = (float)(1.0 / 5040);
  if (y < -87.0f) return 0.0f;
  const float n = rintf(y * kLog2e);
  float r = fmaf(-n, kLn2Hi, y);
  r = fmaf(-n, kLn2Lo, r);
  float p = c7;
  p = fmaf(p, r, c6);
  p = fmaf(p, r, c5);
  p = fmaf(p, r, c4);
  p = fmaf(p, r, c3);
  p = fmaf(p, r, c2);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

__device__ __forceinline__ float pinned_sigmoid(float x) {
  const float t = pinned_exp_nonpos(-fabsf(x));
  const float den = 1.0f + t;
  return x >= 0.0f ? 1.0f / den : t / den;
}

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

constexpr int kNone = 0x7fffffff;

// (key, id) lexicographic order: larger key first, then lower id; kNone last.
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ia != kNone && (ib == kNone || ka > kb || (ka == kb && ia < ib));
}

__device__ __forceinline__ void wave_argmax(float &k, int &i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ok = __shfl_xor(k, off);
    const int oi = __shfl_xor(i, off);
    if (better(ok, oi, k, i)) { k = ok; i = oi; }
  }
}

// One wave per token.  Lane l holds experts l, l + 64, ... (NPER of them), so
// each pass over the logits row is one coalesced 256-byte load.  With a bias
// (auxiliary-loss-free balancing, "05 - Expert Parallelism (MoE)", section
// "Load balancing"), the choice -- group scores included -- is taken on the
// keys fl32(logit + bias) and the gates on the unbiased logits.
template <int NPER>
__global__ __launch_bounds__(256) void k_route_topk(const float *__restrict__ logits,
                                                    const float *__restrict__ bias, int T, int E,
                                                    int k, int gating, int renorm, int n_groups,
                                                    int topk_groups, int32_t *__restrict__ ids,
                                                    float *__restrict__ w) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (t >= T) return;
  const float *row = logits + (size_t)t * E;

  float key[NPER], lg[NPER];
  uint32_t cand = 0;  // bit i: slot i holds a selectable expert
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = i * kWave + lane;
    key[i] = -INFINITY;
    lg[i] = -INFINITY;
    if (e < E) {
      lg[i] = row[e] + 0.0f;  // -0 becomes +0
      key[i] = bias ? (row[e] + bias[e]) + 0.0f : lg[i];
      cand |= 1u << i;
    }
  }

  if (n_groups > 1) {
    // Group score: fp32 sum of the two largest pinned-sigmoid affinities.
    const int gs = E / n_groups;
    float aff[NPER];
    int grp[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = i * kWave + lane;
      aff[i] = pinned_sigmoid(key[i]);
      grp[i] = (cand >> i & 1u) ? e / gs : -1;
    }
    float my_score = -INFINITY;  // lane g keeps group g's score
    for (int g = 0; g < n_groups; ++g) {
      float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPER; ++i) {
        if (grp[i] == g) {
          const float a = aff[i];
          if (a > a1) { a2 = a1; a1 = a; }
          else if (a > a2) { a2 = a; }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float b1 = __shfl_xor(a1, off);
        const float b2 = __shfl_xor(a2, off);
        const float hi = fmaxf(a1, b1);
        a2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
        a1 = hi;
      }
      if (lane == g) my_score = a1 + a2;
    }
    // Keep the topk_groups best groups (higher score, then lower group id).
    uint64_t kept = 0;
    bool open = lane < n_groups;
    for (int r = 0; r < topk_groups; ++r) {
      float bk = my_score;
      int bi = open ? lane : kNone;
      wave_argmax(bk, bi);
      kept |= 1ull << bi;
      if (lane == bi) open = false;
    }
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (grp[i] >= 0 && !((kept >> grp[i]) & 1ull)) cand &= ~(1u << i);
  }

  // k rounds of a wave-wide argmax; lane j keeps the j-th pick and its
  // unbiased logit (fetched from the lane that holds the winner).
  int my_id = kNone;
  float my_key = -INFINITY, first_key = -INFINITY;
  for (int j = 0; j < k; ++j) {
    float bk = -INFINITY;
    int bi = kNone;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = i * kWave + lane;
      if ((cand >> i & 1u) && (bi == kNone || key[i] > bk)) { bk = key[i]; bi = e; }
    }
    wave_argmax(bk, bi);
    float bl = bk;
    if (bias) {
      float mine = 0.0f;
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (i == (bi >> 6)) mine = lg[i];
      bl = __shfl(mine, bi & (kWave - 1));
    }
    if (lane == (bi & (kWave - 1))) cand &= ~(1u << (bi >> 6));
    if (lane == j) { my_id = bi; my_key = bl; }
    if (j == 0) first_key = bl;
  }

  float v = 0.0f, denom = 1.0f;
  if (gating == MOE_SOFTMAX) {
    if (renorm) {
      v = lane < k ? expf(my_key - first_key) : 0.0f;
      denom = wave_sum(v);
    } else {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (i * kWave + lane < E) m = fmaxf(m, lg[i]);
      m = wave_max(m);
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (i * kWave + lane < E) s += expf(lg[i] - m);
      denom = wave_sum(s);
      v = lane < k ? expf(my_key - m) : 0.0f;
    }
  } else {
    v = lane < k ? pinned_sigmoid(my_key) : 0.0f;
    if (renorm) denom = wave_sum(v);
  }
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = v / denom;
  }
}

__global__ void k_sigmoid_pinned(const float *__restrict__ x, float *__restrict__ y, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    y[i] = pinned_sigmoid(x[i]);
}

// One block per source rank: an LDS histogram over destination ranks.
__global__ __launch_bounds__(256) void k_send_counts(const int32_t *__restrict__ ids, int T_loc,
                                                     int k, int E, int n_ep,
                                                     int32_t *__restrict__ S) {
  extern __shared__ int hist[];
  const int s = blockIdx.x;
  for (int q = threadIdx.x; q < n_ep; q += blockDim.x) hist[q] = 0;
  __syncthreads();
  const int64_t n = (int64_t)T_loc * k;
  const int32_t *src = ids + (int64_t)s * n;
  for (int64_t a = threadIdx.x; a < n; a += blockDim.x) {
    const int e = src[a];
    if (e >= 0 && e < E) atomicAdd(&hist[(int)(((int64_t)e * n_ep) / E)], 1);
  }
  __syncthreads();
  for (int q = threadIdx.x; q < n_ep; q += blockDim.x) S[(int64_t)s * n_ep + q] = hist[q];
}

}  // namespace
}  // namespace moe

using namespace moe;

static moe_status route_topk(const float *logits, const float *bias, int T, int E, int k,
                             moe_gating gating, int renormalize, int n_groups, int topk_groups,
                             int32_t *topk_ids, float *topk_w, hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || n_groups < 1 || topk_groups < 1 ||
      topk_groups > n_groups || E % n_groups != 0)
    return MOE_ERR_INVALID_ARG;
  if (gating != MOE_SOFTMAX && gating != MOE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (n_groups > 1 && (E / n_groups < 2 || topk_groups * (E / n_groups) < k))
    return MOE_ERR_INVALID_ARG;
  if (E > 1024 || k > 16 || n_groups > 64) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  const dim3 grid((T + 3) / 4), block(256);
  const int rn = renormalize ? 1 : 0;
  if (E <= 64)
    k_route_topk<1><<<grid, block, 0, stream>>>(logits, bias, T, E, k, gating, rn, n_groups, topk_groups, topk_ids, topk_w);
  else if (E <= 128)
    k_route_topk<2><<<grid, block, 0, stream>>>(logits, bias, T, E, k, gating, rn, n_groups, topk_groups, topk_ids, topk_w);
  else if (E <= 256)
    k_route_topk<4><<<grid, block, 0, stream>>>(logits, bias, T, E, k, gating, rn, n_groups, topk_groups, topk_ids, topk_w);
  else if (E <= 512)
    k_route_topk<8><<<grid, block, 0, stream>>>(logits, bias, T, E, k, gating, rn, n_groups, topk_groups, topk_ids, topk_w);
  else
    k_route_topk<16><<<grid, block, 0, stream>>>(logits, bias, T, E, k, gating, rn, n_groups, topk_groups, topk_ids, topk_w);
  return launch_status();
}

extern "C" moe_status moe_route_topk(const float *logits, int T, int E, int k, moe_gating gating,
                                     int renormalize, int n_groups, int topk_groups,
                                     int32_t *topk_ids, float *topk_w, hipStream_t stream) {
  return route_topk(logits, nullptr, T, E, k, gating, renormalize, n_groups, topk_groups, topk_ids,
                    topk_w, stream);
}

extern "C" moe_status moe_route_topk_biased(const float *logits, const float *bias, int T, int E,
                                            int k, moe_gating gating, int renormalize,
                                            int n_groups, int topk_groups, int32_t *topk_ids,
                                            float *topk_w, hipStream_t stream) {
  if (T > 0 && !bias) return MOE_ERR_INVALID_ARG;
  return route_topk(logits, bias, T, E, k, gating, renormalize, n_groups, topk_groups, topk_ids,
                    topk_w, stream);
}

extern "C" moe_status moe_sigmoid_pinned(const float *x, float *y, int64_t n, hipStream_t stream) {
  if (n < 0) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  if (!x || !y) return MOE_ERR_INVALID_ARG;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  k_sigmoid_pinned<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(x, y, n);
  return launch_status();
}

extern "C" moe_status moe_send_counts(const int32_t *topk_ids, int T, int k, int E, int n_ep,
                                      int32_t *send_counts, hipStream_t stream) {
  if (T < 0 || k < 1 || E < 1 || n_ep < 1 || T % n_ep != 0 || E % n_ep != 0)
    return MOE_ERR_INVALID_ARG;
  if (n_ep > 1024) return MOE_ERR_UNSUPPORTED;
  if (!send_counts || (T > 0 && !topk_ids)) return MOE_ERR_INVALID_ARG;
  // T == 0 still launches: every row is empty and the kernel writes zeros.
  k_send_counts<<<dim3(n_ep), dim3(256), sizeof(int) * n_ep, stream>>>(topk_ids, T / n_ep, k, E,
                                                                        n_ep, send_counts);
  return launch_status();
}

extern "C" const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or option not implemented";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error at launch";
  }
  return "unknown moe_status";
}
