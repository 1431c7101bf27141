// Router front end: the router product that turns token rows into logits,
// and the bias update of auxiliary-loss-free balancing.  Compiled with
// -ffp-contract=off: the bias update is exactly the operation sequence
// written here.
//
// Step 1 of the forward pass in "Expert parallelism" (zerotofrontier.app)
// computes the router before the top-k choice; "05 - Expert Parallelism
// (MoE)" (project-fortress), section "Load balancing", family (b), adjusts
// the choice with a per-expert bias that follows the experts' loads.
#include "common.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// c += a b^T over one 16-byte chunk of K per lane (8 bf16 or 4 fp32 values;
// the fp32 chunk is four K positions, taken in the same order for a and b).
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

constexpr int kTM = 64, kTN = 64;   // tokens x experts per workgroup
constexpr int kStages = 3;          // ring of 128-byte K slices
constexpr int kRowChunks = 8;       // 16-byte chunks per row per slice

// Chunk cc of staged row r sits at slot cc ^ key(r): any 16 consecutive rows
// read at one logical chunk (an MFMA operand fetch) hit every bank once.
__device__ __forceinline__ int swz(int r, int cc) {
  return r * kRowChunks + (cc ^ ((r & 7) ^ ((r >> 3) & 1)));
}

// logits[t][e] = sum_i x[t][i] wg[e][i] with fp32 accumulation.  Workgroup
// (bx, by) computes tokens 64 bx .. and experts 64 by ..; wave (wm, wn) one
// 32 x 32 block.  Waves 0-1 stage the token rows, waves 2-3 the router rows,
// 128 bytes of K per row per slice, with direct global-to-LDS loads two
// slices ahead.  Rows past T or E re-read the last row; their results are
// never stored.
template <bool BF16>
__global__ __launch_bounds__(256) void k_router_logits(const u32x4 *__restrict__ x, int T,
                                                       const u32x4 *__restrict__ wg, int E,
                                                       int kvec, float *__restrict__ logits) {
  constexpr int STAGE = (kTM + kTN) * kRowChunks;
  __shared__ u32x4 smem[kStages * STAGE];
  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int t0 = blockIdx.x * kTM, e0 = blockIdx.y * kTN;
  const bool a_loader = wave < 2;
  const int lw = wave & 1;
  const int ld_row = lane >> 3, ld_slot = lane & 7;
  const int KT = kvec / kRowChunks;

  // 8-row groups lw, lw + 2, lw + 4, lw + 6 of this wave's operand tile.
  uint32_t off[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = (lw + 2 * g) * 8 + ld_row;
    const int key = (r & 7) ^ ((r >> 3) & 1);
    int row = (a_loader ? t0 : e0) + r;
    const int lim = a_loader ? T : E;
    row = row < lim ? row : lim - 1;
    off[g] = (uint32_t)row * (uint32_t)kvec + (uint32_t)(ld_slot ^ key);
  }
  const u32x4 *base = a_loader ? x : wg;
  auto issue = [&](int kt) {
    u32x4 *stage = smem + (kt % kStages) * STAGE + (a_loader ? 0 : kTM * kRowChunks);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      __builtin_amdgcn_global_load_lds((const void *)(base + off[g] + (uint32_t)kt * kRowChunks),
                                       (__attribute__((address_space(3))) void *)(stage + (lw + 2 * g) * 64),
                                       16, 0, 0);
  };

  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  issue(0);
  if (KT > 1) issue(1);
  for (int kt = 0; kt < KT; ++kt) {
    // This wave's loads of slice kt are done once at most those of slice
    // kt + 1 (four) remain; the barrier then makes every wave's part visible
    // and frees the stage of slice kt - 1 for slice kt + 2.
    asm volatile("" ::: "memory");
    if (kt + 1 < KT)
      __builtin_amdgcn_s_waitcnt(0x0F70 | 4);   // vmcnt(4)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 2 < KT) issue(kt + 2);
    const u32x4 *As = smem + (kt % kStages) * STAGE;
    const u32x4 *Bs = As + kTM * kRowChunks;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cc = 2 * q + (lane >> 5);
      const u32x4 a = As[swz(wm * 32 + (lane & 31), cc)];
      const u32x4 b = Bs[swz(wn * 32 + (lane & 31), cc)];
      mma<BF16>(a, b, acc);
    }
  }

  // MFMA 32x32 output layout: lane l holds column l % 32 and, in register v,
  // row 8 (v / 4) + 4 (l / 32) + v % 4.
  const int e = e0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (t < T && e < E) logits[(size_t)t * E + e] = acc[v];
  }
}

// bias[e] += lr (avg - counts[e]), avg = fl(M) / fl(E), M = sum of counts;
// one rounding per written operation.  One block, E <= 1024.
__global__ __launch_bounds__(1024) void k_bias_update(const int32_t *__restrict__ counts, int E,
                                                      float lr, float *__restrict__ bias) {
  __shared__ long long part[16];
  const int e = threadIdx.x;
  const int c = e < E ? counts[e] : 0;
  long long s = c;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if ((e & 63) == 0) part[e >> 6] = s;
  __syncthreads();
  long long M = 0;
  for (int i = 0; i < 16; ++i) M += part[i];
  if (e < E) {
    const float avg = (float)M / (float)E;
    const float dev = avg - (float)c;
    const float step = lr * dev;
    bias[e] = bias[e] + step;
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_router_logits(const void *x, moe_dtype dt, int T, int d, const void *w_router,
                                        int E, float *logits, hipStream_t stream) {
  if (T < 0 || d < 1 || E < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  const int64_t elem = dt == MOE_F32 ? 4 : 2;
  if ((d * elem) % 128 != 0 || E > 65535 * kTN) return MOE_ERR_UNSUPPORTED;
  // 32-bit vector offsets into x and w_router.
  if ((int64_t)T * d * elem >= ((int64_t)1 << 36) || (int64_t)E * d * elem >= ((int64_t)1 << 36))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
  const int kvec = (int)(d * elem / 16);
  const dim3 grid((T + kTM - 1) / kTM, (E + kTN - 1) / kTN), block(256);
  if (dt == MOE_BF16)
    k_router_logits<true><<<grid, block, 0, stream>>>(static_cast<const u32x4 *>(x), T,
                                                      static_cast<const u32x4 *>(w_router), E, kvec,
                                                      logits);
  else
    k_router_logits<false><<<grid, block, 0, stream>>>(static_cast<const u32x4 *>(x), T,
                                                       static_cast<const u32x4 *>(w_router), E, kvec,
                                                       logits);
  return launch_status();
}

extern "C" moe_status moe_router_bias_update(const int32_t *counts, int E, float lr, float *bias,
                                             hipStream_t stream) {
  if (E < 1) return MOE_ERR_INVALID_ARG;
  if (E > 1024) return MOE_ERR_UNSUPPORTED;
  if (!counts || !bias) return MOE_ERR_INVALID_ARG;
  k_bias_update<<<dim3(1), dim3(1024), 0, stream>>>(counts, E, lr, bias);
  return launch_status();
}
