// One expert's SwiGLU MLP over few rows, with each reduction split over many
// workgroups: the shared expert of a decode step.
//
// "05 -- Expert Parallelism (MoE)" (project-fortress), "Fine-grained vs
// coarse experts": DeepSeek-V3 adds one always-active shared expert to its
// 256 routed ones, a SwiGLU MLP of 3 d ffn weights ("Expert parallelism",
// zerotofrontier.app, "A worked example at DeepSeek-V3's shape") that every
// token goes through; and at decode a layer's time is the weights it reads
// (the first page, "The serving asymmetry").  Tiling such a product
// by output columns alone gives one workgroup per 64-256 weight rows, a few
// dozen for the whole GPU, each streaming the full reduction length; the
// split here gives every workgroup one K range of one 64-column tile, so
// hundreds of workgroups stream the weights at once.
//
//   pass 1  P[s, m, n] = sum over k in K range s of A[m, k] W[n, k]   (fp32)
//   pass 2  sum over s in order 0, 1, ... (a fixed order: the result does
//           not depend on the schedule), then SwiGLU (gate/up) or a plain
//           cast (down), rounded once to bf16.
//
// A (rows) and W (weights) are bf16, row-major and K-contiguous.  A
// workgroup streams its K range in 64-byte slices of the token rows and of
// its 64 weight rows into LDS with direct buffer-to-LDS loads (each load
// instruction fills 16 rows x 64 bytes; a ring of 4 stages, 3 slices ahead),
// and every wave reads its MFMA operands from there: lane l holds row l % 32
// and K positions 8 (l / 32) .. + 7 of a 16-deep K step.  Each weight byte
// thus crosses the memory system once per workgroup, in whole 64-byte row
// segments.
#include "common.hpp"
#include "gemm_common.hpp"

namespace moe {
namespace {

constexpr int kDenseBN = 64;       // output columns (weight rows) per workgroup
constexpr int kDenseMaxRows = 256;  // 8 row blocks of 32, two per wave

__device__ __forceinline__ void mma_bf16(const u32x4 &a, const u32x4 &b, f32x16 &c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                              c, 0, 0, 0);
}

// Stage position (16-byte units) of chunk cc (0..3) of row r in a stage of
// 64-byte rows: 16 consecutive rows at one chunk cover all 64 banks once.
__device__ __forceinline__ int dense_slot(int r, int cc) { return r * 4 + (cc ^ ((r >> 2) & 3)); }

// Workgroup (n tile blockIdx.x, K range blockIdx.y), 4 waves; wave w owns
// row blocks w and w + 4 (the second only when RB == 2) and both 32-column
// blocks of the tile.  AR = 128 RB token rows are staged per slice (rows
// past M re-read row M - 1 and are not stored), with the tile's 64 weight
// rows.  Host guarantees: 1 <= M <= AR, N % 64 == 0, kchunk = K / S a
// multiple of 32, gridDim = (N / 64, S).
template <int RB>
__global__ __launch_bounds__(256) void k_dense_partial(const u32x4 *__restrict__ A, int M, int K,
                                                       const u32x4 *__restrict__ W, int N, int kchunk,
                                                       float *__restrict__ P) {
  constexpr int CPR = 4, RPI = 16, S = 4, DIST = S - 1;
  constexpr int AR = 128 * RB, BRW = kDenseBN;
  constexpr int ASTAGE = AR * CPR, STAGE = (AR + BRW) * CPR;
  constexpr int NLA = AR / RPI / 4, NLB = BRW / RPI / 4;   // loads per wave per slice
  __shared__ u32x4 smem[S * STAGE];

  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int nrb = (M + 31) / 32;
  const int n0 = blockIdx.x * kDenseBN, s = blockIdx.y;
  const int kvec = K / 8;                       // 16-byte chunks per row
  const int KT = kchunk / 32;                   // 64-byte slices in the K range
  const uint32_t kbase = (uint32_t)(s * (kchunk / 8)) * 16u;   // byte offset of the range in a row

  // Load lane mapping: lane l fills row l / 4 of a 16-row group, slot l % 4,
  // which holds global chunk (l % 4) ^ key of that row.
  const int ld_row = lane / CPR, ld_slot = lane % CPR;
  const uint32_t key = (uint32_t)((ld_row >> 2) & 3);
  uint32_t aoff[NLA], boff[NLB];
#pragma unroll
  for (int r = 0; r < NLA; ++r) {
    int row = (wave + 4 * r) * RPI + ld_row;
    row = row < M ? row : M - 1;
    aoff[r] = ((uint32_t)row * (uint32_t)kvec + ((uint32_t)ld_slot ^ key)) * 16u + kbase;
  }
#pragma unroll
  for (int r = 0; r < NLB; ++r)
    boff[r] = ((uint32_t)(n0 + (wave + 4 * r) * RPI + ld_row) * (uint32_t)kvec + ((uint32_t)ld_slot ^ key)) * 16u +
              kbase;
  const uint32_t a_bytes = (uint32_t)M * (uint32_t)kvec * 16u;
  const uint32_t b_bytes = (uint32_t)N * (uint32_t)kvec * 16u;
  auto issue = [&](int kt) {
    u32x4 *stage = smem + (kt % S) * STAGE;
#pragma unroll
    for (int r = 0; r < NLA; ++r)
      buffer_load_lds16(A, a_bytes, stage + (wave + 4 * r) * 64, aoff[r], (uint32_t)kt * 64u);
#pragma unroll
    for (int r = 0; r < NLB; ++r)
      buffer_load_lds16(W, b_bytes, stage + ASTAGE + (wave + 4 * r) * 64, boff[r], (uint32_t)kt * 64u);
  };

  f32x16 acc[RB][2];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const bool live[2] = {wave < nrb, wave + 4 < nrb};

  for (int j = 0; j < DIST && j < KT; ++j) issue(j);
  // Slice kt: wait for this wave's loads of it (later slices stay in flight),
  // barrier, refill the stage of slice kt - 1 (every wave's MFMAs consumed
  // their reads of it before this barrier), then two K steps of MFMAs.
  for (int kt = 0; kt < KT; ++kt) {
    const int ahead = (KT - 1 < kt + DIST - 1 ? KT - 1 : kt + DIST - 1) - kt;
    wait_vmcnt(ahead * (NLA + NLB));
    __builtin_amdgcn_s_barrier();
    if (kt + DIST < KT) issue(kt + DIST);
    const u32x4 *st = smem + (kt % S) * STAGE;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int cc = 2 * q + (lane >> 5);
      const u32x4 fb0 = st[ASTAGE + dense_slot(lane & 31, cc)];
      const u32x4 fb1 = st[ASTAGE + dense_slot(32 + (lane & 31), cc)];
#pragma unroll
      for (int i = 0; i < RB; ++i)
        if (live[i]) {
          const u32x4 fa = st[dense_slot((wave + 4 * i) * 32 + (lane & 31), cc)];
          mma_bf16(fa, fb0, acc[i][0]);
          mma_bf16(fa, fb1, acc[i][1]);
        }
    }
  }

  // MFMA 32x32 output layout: lane l holds column l % 32 and, in register v,
  // row 8 (v / 4) + 4 (l / 32) + v % 4 of the block.
  float *out = P + (int64_t)s * M * N;
  const int kh = lane >> 5, lr = lane & 31;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    if (!live[i]) continue;
    const int rb = (wave + 4 * i) * 32;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = rb + 8 * (v >> 2) + 4 * kh + (v & 3);
        if (row < M) out[(int64_t)row * N + n0 + 32 * j + lr] = acc[i][j][v];
      }
  }
}

// h[m, f] = SiLU(g) u with g = sum_s P[s, m, f], u = sum_s P[s, m, ffn + f];
// gu (optional) keeps (g, u) in bf16 as a [M, 2 ffn] row.  Four columns per
// thread.
__global__ __launch_bounds__(256) void k_dense_reduce_swiglu(const float *__restrict__ P, int S, int M,
                                                             int ffn, uint16_t *__restrict__ h,
                                                             uint16_t *__restrict__ gu) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;   // group of 4 columns
  const int64_t nq = (int64_t)M * ffn / 4;
  if (q >= nq) return;
  const int64_t m = q / (ffn / 4);
  const int f = (int)(q - m * (ffn / 4)) * 4;
  const int64_t N = 2 * (int64_t)ffn;
  float g[4] = {0, 0, 0, 0}, u[4] = {0, 0, 0, 0};
  for (int s = 0; s < S; ++s) {
    const float4 pg = *reinterpret_cast<const float4 *>(P + ((int64_t)s * M + m) * N + f);
    const float4 pu = *reinterpret_cast<const float4 *>(P + ((int64_t)s * M + m) * N + ffn + f);
    g[0] += pg.x; g[1] += pg.y; g[2] += pg.z; g[3] += pg.w;
    u[0] += pu.x; u[1] += pu.y; u[2] += pu.z; u[3] += pu.w;
  }
  uint2 hv;
  hv.x = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
  hv.y = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
  *reinterpret_cast<uint2 *>(h + m * ffn + f) = hv;
  if (gu) {
    *reinterpret_cast<uint2 *>(gu + m * N + f) = make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]));
    *reinterpret_cast<uint2 *>(gu + m * N + ffn + f) =
        make_uint2(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]));
  }
}

// y[m, n] = sum_s P[s, m, n], four columns per thread.
__global__ __launch_bounds__(256) void k_dense_reduce(const float *__restrict__ P, int S, int M, int N,
                                                      uint16_t *__restrict__ y) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nq = (int64_t)M * N / 4;
  if (q >= nq) return;
  float a[4] = {0, 0, 0, 0};
  for (int s = 0; s < S; ++s) {
    const float4 p = *reinterpret_cast<const float4 *>(P + (int64_t)s * M * N + 4 * q);
    a[0] += p.x; a[1] += p.y; a[2] += p.z; a[3] += p.w;
  }
  *reinterpret_cast<uint2 *>(y + 4 * q) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
}

// Splits of a K-deep reduction over N / 64 column tiles: enough workgroups
// for two per CU (512), at most 16 splits, each split a multiple of 32 deep
// (whole 64-byte slices).
int dense_splits(int K, int N) {
  const int tiles = N / kDenseBN;
  int s = (512 + tiles - 1) / tiles;
  s = s < 1 ? 1 : (s > 16 ? 16 : s);
  while (s > 1 && K % (32 * s) != 0) --s;
  return s;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_dense_swiglu_workspace_bytes(int M, int d, int ffn) {
  if (M < 1 || d < 1 || ffn < 1) return 16;
  const size_t p1 = (size_t)dense_splits(d, 2 * ffn) * (size_t)M * 2 * (size_t)ffn;
  const size_t p2 = (size_t)dense_splits(ffn, d) * (size_t)M * (size_t)d;
  return (p1 > p2 ? p1 : p2) * sizeof(float);
}

extern "C" moe_status moe_dense_swiglu(const void *x, moe_dtype dt, int M, int d, int ffn,
                                       const void *w13, const void *w2, void *h, void *gu, void *y,
                                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (M < 0 || d < 1 || ffn < 1) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_BF16 || M > kDenseMaxRows || d % 64 != 0 || ffn % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (!x || !w13 || !w2 || !h || !y || !workspace) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(w2) || !aligned16(h) || !aligned16(y) ||
      !aligned16(workspace) || (gu && !aligned16(gu)))
    return MOE_ERR_INVALID_ARG;
  if (workspace_bytes < moe_dense_swiglu_workspace_bytes(M, d, ffn)) return MOE_ERR_INVALID_ARG;
  float *P = static_cast<float *>(workspace);

  // Gate/up: N = 2 ffn weight rows (gate rows, then up rows), K = d.
  const int s1 = dense_splits(d, 2 * ffn);
  if (M <= 128)
    k_dense_partial<1><<<dim3(2 * ffn / kDenseBN, s1), dim3(256), 0, stream>>>(
        static_cast<const u32x4 *>(x), M, d, static_cast<const u32x4 *>(w13), 2 * ffn, d / s1, P);
  else
    k_dense_partial<2><<<dim3(2 * ffn / kDenseBN, s1), dim3(256), 0, stream>>>(
        static_cast<const u32x4 *>(x), M, d, static_cast<const u32x4 *>(w13), 2 * ffn, d / s1, P);
  const int64_t q1 = (int64_t)M * ffn / 4;
  k_dense_reduce_swiglu<<<dim3((unsigned)((q1 + 255) / 256)), dim3(256), 0, stream>>>(
      P, s1, M, ffn, static_cast<uint16_t *>(h), static_cast<uint16_t *>(gu));
  // Down: N = d, K = ffn.
  const int s2 = dense_splits(ffn, d);
  if (M <= 128)
    k_dense_partial<1><<<dim3(d / kDenseBN, s2), dim3(256), 0, stream>>>(
        static_cast<const u32x4 *>(h), M, ffn, static_cast<const u32x4 *>(w2), d, ffn / s2, P);
  else
    k_dense_partial<2><<<dim3(d / kDenseBN, s2), dim3(256), 0, stream>>>(
        static_cast<const u32x4 *>(h), M, ffn, static_cast<const u32x4 *>(w2), d, ffn / s2, P);
  const int64_t q2 = (int64_t)M * d / 4;
  k_dense_reduce<<<dim3((unsigned)((q2 + 255) / 256)), dim3(256), 0, stream>>>(P, s2, M, d,
                                                                             static_cast<uint16_t *>(y));
  return launch_status();
}
