// Step 1 of VSA: cube mean-pool (or the max-pool variant).
//
// VSA summary page (paperlayer.ai, arXiv 2505.13389), section 2 "Methods"
// (coarse stage mean-pools each cube) and Appendix B (block-mean of q, k, v);
// VSA reading notes, key design 1 (Q_c, K_c, V_c: 64x shorter sequence).
//
// One workgroup per (b, h, cube). Each thread owns one 8-channel chunk of a
// set of token rows, sums them in fp32 (or keeps their maximum and its first
// position), and the partial results are reduced through LDS. The max-pool
// variant is the pooling the VSA summary page's ablation study compares
// (section 3, Experiments). HBM-bound: every input element is read once and
// the pooled values (fp32) are written once.
#include "vsa_kernels.h"

namespace vsa {

template <typename T, int D, bool MAX, int BT>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, float* __restrict__ qc,
                                                   float* __restrict__ kc, float* __restrict__ vc,
                                                   uint8_t* __restrict__ args, Grid g) {
  constexpr int CH = D / 8;            // 8-channel chunks per token row
  constexpr int RPP = 256 / CH;        // token rows per pass
  constexpr int PASSES = BT / RPP;     // BT = tokens per cube
  __shared__ float part[3][RPP][D + 4];
  __shared__ uint8_t parg[MAX ? 3 : 1][MAX ? RPP : 1][D + 4];

  const int tid = threadIdx.x;
  const long bh = blockIdx.y;
  const int c = blockIdx.x;
  const int ch = tid % CH, rsub = tid / CH;
  const long base = bh * (long)g.N * D;
  const long plane = (long)gridDim.y * g.Nc * D;   // one tensor's args

  const T* srcs[3] = {q + base, k + base, v + base};
  float* dsts[3] = {qc, kc, vc};
  // Every load of the three tensors is issued before any reduction, so a
  // thread keeps 3 * PASSES independent 16-byte loads in flight.
  float acc[3][8];
  int am[3][8];
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int e = 0; e < 8; ++e) { acc[w][e] = MAX ? -INFINITY : 0.f; am[w][e] = 0; }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int l = p * RPP + rsub;   // increasing: a strict compare keeps the first maximum
    const long off = (long)cube_token(g, c, l) * D + ch * 8;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      float x[8];
      load8(srcs[w] + off, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (MAX) {
          if (x[e] > acc[w][e]) { acc[w][e] = x[e]; am[w][e] = l; }
        } else {
          acc[w][e] += x[e];
        }
      }
    }
  }
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      part[w][rsub][ch * 8 + e] = acc[w][e];
      if (MAX) parg[w][rsub][ch * 8 + e] = (uint8_t)am[w][e];
    }
  __syncthreads();
  for (int t = tid; t < 3 * D; t += 256) {
    const int w = t / D, col = t - w * D;
    if (MAX) {
      float best = part[w][0][col];
      int ba = parg[w][0][col];
#pragma unroll
      for (int r = 1; r < RPP; ++r) {
        const float y = part[w][r][col];
        const int a = parg[w][r][col];
        if (y > best || (y == best && a < ba)) { best = y; ba = a; }   // ties: first in cube order
      }
      if (dsts[w] != nullptr) dsts[w][(bh * g.Nc + c) * D + col] = best;
      if (args != nullptr) args[w * plane + (bh * g.Nc + c) * D + col] = (uint8_t)ba;
    } else {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < RPP; ++r) s += part[w][r][col];
      if (dsts[w] != nullptr) dsts[w][(bh * g.Nc + c) * D + col] = s * (1.0f / BT);
    }
  }
}

template <typename T, bool MAX, int BT>
static void pool_launch_bt(const Launch& L, const void* q, const void* k, const void* v, float* qc, float* kc,
                           float* vc, uint8_t* args) {
  const dim3 grid(L.g.Nc, L.BH), block(256);
  if (L.D == 64)
    hipLaunchKernelGGL((pool_kernel<T, 64, MAX, BT>), grid, block, 0, L.stream, (const T*)q, (const T*)k,
                       (const T*)v, qc, kc, vc, args, L.g);
  else
    hipLaunchKernelGGL((pool_kernel<T, 128, MAX, BT>), grid, block, 0, L.stream, (const T*)q, (const T*)k,
                       (const T*)v, qc, kc, vc, args, L.g);
}

template <typename T, bool MAX>
static void pool_launch(const Launch& L, const void* q, const void* k, const void* v, float* qc, float* kc,
                        float* vc, uint8_t* args) {
  if (L.g.B == 32) pool_launch_bt<T, MAX, 32>(L, q, k, v, qc, kc, vc, args);
  else if (L.g.B == 128) pool_launch_bt<T, MAX, 128>(L, q, k, v, qc, kc, vc, args);
  else pool_launch_bt<T, MAX, 64>(L, q, k, v, qc, kc, vc, args);
}

hipError_t launch_pool(const Launch& L, const void* q, const void* k, const void* v, float* qc, float* kc,
                       float* vc, uint8_t* args) {
  if (L.bf16) {
    if (L.pool_max) pool_launch<bf16, true>(L, q, k, v, qc, kc, vc, args);
    else pool_launch<bf16, false>(L, q, k, v, qc, kc, vc, nullptr);
  } else {
    if (L.pool_max) pool_launch<float, true>(L, q, k, v, qc, kc, vc, args);
    else pool_launch<float, false>(L, q, k, v, qc, kc, vc, nullptr);
  }
  return hipGetLastError();
}

}  // namespace vsa
