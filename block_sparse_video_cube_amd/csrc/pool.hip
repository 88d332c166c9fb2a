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

// SEL: bit w set = tensor w (q, k, v) is pooled by this launch (all three
// when queries and keys share the cube shape, else q alone or k and v).
template <typename T, int D, bool MAX, int BT, int SEL>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, float* __restrict__ qc,
                                                   float* __restrict__ kc, float* __restrict__ vc,
                                                   uint8_t* __restrict__ qa, uint8_t* __restrict__ ka,
                                                   uint8_t* __restrict__ va, Grid g) {
  constexpr int CH = D / 8;                      // 8-channel chunks per token row
  constexpr int RPP = 256 / CH < BT ? 256 / CH : BT;   // token rows per pass (BT = tokens per cube)
  constexpr int PASSES = BT / RPP;
  __shared__ float part[3][RPP][D + 4];
  __shared__ uint8_t parg[MAX ? 3 : 1][MAX ? RPP : 1][D + 4];

  const int tid = threadIdx.x;
  const long bh = blockIdx.y;
  const int c = blockIdx.x;
  const int ch = tid % CH, rsub = tid / CH;
  const long base = bh * (long)g.N * D;
  const bool active = rsub < RPP;   // small cubes leave threads without a row

  const T* srcs[3] = {q, k, v};
  float* dsts[3] = {qc, kc, vc};
  uint8_t* args[3] = {qa, ka, va};
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
    if (!active) break;
    const int l = p * RPP + rsub;   // increasing: a strict compare keeps the first maximum
    const long off = base + (long)cube_token(g, c, l) * D + ch * 8;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      if (!(SEL & (1 << w))) continue;
      float x[8];
      load8_nt(srcs[w] + off, x);
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
  if (active) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        part[w][rsub][ch * 8 + e] = acc[w][e];
        if (MAX) parg[w][rsub][ch * 8 + e] = (uint8_t)am[w][e];
      }
  }
  __syncthreads();
  for (int t = tid; t < 3 * D; t += 256) {
    const int w = t / D, col = t - w * D;
    if (!(SEL & (1 << w))) continue;
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
      if (args[w] != nullptr) args[w][(bh * g.Nc + c) * D + col] = (uint8_t)ba;
    } else {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < RPP; ++r) s += part[w][r][col];
      if (dsts[w] != nullptr) dsts[w][(bh * g.Nc + c) * D + col] = s * (1.0f / BT);
    }
  }
}

template <typename T, bool MAX, int BT, int SEL>
static void pool_launch_bt(const Launch& L, const Grid& g, const void* q, const void* k, const void* v, float* qc,
                           float* kc, float* vc, uint8_t* qa, uint8_t* ka, uint8_t* va) {
  const dim3 grid(g.Nc, L.BH), block(256);
  if (L.D == 64)
    hipLaunchKernelGGL((pool_kernel<T, 64, MAX, BT, SEL>), grid, block, 0, L.stream, (const T*)q, (const T*)k,
                       (const T*)v, qc, kc, vc, qa, ka, va, g);
  else
    hipLaunchKernelGGL((pool_kernel<T, 128, MAX, BT, SEL>), grid, block, 0, L.stream, (const T*)q, (const T*)k,
                       (const T*)v, qc, kc, vc, qa, ka, va, g);
}

template <typename T, bool MAX, int SEL>
static void pool_grid(const Launch& L, const Grid& g, const void* q, const void* k, const void* v, float* qc,
                      float* kc, float* vc, uint8_t* qa, uint8_t* ka, uint8_t* va) {
  if (g.B == 16) pool_launch_bt<T, MAX, 16, SEL>(L, g, q, k, v, qc, kc, vc, qa, ka, va);
  else if (g.B == 32) pool_launch_bt<T, MAX, 32, SEL>(L, g, q, k, v, qc, kc, vc, qa, ka, va);
  else if (g.B == 128) pool_launch_bt<T, MAX, 128, SEL>(L, g, q, k, v, qc, kc, vc, qa, ka, va);
  else if (g.B == 256) pool_launch_bt<T, MAX, 256, SEL>(L, g, q, k, v, qc, kc, vc, qa, ka, va);
  else pool_launch_bt<T, MAX, 64, SEL>(L, g, q, k, v, qc, kc, vc, qa, ka, va);
}

// Queries pool over query cubes, keys and values over key blocks: one launch
// when the two shapes agree, two otherwise.
template <typename T, bool MAX>
static void pool_launch(const Launch& L, const void* q, const void* k, const void* v, float* qc, float* kc,
                        float* vc, uint8_t* args) {
  uint8_t* qa = args;
  uint8_t* ka = args != nullptr ? args + (size_t)L.BH * L.g.Nc * L.D : nullptr;
  uint8_t* va = args != nullptr ? ka + (size_t)L.BH * L.gk.Nc * L.D : nullptr;
  const bool same = L.g.B == L.gk.B && L.g.lct == L.gk.lct && L.g.lch == L.gk.lch;
  if (same) {
    pool_grid<T, MAX, 7>(L, L.g, q, k, v, qc, kc, vc, qa, ka, va);
  } else {
    pool_grid<T, MAX, 1>(L, L.g, q, nullptr, nullptr, qc, nullptr, nullptr, qa, nullptr, nullptr);
    pool_grid<T, MAX, 6>(L, L.gk, nullptr, k, v, nullptr, kc, vc, nullptr, ka, va);
  }
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
