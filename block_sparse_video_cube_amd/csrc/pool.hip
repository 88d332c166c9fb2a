// Step 1 of VSA: cube mean-pool, and the transposed V tiles of the fine stage.
//
// VSA summary page (paperlayer.ai, arXiv 2505.13389), section 2 "Methods"
// (coarse stage mean-pools each cube) and Appendix B (block-mean of q, k, v);
// VSA reading notes, key design 1 (Q_c, K_c, V_c: 64x shorter sequence).
//
// One workgroup per (b, h, cube). Each thread owns one 8-channel chunk of a
// set of token rows, sums them in fp32, and the partial sums are reduced
// through LDS. HBM-bound: every input element is read once; pooled means
// (fp32) and optionally the bf16 V chunk tiles of the fine forward kernel
// (layout in vsa_common.h) are written once.
#include "vsa_kernels.h"

namespace vsa {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, float* __restrict__ qc,
                                                   float* __restrict__ kc, float* __restrict__ vc,
                                                   bf16* __restrict__ vt, Grid g) {
  constexpr int CH = D / 8;            // 8-channel chunks per token row
  constexpr int RPP = 256 / CH;        // token rows per pass
  constexpr int PASSES = kTile / RPP;
  constexpr int VPITCH = D + 8;        // LDS row pitch of the staged V tile (bf16)
  __shared__ float part[RPP][D + 4];
  __shared__ bf16 vtile[kTile][VPITCH];

  const int tid = threadIdx.x;
  const long bh = blockIdx.y;
  const int c = blockIdx.x;
  const int ch = tid % CH, rsub = tid / CH;
  const long base = bh * (long)g.N * D;

  const T* srcs[3] = {q, k, v};
  float* dsts[3] = {qc, kc, vc};
#pragma unroll
  for (int which = 0; which < 3; ++which) {
    const T* src = srcs[which] + base;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int l = p * RPP + rsub;
      float x[8];
      load8(src + (long)cube_token(g, c, l) * D + ch * 8, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[e];
      if (which == 2 && vt != nullptr) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vtile[l][ch * 8 + e] = (bf16)x[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rsub][ch * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < RPP; ++r) s += part[r][tid];
      dsts[which][(bh * g.Nc + c) * D + tid] = s * (1.0f / kTile);
    }
    __syncthreads();
  }

  if (vt != nullptr) store_chunk_tiles<D, VPITCH>(vtile, vt + (bh * g.Nc + c) * (long)D * kTile, tid, 256);
}

// Chunk tiles of a raster bf16 tensor (the backward's Q and K).
template <int D>
__global__ __launch_bounds__(256) void ctile_kernel(const bf16* __restrict__ x, bf16* __restrict__ xt, Grid g) {
  constexpr int CH = D / 8, RPP = 256 / CH, PASSES = kTile / RPP, VPITCH = D + 8;
  __shared__ bf16 tile[kTile][VPITCH];
  const int tid = threadIdx.x;
  const long bh = blockIdx.y;
  const int c = blockIdx.x;
  const int ch = tid % CH, rsub = tid / CH;
  const bf16* src = x + bh * (long)g.N * D;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int l = p * RPP + rsub;
    *reinterpret_cast<bf16x8*>(&tile[l][ch * 8]) =
        *reinterpret_cast<const bf16x8*>(src + (long)cube_token(g, c, l) * D + ch * 8);
  }
  __syncthreads();
  store_chunk_tiles<D, VPITCH>(tile, xt + (bh * g.Nc + c) * (long)D * kTile, tid, 256);
}

hipError_t launch_pool(const Launch& L, const void* q, const void* k, const void* v, float* qc, float* kc,
                       float* vc, bf16* vt) {
  const dim3 grid(L.g.Nc, L.BH), block(256);
  if (L.bf16) {
    if (L.D == 64)
      hipLaunchKernelGGL((pool_kernel<bf16, 64>), grid, block, 0, L.stream, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, qc, kc, vc, vt, L.g);
    else
      hipLaunchKernelGGL((pool_kernel<bf16, 128>), grid, block, 0, L.stream, (const bf16*)q, (const bf16*)k,
                         (const bf16*)v, qc, kc, vc, vt, L.g);
  } else {
    if (L.D == 64)
      hipLaunchKernelGGL((pool_kernel<float, 64>), grid, block, 0, L.stream, (const float*)q, (const float*)k,
                         (const float*)v, qc, kc, vc, (bf16*)nullptr, L.g);
    else
      hipLaunchKernelGGL((pool_kernel<float, 128>), grid, block, 0, L.stream, (const float*)q,
                         (const float*)k, (const float*)v, qc, kc, vc, (bf16*)nullptr, L.g);
  }
  return hipGetLastError();
}

hipError_t launch_ctile(const Launch& L, const bf16* x, bf16* xt) {
  const dim3 grid(L.g.Nc, L.BH), block(256);
  if (L.D == 64)
    hipLaunchKernelGGL((ctile_kernel<64>), grid, block, 0, L.stream, x, xt, L.g);
  else
    hipLaunchKernelGGL((ctile_kernel<128>), grid, block, 0, L.stream, x, xt, L.g);
  return hipGetLastError();
}

}  // namespace vsa
