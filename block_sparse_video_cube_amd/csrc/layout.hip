// Token-order conversion and latent cropping: copies of token tensors, no
// arithmetic.
//
// VSA summary page (paperlayer.ai, arXiv 2505.13389), Appendix B: the video
// is tiled into cube-major order before the attention layer and untiled after
// it. Same page, section 5 "Limitation and Conclusion": (4, 4, 4) cubes need
// latent sides that are multiples of 4, and the remedy named there is to
// generate a slightly larger latent and crop it. vsa_crop / vsa_pad move a tensor between the requested
// latent (raster order) and the compatible one (either token order).
//
// All kernels move 16-byte units (a token row is 128 to 512 bytes), so every
// access is a full 16-byte vector load or store and neighbouring lanes touch
// neighbouring units of one row: HBM-bound, each byte read once, written once.
#include <algorithm>

#include "vsa_kernels.h"

namespace vsa {

// One workgroup per (b, h, cube): the cube's Bt token rows move between
// raster and cube-major order.
template <typename T>
__global__ __launch_bounds__(256) void relayout_kernel(const T* __restrict__ src, T* __restrict__ dst, Grid g,
                                                       int D, int to_tiled) {
  const long bh = blockIdx.y;
  const int c = blockIdx.x;
  Grid r = g;
  r.tiled = 0;
  const int units = D * (int)sizeof(T) / 16;   // 16-byte units per token row
  for (int w = threadIdx.x; w < g.B * units; w += 256) {
    const int l = w / units, u = w - l * units;
    const long ras = bh * g.N + cube_token(r, c, l);
    const long til = bh * g.N + (long)c * g.B + l;
    const long from = to_tiled ? ras : til, to = to_tiled ? til : ras;
    reinterpret_cast<uint4*>(dst + to * D)[u] = reinterpret_cast<const uint4*>(src + from * D)[u];
  }
}

hipError_t launch_relayout(const Launch& L, const void* src, void* dst, bool to_tiled) {
  const dim3 grid(L.g.Nc, L.BH), block(256);
  if (L.bf16)
    hipLaunchKernelGGL((relayout_kernel<bf16>), grid, block, 0, L.stream, (const bf16*)src, (bf16*)dst, L.g, L.D,
                       (int)to_tiled);
  else
    hipLaunchKernelGGL((relayout_kernel<float>), grid, block, 0, L.stream, (const float*)src, (float*)dst, L.g,
                       L.D, (int)to_tiled);
  return hipGetLastError();
}

// ---- 256-token tiles as two 128-token halves (see half_grid) ------------
// Lists of the query halves: half s of query cube c gets c's list, every
// listed key block replaced by its two halves when key blocks are split (the
// lists of the halves are not ascending; no fine kernel needs them to be).
__global__ __launch_bounds__(256) void split_lists_kernel(const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ len, int32_t* __restrict__ idx2,
                                                          int32_t* __restrict__ len2, Grid gq, Grid gq2, Grid gk,
                                                          Grid gk2, int qsplit, int ksplit, int stride, int stride2) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  const long bh = blockIdx.y;
  if (s >= gq2.Nc) return;
  int c = s, hh = 0;
  if (qsplit) half_parent(gq, gq2, s, c, hh);
  const long row = bh * gq.Nc + c, row2 = bh * gq2.Nc + s;
  const int L = min(max(len[row], 0), stride);
  for (int t = 0; t < L; ++t) {
    int j = idx[row * stride + t];
    j = (j >= 0 && j < gk.Nc) ? j : 0;   // malformed entries stay in range
    if (ksplit) {
      idx2[row2 * stride2 + 2 * t] = half_index(gk, gk2, j, 0);
      idx2[row2 * stride2 + 2 * t + 1] = half_index(gk, gk2, j, 1);
    } else {
      idx2[row2 * stride2 + t] = j;
    }
  }
  len2[row2] = ksplit ? 2 * L : L;
}

// Per-half copies of per-cube fp32 rows of D values (O_c for the fused
// combine, pooled gradients) scaled by mul, and of max-pool argmax positions
// (the position within the half, or 255 = none when the maximum lies in the
// other half). One workgroup per (b, h, half).
__global__ __launch_bounds__(128) void split_rows_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                         const uint8_t* __restrict__ asrc, uint8_t* __restrict__ adst,
                                                         Grid g, Grid g2, int D, float mul) {
  const int s = blockIdx.x;
  const long bh = blockIdx.y;
  int c, hh;
  half_parent(g, g2, s, c, hh);
  const long from = (bh * g.Nc + c) * D, to = (bh * g2.Nc + s) * D;
  for (int ch = threadIdx.x; ch < D; ch += 128) {
    if (src != nullptr) dst[to + ch] = src[from + ch] * mul;
    if (asrc != nullptr) {
      const int a = asrc[from + ch] - 128 * hh;
      adst[to + ch] = (a >= 0 && a < 128) ? (uint8_t)a : (uint8_t)255;
    }
  }
}

hipError_t launch_split_lists(const Launch& L, const Launch& S, const int32_t* idx, const int32_t* len, int32_t* idx2,
                              int32_t* len2) {
  const dim3 grid((S.g.Nc + 255) / 256, L.BH);
  hipLaunchKernelGGL(split_lists_kernel, grid, dim3(256), 0, L.stream, idx, len, idx2, len2, L.g, S.g, L.gk, S.gk,
                     (int)(L.g.B != S.g.B), (int)(L.gk.B != S.gk.B), L.stride, S.stride);
  return hipGetLastError();
}

hipError_t launch_split_rows(const Launch& L, const Grid& g, const Grid& g2, const float* src, float* dst,
                             const uint8_t* asrc, uint8_t* adst, float mul) {
  hipLaunchKernelGGL(split_rows_kernel, dim3(g2.Nc, L.BH), dim3(128), 0, L.stream, src, dst, asrc, adst, g, g2, L.D,
                     mul);
  return hipGetLastError();
}

// Index, in the problem's token order, of raster token (t, y, x).
__device__ __forceinline__ long token_index(const Grid& g, int t, int y, int x) {
  if (!g.tiled) return ((long)t * g.H + y) * g.W + x;
  const int c = ((t >> g.lct) * g.Hn + (y >> g.lch)) * g.Wn + (x >> g.lcw);
  const int ct = t & ((1 << g.lct) - 1), cy = y & ((1 << g.lch) - 1), cx = x & ((1 << g.lcw) - 1);
  return (long)c * g.B + (((ct << g.lch) | cy) << g.lcw | cx);
}

// Crop (to_small = 1): small[b, h, t, y, x] = big[b, h, token (t, y, x)] for
// the small raster grid ts x hs x ws. Pad (to_small = 0): big[b, h, token
// (t, y, x)] = small[b, h, t, y, x] inside that region, 0 elsewhere. The
// grid-stride loop runs over the 16-byte units of the small tensor (crop) or
// the big one (pad); consecutive lanes take consecutive units.
__global__ __launch_bounds__(256) void crop_pad_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                       Grid g, int ts, int hs, int ws, int units, long bh_count,
                                                       int to_small) {
  const long small_n = (long)ts * hs * ws;
  const long rows = bh_count * (to_small ? small_n : (long)g.N);
  const long total = rows * units;
  for (long w = (long)blockIdx.x * 256 + threadIdx.x; w < total; w += (long)gridDim.x * 256) {
    const long row = w / units;
    const int u = (int)(w - row * units);
    if (to_small) {
      const long bh = row / small_n, n = row - bh * small_n;
      const int x = (int)(n % ws), r = (int)(n / ws), y = r % hs, t = r / hs;
      dst[w] = src[(bh * g.N + token_index(g, t, y, x)) * units + u];
    } else {
      const long bh = row / g.N;
      const int n = (int)(row - bh * g.N);
      int t, y, x;
      if (g.tiled) {
        const int c = n / g.B, l = n % g.B;
        x = ((c % g.Wn) << g.lcw) + (l & ((1 << g.lcw) - 1));
        y = (((c / g.Wn) % g.Hn) << g.lch) + ((l >> g.lcw) & ((1 << g.lch) - 1));
        t = ((c / (g.Wn * g.Hn)) << g.lct) + (l >> (g.lch + g.lcw));
      } else {
        x = n % g.W;
        y = (n / g.W) % g.H;
        t = n / (g.W * g.H);
      }
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (t < ts && y < hs && x < ws) val = src[((bh * ts + t) * hs + y) * (long)ws * units + (long)x * units + u];
      dst[w] = val;
    }
  }
}

hipError_t launch_crop_pad(const Launch& L, const void* src, void* dst, int ts, int hs, int ws, bool to_small) {
  const int units = L.D * (L.bf16 ? 2 : 4) / 16;
  const long rows = (long)L.BH * (to_small ? (long)ts * hs * ws : (long)L.g.N);
  const long blocks = std::min<long>((rows * units + 255) / 256, 8L * 1024);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(crop_pad_kernel, dim3((unsigned)blocks), dim3(256), 0, L.stream, (const uint4*)src,
                     (uint4*)dst, L.g, ts, hs, ws, units, (long)L.BH, (int)to_small);
  return hipGetLastError();
}

}  // namespace vsa
