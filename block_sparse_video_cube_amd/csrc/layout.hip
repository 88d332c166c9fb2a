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
