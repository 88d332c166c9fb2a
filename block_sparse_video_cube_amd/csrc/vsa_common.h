// Shared device-side definitions of the VSA HIP kernels (gfx950 / CDNA4).
//
// Layout facts used by every kernel:
//  * Token tensors are [B, heads, T, H, W, D] (raster order) or, with the
//    tiled layout, [B, heads, Nc, 64, D] (cube-major); D fastest. Kernels
//    address tokens only through cube_token / cube_row / token_cube /
//    chunk_row, which know the order.
//  * Cube c of a (T, H, W) latent has origin (4*tc, 4*yc, 4*xc) with
//    c = (tc * H4 + yc) * W4 + xc (row-major cube order); token l of a cube
//    (0..63) is (t', y', x') = (l / 16, (l / 4) % 4, l % 4). Within a cube the
//    four tokens x' = 0..3 are contiguous in raster memory (4*D elements).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;   // tokens per (4,4,4) cube
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Grid {
  int T, H, W;       // latent
  int H4, W4;        // cube grid (T4 implied)
  int N, Nc;         // tokens, cubes
  int tiled;         // token order: 0 = raster (t, y, x); 1 = cube-major (token l of cube c at 64c + l)
};

__host__ __device__ inline Grid make_grid(int T, int H, int W, int tiled = 0) {
  Grid g;
  g.T = T; g.H = H; g.W = W;
  g.H4 = H / 4; g.W4 = W / 4;
  g.N = T * H * W; g.Nc = g.N / kTile;
  g.tiled = tiled;
  return g;
}

// Index (row) of token l (0..63) of cube c in the problem's token order.
__device__ __forceinline__ int cube_token(const Grid& g, int c, int l) {
  if (g.tiled) return c * kTile + l;
  const int xc = c % g.W4;
  const int r = c / g.W4;
  const int yc = r % g.H4;
  const int tc = r / g.H4;
  const int t = 4 * tc + (l >> 4), y = 4 * yc + ((l >> 2) & 3), x = 4 * xc + (l & 3);
  return (t * g.H + y) * g.W + x;
}

// Index of the first token of row (t', y') of cube c; the row's four tokens
// x' = 0..3 follow contiguously in either token order.
__device__ __forceinline__ int cube_row(const Grid& g, int c, int tl, int yl) {
  if (g.tiled) return c * kTile + 16 * tl + 4 * yl;
  const int xc = c % g.W4;
  const int r = c / g.W4;
  const int yc = r % g.H4;
  const int tc = r / g.H4;
  return ((4 * tc + tl) * g.H + 4 * yc + yl) * g.W + 4 * xc;
}

// Cube of the token at index n.
__device__ __forceinline__ int token_cube(const Grid& g, int n) {
  if (g.tiled) return n / kTile;
  const int x = n % g.W;
  const int r = n / g.W;
  const int y = r % g.H;
  const int t = r / g.H;
  return ((t >> 2) * g.H4 + (y >> 2)) * g.W4 + (x >> 2);
}

// Rows between token (t', y', x') of a chunk (half h: t' = 2h, 2h + 1) and
// its first token (2h, 0, 0): kappa = 16(t' - 2h) + 4y' + x' is the token's
// position in the chunk. And rows between the first tokens of the two halves.
__host__ __device__ __forceinline__ int chunk_row(const Grid& g, int kappa) {
  if (g.tiled) return kappa;
  return ((kappa >> 4) * g.H + ((kappa >> 2) & 3)) * g.W + (kappa & 3);
}
__host__ __device__ __forceinline__ int half_rows(const Grid& g) { return g.tiled ? 32 : 2 * g.H * g.W; }

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Map block b so that every XCD gets one contiguous range of work items:
// neighbouring items (same head, neighbouring cubes) then share an L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int q = nblocks >> 3, rem = nblocks & 7;
  const int x = b & 7, k = b >> 3;
  return x * q + (x < rem ? x : rem) + k;
}

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }
__device__ __forceinline__ bf16 f2bf(float v) { return (bf16)v; }  // round to nearest even

template <typename T> struct Io;
template <> struct Io<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <> struct Io<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p) { return (float)*p; }
  static __device__ __forceinline__ void st(bf16* p, float v) { *p = (bf16)v; }
};

// Value after a store/load round trip through T (bf16: round to nearest even).
template <typename T> __device__ __forceinline__ float round_to(float v);
template <> __device__ __forceinline__ float round_to<float>(float v) { return v; }
template <> __device__ __forceinline__ float round_to<bf16>(float v) { return (float)(bf16)v; }

// 8 consecutive elements as fp32 (16-byte load for bf16, two for fp32).
__device__ __forceinline__ void load8(const bf16* p, float* o) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
  *reinterpret_cast<bf16x8*>(p) = r;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ unsigned wave_min_u32(unsigned v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (unsigned)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ f32x4 mfma16_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace vsa
