// Shared device-side definitions of the VSA HIP kernels (gfx950 / CDNA4).
//
// Layout facts used by every kernel:
//  * Token tensors are [B, heads, T, H, W, D] (raster order) or, with the
//    tiled layout, [B, heads, Nc, Bt, D] (cube-major, Bt tokens per cube);
//    D fastest. Kernels address tokens only through cube_first / cube_rel /
//    cube_token / token_cube / chunk_row, which know the order.
//  * Cubes are (Ct, Ch, Cw) blocks of Bt = Ct*Ch*Cw tokens (every side a
//    power of two; (4, 4, 4) and 64 tokens by default). Cube c of a (T, H, W)
//    latent has origin (Ct*tc, Ch*yc, Cw*xc) with c = (tc * Hn + yc) * Wn + xc
//    (row-major cube order); token l of a cube is (t', y', x') =
//    (l / (Ch*Cw), (l / Cw) % Ch, l % Cw). Within a cube the Cw tokens of a
//    row are contiguous in raster memory.
//  * A chunk is 32 consecutive tokens of a cube (l = 32h .. 32h + 31); the
//    offset of its token kappa from its first token does not depend on h or
//    on the cube, because 32 and Ch*Cw are powers of two (one divides the
//    other) and Cw divides 32 or 32 divides Cw.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Grid {
  int T, H, W;       // latent
  int lct, lch, lcw; // log2 of the cube sides (Ct, Ch, Cw)
  int B;             // tokens per cube, Ct * Ch * Cw
  int Hn, Wn;        // cubes along H and along W (T / Ct along T)
  int N, Nc;         // tokens, cubes
  int tiled;         // token order: 0 = raster (t, y, x); 1 = cube-major (token l of cube c at B*c + l)
};

__host__ __device__ inline int ilog2(int v) {
  int r = 0;
  while ((1 << (r + 1)) <= v) ++r;
  return r;
}

// Cube sides must be powers of two dividing T, H, W (checked on the host).
__host__ __device__ inline Grid make_grid(int T, int H, int W, int tiled = 0, int ct = 4, int ch = 4, int cw = 4) {
  Grid g;
  g.T = T; g.H = H; g.W = W;
  g.lct = ilog2(ct); g.lch = ilog2(ch); g.lcw = ilog2(cw);
  g.B = ct * ch * cw;
  g.Hn = H / ch; g.Wn = W / cw;
  g.N = T * H * W; g.Nc = g.N / g.B;
  g.tiled = tiled;
  return g;
}

// Halves of a 256-token cube or key block: the cube split in two along its
// first side longer than 1 (t, else y, else x). Tokens keep their order: in
// row-major (t', y', x') order the first 128 tokens of the cube are exactly
// its first half, in the half's own row-major order. In the raster layout the
// halves form the grid of the halved shape (row-major); in the tiled layout
// half hh of cube c is entry 2c + hh (tokens 256c + 128hh + l). The fine
// kernels handle 256-token tiles as these 128-token halves.
__host__ __device__ inline Grid half_grid(const Grid& g) {
  int ct = 1 << g.lct, ch = 1 << g.lch, cw = 1 << g.lcw;
  if (ct > 1) ct >>= 1;
  else if (ch > 1) ch >>= 1;
  else cw >>= 1;
  return make_grid(g.T, g.H, g.W, g.tiled, ct, ch, cw);
}
// Index in h2 = half_grid(g) of half hh of cube c of g.
__host__ __device__ inline int half_index(const Grid& g, const Grid& h2, int c, int hh) {
  if (g.tiled) return 2 * c + hh;
  const int xc = c % g.Wn, r = c / g.Wn, yc = r % g.Hn, tc = r / g.Hn;
  if (g.lct > 0) return ((2 * tc + hh) * h2.Hn + yc) * h2.Wn + xc;
  if (g.lch > 0) return (tc * h2.Hn + 2 * yc + hh) * h2.Wn + xc;
  return (tc * h2.Hn + yc) * h2.Wn + 2 * xc + hh;
}
// The cube c of g and half hh of entry s of h2 = half_grid(g).
__host__ __device__ inline void half_parent(const Grid& g, const Grid& h2, int s, int& c, int& hh) {
  if (g.tiled) { c = s >> 1; hh = s & 1; return; }
  const int xs = s % h2.Wn, r = s / h2.Wn, ys = r % h2.Hn, ts = r / h2.Hn;
  if (g.lct > 0) { hh = ts & 1; c = ((ts >> 1) * g.Hn + ys) * g.Wn + xs; }
  else if (g.lch > 0) { hh = ys & 1; c = (ts * g.Hn + (ys >> 1)) * g.Wn + xs; }
  else { hh = xs & 1; c = (ts * g.Hn + ys) * g.Wn + (xs >> 1); }
}

// Index (row) of token 0 of cube c in the problem's token order.
__host__ __device__ __forceinline__ int cube_first(const Grid& g, int c) {
  if (g.tiled) return c * g.B;
  const int xc = c % g.Wn;
  const int r = c / g.Wn;
  const int yc = r % g.Hn;
  const int tc = r / g.Hn;
  return ((tc << g.lct) * g.H + (yc << g.lch)) * g.W + (xc << g.lcw);
}

// Rows between in-cube token l and token 0 of the same cube (any cube).
__host__ __device__ __forceinline__ int cube_rel(const Grid& g, int l) {
  if (g.tiled) return l;
  const int t = l >> (g.lch + g.lcw), y = (l >> g.lcw) & ((1 << g.lch) - 1), x = l & ((1 << g.lcw) - 1);
  return (t * g.H + y) * g.W + x;
}

// Index of token l of cube c in the problem's token order.
__host__ __device__ __forceinline__ int cube_token(const Grid& g, int c, int l) { return cube_first(g, c) + cube_rel(g, l); }

// Cube of the token at index n.
__device__ __forceinline__ int token_cube(const Grid& g, int n) {
  if (g.tiled) return n / g.B;
  const int x = n % g.W;
  const int r = n / g.W;
  const int y = r % g.H;
  const int t = r / g.H;
  return ((t >> g.lct) * g.Hn + (y >> g.lch)) * g.Wn + (x >> g.lcw);
}

// Rows between token kappa (0..31) of a chunk and the chunk's first token:
// the same for every chunk of every cube (see the layout facts above).
__host__ __device__ __forceinline__ int chunk_row(const Grid& g, int kappa) { return cube_rel(g, kappa); }
// Rows between the first token of chunk h of a cube and the cube's first token.
__host__ __device__ __forceinline__ int chunk_first(const Grid& g, int h) { return cube_rel(g, 32 * h); }
// log2 of the 32-token chunks per cube (Bt in {32, 64, 128}).
__host__ __device__ __forceinline__ int chunk_shift(const Grid& g) { return g.lct + g.lch + g.lcw - 5; }

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Map block b so that every XCD gets one contiguous range of work items:
// neighbouring items (same head, neighbouring cubes) then share an L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int q = nblocks >> 3, rem = nblocks & 7;
  const int x = b & 7, k = b >> 3;
  return x * q + (x < rem ? x : rem) + k;
}
// Tile (x, y) of head z of a 1-D grid over nx * ny tiles per head (x
// fastest), through xcd_remap: each XCD takes whole heads, whose operands
// then stay in its L2 instead of being fetched by every XCD.
struct Tile3 {
  int x, y;
  long z;
};
__device__ __forceinline__ Tile3 tile3(int nx, int ny) {
  const int s = xcd_remap(blockIdx.x, gridDim.x);
  const int r = s / nx;
  return Tile3{s - r * nx, r % ny, r / ny};
}


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
// The same with the non-temporal hint, for data touched once per launch
// (streaming stages, epilogues): such lines are not kept in the caches, so
// the streams neither evict reused operands nor pay for cache allocation; a
// streaming read measured 7.06 TB/s with the hint against 6.31 TB/s without.
__device__ __forceinline__ void load8_nt(const bf16* p, float* o) {
  const bf16x8 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
}
__device__ __forceinline__ void load8_nt(const float* p, float* o) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
  for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[4 + e] = b[e]; }
}
__device__ __forceinline__ void store8_nt(bf16* p, const float* v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
  __builtin_nontemporal_store(r, reinterpret_cast<bf16x8*>(p));
}
__device__ __forceinline__ void store8_nt(float* p, const float* v) {
  const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p + 4));
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
