// Step 5 of VSA (gated combine + untile) and its backward.
//
// VSA reading notes, key design 3 (O = O_c * G_c + O_f * G_f with gates from
// the hidden states); VSA summary page (paperlayer.ai, arXiv 2505.13389),
// Appendix B (coarse output repeated over each block, combination, untile).
// The backward is the calculus of that elementwise sum; the repeat's gradient
// sums over the cube's tokens.
#include "vsa_kernels.h"

namespace vsa {

// o[token] = O_c[cube(token)] * g_c + o_f * g_f; one thread per 8 channels.
template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ oc, const T* __restrict__ of,
                                                      const T* __restrict__ gc, const T* __restrict__ gf,
                                                      T* __restrict__ o, Grid g, long nchunks) {
  constexpr int CH = D / 8;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= nchunks) return;
  const long tok = e / CH;
  const int ch = (int)(e - tok * CH) * 8;
  const long bh = tok / g.N;
  const int n = (int)(tok - bh * g.N);
  const int c = token_cube(g, n);
  float a[8], b[8], x[8], cv[8], r[8];
  load8(of + tok * D + ch, x);
  load8(oc + (bh * g.Nc + c) * D + ch, cv);
  if (gc != nullptr) load8(gc + tok * D + ch, a);
  else for (int i = 0; i < 8; ++i) a[i] = 1.f;
  if (gf != nullptr) load8(gf + tok * D + ch, b);
  else for (int i = 0; i < 8; ++i) b[i] = 1.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = cv[i] * a[i] + x[i] * b[i];
  store8(o + tok * D + ch, r);
}

// Backward of the combine, one workgroup per (b, h, cube):
//   dg_c = dO * O_c[c], dg_f = dO * O_f, d_o_f = dO * G_f (rounded to T),
//   delta[token] = sum_ch d_o_f * O_f, d_o_c[c] = sum over the cube of dO * G_c,
template <typename T, int D, int BT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const T* __restrict__ d_o, const float* __restrict__ oc, const T* __restrict__ of, const T* __restrict__ gc,
    const T* __restrict__ gf, T* __restrict__ dgc, T* __restrict__ dgf, T* __restrict__ dof,
    float* __restrict__ delta, float* __restrict__ doc, Grid g) {
  constexpr int CH = D / 8, RPP = 256 / CH, PASSES = BT / RPP;   // BT = tokens per cube
  __shared__ float part[RPP][D + 4];
  const int tid = threadIdx.x;
  const long bh = blockIdx.y;
  const int c = blockIdx.x;
  const int ch = tid % CH, rsub = tid / CH;
  const long base = bh * (long)g.N;
  float cv[8];
  load8(oc + (bh * g.Nc + c) * D + ch * 8, cv);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int l = p * RPP + rsub;
    const long tok = base + cube_token(g, c, l);
    const long off = tok * D + ch * 8;
    float dov[8], ofv[8], a[8], b[8];
    load8_nt(d_o + off, dov);
    load8_nt(of + off, ofv);
    if (gc != nullptr) load8_nt(gc + off, a);
    else for (int i = 0; i < 8; ++i) a[i] = 1.f;
    if (gf != nullptr) load8_nt(gf + off, b);
    else for (int i = 0; i < 8; ++i) b[i] = 1.f;
    float r1[8], r2[8], r3[8];
    float dsum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      r1[i] = dov[i] * cv[i];
      r2[i] = dov[i] * ofv[i];
      r3[i] = round_to<T>(dov[i] * b[i]);  // d_o_f as stored
      dsum += r3[i] * ofv[i];
      acc[i] += dov[i] * a[i];
    }
    if (dgc != nullptr) store8_nt(dgc + off, r1);
    if (dgf != nullptr) store8_nt(dgf + off, r2);
    store8_nt(dof + off, r3);
#pragma unroll
    for (int o = CH / 2; o >= 1; o >>= 1) dsum += __shfl_xor(dsum, o, 64);
    if (ch == 0) delta[tok] = dsum;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[rsub][ch * 8 + i] = acc[i];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += part[r][tid];
    doc[(bh * g.Nc + c) * D + tid] = s;
  }
}

hipError_t launch_combine(const Launch& L, const float* oc, const void* of, const void* gc, const void* gf,
                          void* o) {
  const long nchunks = (long)L.BH * L.g.N * (L.D / 8);
  const dim3 grid((unsigned)((nchunks + 255) / 256)), block(256);
  if (L.bf16) {
    if (L.D == 64)
      hipLaunchKernelGGL((combine_kernel<bf16, 64>), grid, block, 0, L.stream, oc, (const bf16*)of,
                         (const bf16*)gc, (const bf16*)gf, (bf16*)o, L.g, nchunks);
    else
      hipLaunchKernelGGL((combine_kernel<bf16, 128>), grid, block, 0, L.stream, oc, (const bf16*)of,
                         (const bf16*)gc, (const bf16*)gf, (bf16*)o, L.g, nchunks);
  } else {
    if (L.D == 64)
      hipLaunchKernelGGL((combine_kernel<float, 64>), grid, block, 0, L.stream, oc, (const float*)of,
                         (const float*)gc, (const float*)gf, (float*)o, L.g, nchunks);
    else
      hipLaunchKernelGGL((combine_kernel<float, 128>), grid, block, 0, L.stream, oc, (const float*)of,
                         (const float*)gc, (const float*)gf, (float*)o, L.g, nchunks);
  }
  return hipGetLastError();
}

template <typename T, int D>
static void combine_bwd_launch(const Launch& L, const void* d_o, const float* oc, const void* of, const void* gc,
                               const void* gf, void* dgc, void* dgf, void* dof, float* delta, float* doc) {
  const dim3 grid(L.g.Nc, L.BH), block(256);
#define VSA_COMBINE_BWD(BT)                                                                                   \
  hipLaunchKernelGGL((combine_bwd_kernel<T, D, BT>), grid, block, 0, L.stream, (const T*)d_o, oc, (const T*)of, \
                     (const T*)gc, (const T*)gf, (T*)dgc, (T*)dgf, (T*)dof, delta, doc, L.g)
  if (L.g.B == 32) VSA_COMBINE_BWD(32);
  else if (L.g.B == 128) VSA_COMBINE_BWD(128);
  else if (L.g.B == 256) VSA_COMBINE_BWD(256);
  else VSA_COMBINE_BWD(64);
#undef VSA_COMBINE_BWD
}

hipError_t launch_combine_bwd(const Launch& L, const void* d_o, const float* oc, const void* of,
                              const void* gc, const void* gf, void* dgc, void* dgf, void* dof,
                              float* delta, float* doc) {
  if (L.bf16) {
    if (L.D == 64) combine_bwd_launch<bf16, 64>(L, d_o, oc, of, gc, gf, dgc, dgf, dof, delta, doc);
    else combine_bwd_launch<bf16, 128>(L, d_o, oc, of, gc, gf, dgc, dgf, dof, delta, doc);
  } else {
    if (L.D == 64) combine_bwd_launch<float, 64>(L, d_o, oc, of, gc, gf, dgc, dgf, dof, delta, doc);
    else combine_bwd_launch<float, 128>(L, d_o, oc, of, gc, gf, dgc, dgf, dof, delta, doc);
  }
  return hipGetLastError();
}

}  // namespace vsa
