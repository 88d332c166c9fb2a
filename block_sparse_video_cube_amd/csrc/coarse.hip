// Steps 2-3 of VSA: dense attention over the pooled cubes, the row-wise
// top-K and the mask-to-index conversion.
//
// VSA summary page (paperlayer.ai, arXiv 2505.13389), section 2 "Methods"
// (coarse stage: cube-level attention, Top-K critical cubes, no token-level
// matrix) and Appendix B (dense block attention, top-k of each row); VSA
// reading notes, key design 1 (A_c, O_c, row Top-K into mask M) and the
// training section (softmax, Top-K and mask-to-index fused in one kernel).
//
// Three kernels per call, all fp32:
//   1. coarse_scores: S = scale * Q_c K_c^T (fp32 MFMA GEMM) into workspace;
//   2. coarse_rows:   one wave per row: row max / sum -> LSE_c, then the exact
//                     top-K by a 4-pass radix select on the order-preserving
//                     integer image of the logits (ties: smaller cube id) and
//                     one ordered pass that writes the ascending index list
//                     (softmax, top-K and mask-to-index in one kernel);
//   3. coarse_pv:     O_c = exp(S - LSE_c) V_c (the same GEMM, the softmax
//                     applied to the operand as it is loaded).
// Selecting on the logits picks the same set as selecting on A_c: the
// softmax is increasing within a row. S_c is Nc^2 fp32 per (b, h) of
// workspace, written once and read twice (279 MB at the 720p latent).
#include "vsa_kernels.h"

namespace vsa {

constexpr int kCoarseMaxCubes = 2048;   // 32 logits per lane in coarse_rows

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Order-preserving map of an fp32 value to uint32 (+0 and -0 map alike).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// fp32 "NT" GEMM tile: C[m][n] = sum_k A[m][k] * B[n][k], A and B row-major
// with k contiguous. One wave computes a 32x32 tile as 2x2 16x16x4 MFMA
// blocks; lane (r = lane%16, g = lane/16) feeds, for every group of four
// k-steps t, the float4 A[r][16t + 4g .. +3] (k-step 4t+e contracts k =
// 16t + 4g + e), so loads are 16 bytes and four lanes cover 64 contiguous
// bytes of a row. Rows/columns beyond the matrix read as zero.
// ---------------------------------------------------------------------------
struct OperandQK {   // scores: A = Q_c, B = K_c, k = channel
  const float* p;
  int rows, ld;
  __device__ float4 ld4(int r, int k) const {
    if (r >= rows) return make_float4(0.f, 0.f, 0.f, 0.f);
    return *reinterpret_cast<const float4*>(p + (long)r * ld + k);
  }
};

struct OperandP {    // P = exp(S - LSE) rows, k = key cube (masked beyond Nc)
  const float* s;
  const float* lse;
  int rows, nk, ld;
  __device__ float4 ld4(int r, int k) const {
    if (r >= rows) return make_float4(0.f, 0.f, 0.f, 0.f);
    const float* row = s + (long)r * ld + k;
    const float l = lse[r];
    float4 o;
    o.x = k + 0 < nk ? __expf(row[0] - l) : 0.f;
    o.y = k + 1 < nk ? __expf(row[1] - l) : 0.f;
    o.z = k + 2 < nk ? __expf(row[2] - l) : 0.f;
    o.w = k + 3 < nk ? __expf(row[3] - l) : 0.f;
    return o;
  }
};

struct OperandVt {   // V_c^T: element (n = channel, k = key) = V_c[k][n]
  const float* v;
  int d, nk;
  __device__ float4 ld4(int n, int k) const {
    float4 o;
    o.x = k + 0 < nk ? v[(long)(k + 0) * d + n] : 0.f;
    o.y = k + 1 < nk ? v[(long)(k + 1) * d + n] : 0.f;
    o.z = k + 2 < nk ? v[(long)(k + 2) * d + n] : 0.f;
    o.w = k + 3 < nk ? v[(long)(k + 3) * d + n] : 0.f;
    return o;
  }
};

template <typename OA, typename OB>
__device__ __forceinline__ void gemm_nt_32x32(const OA& A, const OB& B, int m0, int n0, int K, f32x4 acc[2][2]) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int k = k0 + 4 * g;
    const float4 a0 = A.ld4(m0 + r, k), a1 = A.ld4(m0 + 16 + r, k);
    const float4 b0 = B.ld4(n0 + r, k), b1 = B.ld4(n0 + 16 + r, k);
    const float av[2][4] = {{a0.x, a0.y, a0.z, a0.w}, {a1.x, a1.y, a1.z, a1.w}};
    const float bv[2][4] = {{b0.x, b0.y, b0.z, b0.w}, {b1.x, b1.y, b1.z, b1.w}};
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16_f32(av[i][e], bv[j][e], acc[i][j]);
  }
}

// S[bh][i][j] = scale * Q_c[i] . K_c[j]; workgroup = 4 waves = 64x64 tile.
template <int D>
__global__ __launch_bounds__(256) void coarse_scores_kernel(const float* __restrict__ qc,
                                                            const float* __restrict__ kc, float* __restrict__ s,
                                                            int Nc, float scale) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
  const long bh = blockIdx.z;
  const int m0 = blockIdx.y * 64 + (w >> 1) * 32, n0 = blockIdx.x * 64 + (w & 1) * 32;
  const OperandQK A{qc + bh * (long)Nc * D, Nc, D}, B{kc + bh * (long)Nc * D, Nc, D};
  f32x4 acc[2][2];
  gemm_nt_32x32(A, B, m0, n0, D, acc);
  float* S = s + bh * (long)Nc * Nc;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + 16 * j + c16;
      if (col >= Nc) continue;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = m0 + 16 * i + 4 * g + rr;
        if (row < Nc) S[(long)row * Nc + col] = acc[i][j][rr] * scale;
      }
    }
}

// O_c[bh][i][dd] = sum_j exp(S[i][j] - LSE[i]) V_c[j][dd]; 64 rows x 64 channels per workgroup.
template <int D>
__global__ __launch_bounds__(256) void coarse_pv_kernel(const float* __restrict__ s, const float* __restrict__ lse,
                                                        const float* __restrict__ vc, float* __restrict__ oc, int Nc) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
  const long bh = blockIdx.z;
  const int m0 = blockIdx.y * 64 + (w >> 1) * 32, n0 = blockIdx.x * 64 + (w & 1) * 32;
  const OperandP A{s + bh * (long)Nc * Nc, lse + bh * Nc, Nc, Nc, Nc};
  const OperandVt B{vc + bh * (long)Nc * D, D, Nc};
  f32x4 acc[2][2];
  gemm_nt_32x32(A, B, m0, n0, (Nc + 15) & ~15, acc);
  float* O = oc + bh * (long)Nc * D;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + 16 * j + c16;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = m0 + 16 * i + 4 * g + rr;
        if (row < Nc) O[(long)row * D + col] = acc[i][j][rr];
      }
    }
}

// One wave per row: LSE_c, and with topk > 0 the ascending top-K list.
template <int NCH>
__global__ __launch_bounds__(256) void coarse_rows_kernel(const float* __restrict__ s, float* __restrict__ lse,
                                                          int32_t* __restrict__ idx, int32_t* __restrict__ len,
                                                          long rows, int Nc, int topk, int stride) {
  __shared__ int hist_all[4][256];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + w;
  if (row >= rows) return;   // wave-uniform; no block barrier below
  const float* srow = s + row * Nc;
  float v[NCH];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < NCH; ++t) {
    const int j = t * 64 + lane;
    v[t] = j < Nc ? srow[j] : -INFINITY;
    mx = fmaxf(mx, v[t]);
  }
  mx = wave_max(mx);
  float sm = 0.f;
#pragma unroll
  for (int t = 0; t < NCH; ++t) sm += __expf(v[t] - mx);   // exp(-inf) = 0 for padding
  sm = wave_sum(sm);
  if (lane == 0) lse[row] = mx + __logf(sm);
  if (topk <= 0) return;

  int* h = hist_all[w];
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t key[NCH];
#pragma unroll
  for (int t = 0; t < NCH; ++t) key[t] = (t * 64 + lane) < Nc ? fkey(v[t]) : 0u;
  uint32_t prefix = 0u, pmask = 0u;
  int krem = topk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < 256; b += 64) h[b] = 0;
    wave_sync();
#pragma unroll
    for (int t = 0; t < NCH; ++t)
      if ((t * 64 + lane) < Nc && (key[t] & pmask) == prefix) atomicAdd(&h[(key[t] >> shift) & 255u], 1);
    wave_sync();
    const int b0 = h[4 * lane], b1 = h[4 * lane + 1], b2 = h[4 * lane + 2], b3 = h[4 * lane + 3];
    const int mine = b0 + b1 + b2 + b3;
    int incl = mine;  // sum over lanes >= this lane (higher buckets)
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_down(incl, o, 64);
      if (lane + o < 64) incl += t;
    }
    int acc = incl - mine;
    int found = -1, before = 0;
    const int cnt[4] = {b3, b2, b1, b0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (found < 0 && acc < krem && acc + cnt[q] >= krem) { found = 4 * lane + 3 - q; before = acc; }
      acc += cnt[q];
    }
    const uint64_t bal = __ballot(found >= 0);
    const int src = __ffsll((unsigned long long)bal) - 1;
    const int fb = __shfl(found, src, 64);
    const int fbefore = __shfl(before, src, 64);
    prefix |= (uint32_t)fb << shift;
    pmask |= 0xFFu << shift;
    krem -= fbefore;
    wave_sync();
  }
  // prefix is the key of the K-th largest logit: take every larger one and
  // the first krem equal ones in ascending cube order.
  int32_t* out = idx + row * (long)stride;
  int taken = 0, eq_seen = 0;
#pragma unroll
  for (int t = 0; t < NCH; ++t) {
    const int j = t * 64 + lane;
    const bool valid = j < Nc;
    const bool gt = valid && key[t] > prefix;
    const bool eq = valid && key[t] == prefix;
    const uint64_t beq = __ballot(eq);
    const int eqr = eq_seen + __popcll(beq & lt_mask);
    const bool take = gt || (eq && eqr < krem);
    const uint64_t bt = __ballot(take);
    const int pos = taken + __popcll(bt & lt_mask);
    if (take && pos < topk) out[pos] = j;
    taken += __popcll(bt);
    eq_seen += __popcll(beq);
  }
  for (int j = topk + lane; j < stride; j += 64) out[j] = -1;
  if (lane == 0) len[row] = topk;
}

int coarse_max_cubes() { return kCoarseMaxCubes; }

template <int NCH>
static void launch_rows(const Launch& L, const float* s, float* lse, int32_t* idx, int32_t* len) {
  const long rows = (long)L.BH * L.g.Nc;
  hipLaunchKernelGGL((coarse_rows_kernel<NCH>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, L.stream, s, lse,
                     idx, len, rows, L.g.Nc, L.topk, L.stride);
}

hipError_t launch_coarse(const Launch& L, const float* qc, const float* kc, const float* vc, float* oc,
                         float* lse, int32_t* idx, int32_t* len, float* s_scratch) {
  const int Nc = L.g.Nc;
  const int t64 = (Nc + 63) / 64;
  const dim3 block(256);
  if (L.D == 64)
    hipLaunchKernelGGL((coarse_scores_kernel<64>), dim3(t64, t64, L.BH), block, 0, L.stream, qc, kc, s_scratch, Nc,
                       L.scale);
  else
    hipLaunchKernelGGL((coarse_scores_kernel<128>), dim3(t64, t64, L.BH), block, 0, L.stream, qc, kc, s_scratch, Nc,
                       L.scale);
  if (Nc <= 256) launch_rows<4>(L, s_scratch, lse, idx, len);
  else if (Nc <= 512) launch_rows<8>(L, s_scratch, lse, idx, len);
  else if (Nc <= 1024) launch_rows<16>(L, s_scratch, lse, idx, len);
  else launch_rows<32>(L, s_scratch, lse, idx, len);
  if (L.D == 64)
    hipLaunchKernelGGL((coarse_pv_kernel<64>), dim3(1, t64, L.BH), block, 0, L.stream, s_scratch, lse, vc, oc, Nc);
  else
    hipLaunchKernelGGL((coarse_pv_kernel<128>), dim3(2, t64, L.BH), block, 0, L.stream, s_scratch, lse, vc, oc, Nc);
  return hipGetLastError();
}

}  // namespace vsa
