// Steps 2-3 of VSA: dense attention over the pooled cubes, fused with the
// row-wise top-K and the mask-to-index conversion.
//
// VSA summary page (paperlayer.ai, arXiv 2505.13389), section 2 "Methods"
// (coarse stage: cube-level attention, Top-K critical cubes, no token-level
// matrix) and Appendix B (dense block attention, top-k of each row); VSA
// reading notes, key design 1 (A_c, O_c, row Top-K into mask M) and the
// training section (softmax, Top-K and mask-to-index fused in one kernel).
//
// One workgroup (4 waves) owns 16 query cubes of one (b, h):
//   1. S = scale * Q_c K_c^T for its 16 rows, fp32 MFMA (16x16x4), kept in LDS;
//   2. row max / sum -> LSE_c;
//   3. exact top-K of each row by a 4-pass radix select on the order-
//      preserving integer image of the fp32 logits (ties: smaller cube id),
//      then one ordered pass emits the ascending index list;
//   4. P = softmax rows in place, O_c = P V_c (fp32 MFMA).
// Selecting on the logits picks the same set as selecting on A_c: the
// softmax is increasing within a row.
#include "vsa_kernels.h"

namespace vsa {

constexpr int kCoarseRows = 16;
constexpr int kCoarseMaxCubes = 2048;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Order-preserving map of an fp32 value to uint32 (+0 and -0 map alike).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int D>
__global__ __launch_bounds__(256) void coarse_kernel(const float* __restrict__ qc, const float* __restrict__ kc,
                                                     const float* __restrict__ vc, float* __restrict__ oc,
                                                     float* __restrict__ lse, int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ len, int Nc, int pitch, int topk,
                                                     int stride, float scale) {
  extern __shared__ float smem[];
  float* S = smem;                               // [16][pitch]
  float* rowm = S + kCoarseRows * pitch;         // [16] row max
  float* rowinv = rowm + kCoarseRows;            // [16] 1 / row sum
  int* hist = reinterpret_cast<int*>(rowinv + kCoarseRows);  // [4 waves][256]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const long bh = blockIdx.y;
  const int r0 = blockIdx.x * kCoarseRows;
  const float* Q = qc + bh * (long)Nc * D;
  const float* K = kc + bh * (long)Nc * D;
  const float* V = vc + bh * (long)Nc * D;

  // ---- 1. scores. k-step (j, e) of the MFMA contracts channel 16j + 4g + e.
  float qa[D / 4];
  {
    const int row = r0 + c16;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row < Nc) t = *reinterpret_cast<const float4*>(Q + (long)row * D + 16 * j + 4 * g);
      qa[4 * j] = t.x; qa[4 * j + 1] = t.y; qa[4 * j + 2] = t.z; qa[4 * j + 3] = t.w;
    }
  }
  const int nkb = (Nc + 15) >> 4;
  for (int kb = w; kb < nkb; kb += 4) {
    const int key = kb * 16 + c16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
      if (key < Nc) t = *reinterpret_cast<const float4*>(K + (long)key * D + 16 * j + 4 * g);
      acc = mfma16_f32(qa[4 * j], t.x, acc);
      acc = mfma16_f32(qa[4 * j + 1], t.y, acc);
      acc = mfma16_f32(qa[4 * j + 2], t.z, acc);
      acc = mfma16_f32(qa[4 * j + 3], t.w, acc);
    }
    if (key < Nc) {
#pragma unroll
      for (int r = 0; r < 4; ++r) S[(4 * g + r) * pitch + key] = acc[r] * scale;
    }
  }
  __syncthreads();

  // ---- 2. row statistics (wave w: rows 4w .. 4w+3)
  for (int rr = 0; rr < 4; ++rr) {
    const int row = 4 * w + rr;
    if (r0 + row >= Nc) break;
    const float* srow = S + row * pitch;
    float mx = -INFINITY;
    for (int j = lane; j < Nc; j += 64) mx = fmaxf(mx, srow[j]);
    mx = wave_max(mx);
    float sm = 0.f;
    for (int j = lane; j < Nc; j += 64) sm += __expf(srow[j] - mx);
    sm = wave_sum(sm);
    if (lane == 0) {
      rowm[row] = mx;
      rowinv[row] = 1.0f / sm;
      lse[bh * Nc + r0 + row] = mx + __logf(sm);
    }
  }

  // ---- 3. top-K + mask-to-index (wave w: rows 4w .. 4w+3)
  if (topk > 0) {
    int* h = hist + w * 256;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int rr = 0; rr < 4; ++rr) {
      const int row = 4 * w + rr;
      const int grow = r0 + row;
      if (grow >= Nc) break;
      const float* srow = S + row * pitch;
      uint32_t prefix = 0u, pmask = 0u;
      int krem = topk;
      for (int shift = 24; shift >= 0; shift -= 8) {
        for (int b = lane; b < 256; b += 64) h[b] = 0;
        wave_sync();
        for (int j = lane; j < Nc; j += 64) {
          const uint32_t u = fkey(srow[j]);
          if ((u & pmask) == prefix) atomicAdd(&h[(u >> shift) & 255u], 1);
        }
        wave_sync();
        const int b0 = h[4 * lane], b1 = h[4 * lane + 1], b2 = h[4 * lane + 2], b3 = h[4 * lane + 3];
        const int mine = b0 + b1 + b2 + b3;
        int incl = mine;  // sum over lanes >= lane (buckets at or above this lane's)
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_down(incl, o, 64);
          if (lane + o < 64) incl += t;
        }
        int acc = incl - mine;  // elements in higher buckets
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
      // prefix is now the key of the K-th largest logit; take every larger
      // one and the first krem equal ones in ascending cube order.
      int32_t* out = idx + (bh * Nc + grow) * (long)stride;
      int taken = 0, eq_seen = 0;
      for (int j0 = 0; j0 < Nc; j0 += 64) {
        const int j = j0 + lane;
        const bool valid = j < Nc;
        const uint32_t u = valid ? fkey(srow[j]) : 0u;
        const bool gt = valid && u > prefix;
        const bool eq = valid && u == prefix;
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
      if (lane == 0) len[bh * Nc + grow] = topk;
    }
  }
  __syncthreads();

  // ---- 4. P = softmax rows in place (columns padded to a multiple of 4 with 0)
  const int nc4 = (Nc + 3) & ~3;
  for (int e = tid; e < kCoarseRows * nc4; e += 256) {
    const int row = e / nc4, j = e - row * nc4;
    float p = 0.f;
    if (r0 + row < Nc && j < Nc) p = __expf(S[row * pitch + j] - rowm[row]) * rowinv[row];
    S[row * pitch + j] = p;
  }
  __syncthreads();

  // O_c = P V_c: waves split the 16-channel blocks.
  for (int db = w; db < D / 16; db += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int ks = 0; ks < nc4 / 4; ++ks) {
      const int key = 4 * ks + g;
      const float a = S[c16 * pitch + key];
      const float b = key < Nc ? V[(long)key * D + db * 16 + c16] : 0.f;
      acc = mfma16_f32(a, b, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = r0 + 4 * g + r;
      if (row < Nc) oc[(bh * Nc + row) * D + db * 16 + c16] = acc[r];
    }
  }
}

int coarse_max_cubes() { return kCoarseMaxCubes; }

static size_t coarse_smem(int Nc, int* pitch) {
  *pitch = ((Nc + 15) & ~15) + 4;
  return (size_t)(kCoarseRows * (*pitch) + 2 * kCoarseRows) * sizeof(float) + 4 * 256 * sizeof(int);
}

hipError_t launch_coarse(const Launch& L, const float* qc, const float* kc, const float* vc, float* oc,
                         float* lse, int32_t* idx, int32_t* len) {
  int pitch = 0;
  const size_t smem = coarse_smem(L.g.Nc, &pitch);
  const dim3 grid((L.g.Nc + kCoarseRows - 1) / kCoarseRows, L.BH), block(256);
  hipError_t e;
  if (L.D == 64) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&coarse_kernel<64>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((coarse_kernel<64>), grid, block, smem, L.stream, qc, kc, vc, oc, lse, idx, len, L.g.Nc,
                       pitch, L.topk, L.stride, L.scale);
  } else {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&coarse_kernel<128>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((coarse_kernel<128>), grid, block, smem, L.stream, qc, kc, vc, oc, lse, idx, len, L.g.Nc,
                       pitch, L.topk, L.stride, L.scale);
  }
  return hipGetLastError();
}

}  // namespace vsa
