// Step 4 of VSA: fine block-sparse attention, optionally fused with step 5
// (gated combine + untile) in the epilogue.
//
// VSA summary page (paperlayer.ai, arXiv 2505.13389), section 2 "Methods"
// (fine stage: token attention only inside the selected cubes, expanded to
// 64x64 blocks; gating combines coarse and fine) and Appendix B (token QK,
// mask unselected, softmax, times V; combine, untile); VSA reading notes,
// key designs 2-3. Variable-length lists per query cube: VSA2 abstract.
//
// bf16 kernel: one wave owns one query cube (64 query rows) and walks its
// list of key cubes (in 32-key halves) with an online softmax, all in
// registers:
//   S^T = K_j Q_i^T   16x16x32 bf16 MFMAs, A = K rows, B = Q rows (both read
//                     straight from the raster tensors, 16-byte loads);
//   the accumulator layout gives every lane one query column and 4+4+4+4 key
//   rows, so row max / sum are lane-local plus one exchange over the 4 lane
//   groups, and P^T is already the B operand of
//   O^T += V_j^T P^T  with A = the V T-tile of cube j (channel rows, keys
//                     contiguous in the accumulator's slot order).
// Every lane ends with O^T for its query column, so the 1/l normalisation,
// LSE and the fused gate epilogue need no data exchange.
#include "vsa_kernels.h"

namespace vsa {

// Occupancy: D = 64 fits 2 waves per SIMD (<= 256 registers), D = 128 one.
template <int D> struct FineOcc { static constexpr int kWaves = D == 64 ? 2 : 1; };

template <int D, bool FUSED>
__global__ __launch_bounds__(64, FineOcc<D>::kWaves) void fine_fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ vt,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ len, bf16* __restrict__ o_f,
    float* __restrict__ lse_f, const float* __restrict__ oc, const bf16* __restrict__ gc,
    const bf16* __restrict__ gf, bf16* __restrict__ o, Grid g, int stride, float scale_log2) {
  constexpr int KS = D / 32;   // k-steps of the QK^T contraction
  constexpr int DB = D / 16;   // 16-channel blocks of the output
  const int lane = threadIdx.x, c16 = lane & 15, grp = lane >> 4;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / g.Nc, i = item - bh * g.Nc;
  const long tok0 = (long)bh * g.N;
  const bf16* Q = q + tok0 * D;
  const bf16* K = k + tok0 * D;
  // Lists are validated by contract; the clamps only keep a malformed list
  // from reading outside the tensors.
  const int L = min(max(len[item], 0), stride);
  const int32_t* list = idx + (long)item * stride;

  // Query rows of this lane: token qb*16 + c16 of cube i, qb = 0..3, i.e.
  // (t' = qb, y' = c16 / 4, x' = c16 % 4).
  int qrow[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) qrow[qb] = cube_row(g, i, qb, c16 >> 2) + (c16 & 3);

  bf16x8 qf[4][KS];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qb][ks] = *reinterpret_cast<const bf16x8*>(Q + (long)qrow[qb] * D + ks * 32 + grp * 8);

  f32x4 acc[DB][4], lacc[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Reference max per query (log2 units), common to the 4 lanes of a query.
  float m[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) m[qb] = -INFINITY;
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;

  // The list is walked in 32-key chunks, two per key cube: chunk h of cube j
  // holds the key rows t' = 2h, 2h+1 (tokens 32h .. 32h+31), which is exactly
  // k-step h of the cube's V T-tile. Online softmax over any chunking is the
  // same softmax.
  auto cube_at = [&](int t) { const int j = list[t]; return (j >= 0 && j < g.Nc) ? j : 0; };
  bf16x8 kf[2][KS];
  auto load_k = [&](int j, int h) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const long r = cube_row(g, j, 2 * h + kk, c16 >> 2) + (c16 & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[kk][ks] = *reinterpret_cast<const bf16x8*>(K + r * D + ks * 32 + grp * 8);
    }
  };
  const int nchunks = 2 * L;

  auto scores = [&](f32x4 (&sx)[2][4]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a = mfma16_bf16(kf[kk][ks], qf[qb][ks], a);
        sx[kk][qb] = a;
      }
  };

  // Online softmax against a lazily moved reference max m (log2 units): P =
  // 2^(s*c - m) is formed as long as no exponent exceeds 16 (P < 2^16, so
  // bf16 P and the fp32 sums keep their relative precision). A chunk that
  // would exceed it leaves the hot loop; the reference then moves up to the
  // chunk's row max, O and l are rescaled, and the chunk is redone. O and l
  // always share m, so the result is exact whatever the schedule. The row
  // sum l comes from an MFMA against a ones operand, so the hot loop touches
  // the accumulators only through MFMAs. The first chunk's row max sets the
  // initial reference.
  constexpr float kHeadroom = 16.0f;
  if (nchunks > 0) {
    load_k(cube_at(0), 0);
    f32x4 sx[2][4];
    scores(sx);
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float mx = fmaxf(fmaxf(fmaxf(sx[0][qb][0], sx[0][qb][1]), fmaxf(sx[0][qb][2], sx[0][qb][3])),
                       fmaxf(fmaxf(sx[1][qb][0], sx[1][qb][1]), fmaxf(sx[1][qb][2], sx[1][qb][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      m[qb] = mx * scale_log2;
    }
  }
  int c = 0;
  for (;;) {
    bool retry = false;
    float cmax[4];
    if (c < nchunks) load_k(cube_at(c >> 1), c & 1);
    for (; c < nchunks; ++c) {
      const int h = c & 1;
      const int j = cube_at(c >> 1);
      bf16x8 vf[DB];
      const bf16* vtile = vt + ((long)bh * g.Nc + j) * D * kTile;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        vf[db] = *reinterpret_cast<const bf16x8*>(vtile + (db * 16 + c16) * kTile + h * 32 + grp * 8);
      // S^T[kk][qb]: lane holds keys 32h + 16kk + 4*grp + r of query qb*16 + c16.
      f32x4 sx[2][4];
      scores(sx);
      // exponent arguments x = s*c - m, and the largest of them per query
      float xmax = -INFINITY;
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        float mq = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sx[kk][qb][r] = sx[kk][qb][r] * scale_log2 - m[qb];
            mq = fmaxf(mq, sx[kk][qb][r]);
          }
        cmax[qb] = mq;
        xmax = fmaxf(xmax, mq);
      }
      if (__any(xmax > kHeadroom)) { retry = true; break; }
      if (c + 1 < nchunks) load_k(cube_at((c + 1) >> 1), h ^ 1);
      bf16x8 pf[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 4; ++r) pf[qb][kk * 4 + r] = (bf16)__builtin_amdgcn_exp2f(sx[kk][qb][r]);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        lacc[qb] = mfma16_bf16(ones, pf[qb], lacc[qb]);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db][qb] = mfma16_bf16(vf[db], pf[qb], acc[db][qb]);
      }
    }
    if (!retry) break;
    // Rare path: move each query's reference up to its row max over this
    // chunk (the 4 lanes of a query agree through two exchanges); rescale.
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float mx = cmax[qb];
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float shift = fmaxf(mx, 0.0f);
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      m[qb] += shift;
      lacc[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
    }
  }
  float l[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) l[qb] = lacc[qb][0];

  // Epilogue: lane holds O^T[channel db*16 + 4*grp + r][query qb*16 + c16].
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const float lt = l[qb];
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const long n = tok0 + qrow[qb];
    if (lse_f != nullptr && grp == 0)
      lse_f[n] = lt > 0.f ? (m[qb] + __log2f(lt)) * kLn2 : -INFINITY;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = db * 16 + 4 * grp;
      float of[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) of[r] = acc[db][qb][r] * inv;
      if (o_f != nullptr) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (bf16)of[r];
        *reinterpret_cast<bf16x4*>(o_f + n * D + ch) = w;
      }
      if (FUSED) {
        // Round O_f to bf16 first so the fused output equals the unfused
        // combine of the stored O_f.
        const float4 c4 = *reinterpret_cast<const float4*>(oc + ((long)bh * g.Nc + i) * D + ch);
        const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
        bf16x4 gcv, gfv;
        if (gc != nullptr) gcv = *reinterpret_cast<const bf16x4*>(gc + n * D + ch);
        if (gf != nullptr) gfv = *reinterpret_cast<const bf16x4*>(gf + n * D + ch);
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = gc != nullptr ? (float)gcv[r] : 1.f;
          const float b = gf != nullptr ? (float)gfv[r] : 1.f;
          w[r] = (bf16)(cv[r] * a + (float)(bf16)of[r] * b);
        }
        *reinterpret_cast<bf16x4*>(o + n * D + ch) = w;
      }
    }
  }
}

// fp32 path: one thread per query token, K/V tiles staged in LDS. Used for
// fp32 problems (small, correctness-first shapes).
template <int D, bool FUSED>
__global__ __launch_bounds__(64) void fine_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ len, float* __restrict__ o_f,
    float* __restrict__ lse_f, const float* __restrict__ oc, const float* __restrict__ gc,
    const float* __restrict__ gf, float* __restrict__ o, Grid g, int stride, float scale) {
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  const int tid = threadIdx.x;
  const int item = blockIdx.x;
  const int bh = item / g.Nc, i = item - bh * g.Nc;
  const long tok0 = (long)bh * g.N;
  const long n = tok0 + cube_token(g, i, tid);
  float qv[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { qv[d] = q[n * D + d]; acc[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const int L = min(max(len[item], 0), stride);
  const int32_t* list = idx + (long)item * stride;
  for (int t = 0; t < L; ++t) {
    const int j = list[t];
    if (j < 0 || j >= g.Nc) continue;
    __syncthreads();
    for (int e = tid; e < kTile * D; e += 64) {
      const int r = e / D, d = e - r * D;
      const long src = (tok0 + cube_token(g, j, r)) * D + d;
      ks[r][d] = k[src];
      vs[r][d] = v[src];
    }
    __syncthreads();
    for (int r = 0; r < kTile; ++r) {
      float z = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) z = fmaf(qv[d], ks[r][d], z);
      z *= scale;
      const float mnew = fmaxf(m, z);
      const float alpha = expf(m - mnew);
      const float p = expf(z - mnew);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[r][d], acc[d] * alpha);
      m = mnew;
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (lse_f != nullptr) lse_f[n] = l > 0.f ? m + logf(l) : -INFINITY;
  for (int d = 0; d < D; ++d) {
    const float of = acc[d] * inv;
    if (o_f != nullptr) o_f[n * D + d] = of;
    if (FUSED) {
      const float a = gc != nullptr ? gc[n * D + d] : 1.f;
      const float b = gf != nullptr ? gf[n * D + d] : 1.f;
      o[n * D + d] = oc[((long)bh * g.Nc + i) * D + d] * a + of * b;
    }
  }
}

template <int D, bool FUSED>
static void fine_launch_bf16(const Launch& L, const void* q, const void* k, const bf16* vt, const int32_t* idx,
                             const int32_t* len, void* o_f, float* lse_f, const float* oc, const void* gc,
                             const void* gf, void* o) {
  const int nitems = L.BH * L.g.Nc;
  hipLaunchKernelGGL((fine_fwd_bf16_kernel<D, FUSED>), dim3(nitems), dim3(64), 0, L.stream, (const bf16*)q,
                     (const bf16*)k, vt, idx, len, (bf16*)o_f, lse_f, oc, (const bf16*)gc, (const bf16*)gf,
                     (bf16*)o, L.g, L.stride, L.scale * kLog2e);
}

template <int D, bool FUSED>
static void fine_launch_f32(const Launch& L, const void* q, const void* k, const void* v, const int32_t* idx,
                            const int32_t* len, void* o_f, float* lse_f, const float* oc, const void* gc,
                            const void* gf, void* o) {
  const int nitems = L.BH * L.g.Nc;
  hipLaunchKernelGGL((fine_fwd_f32_kernel<D, FUSED>), dim3(nitems), dim3(64), 0, L.stream, (const float*)q,
                     (const float*)k, (const float*)v, idx, len, (float*)o_f, lse_f, oc, (const float*)gc,
                     (const float*)gf, (float*)o, L.g, L.stride, L.scale);
}

hipError_t launch_fine_fwd(const Launch& L, const void* q, const void* k, const void* v, const bf16* vt,
                           const int32_t* idx, const int32_t* len, void* o_f, float* lse_f, const float* oc,
                           const void* g_c, const void* g_f, void* o) {
  const bool fused = oc != nullptr;
  if (L.bf16) {
    if (L.D == 64) {
      if (fused) fine_launch_bf16<64, true>(L, q, k, vt, idx, len, o_f, lse_f, oc, g_c, g_f, o);
      else fine_launch_bf16<64, false>(L, q, k, vt, idx, len, o_f, lse_f, oc, g_c, g_f, o);
    } else {
      if (fused) fine_launch_bf16<128, true>(L, q, k, vt, idx, len, o_f, lse_f, oc, g_c, g_f, o);
      else fine_launch_bf16<128, false>(L, q, k, vt, idx, len, o_f, lse_f, oc, g_c, g_f, o);
    }
  } else {
    if (L.D == 64) {
      if (fused) fine_launch_f32<64, true>(L, q, k, v, idx, len, o_f, lse_f, oc, g_c, g_f, o);
      else fine_launch_f32<64, false>(L, q, k, v, idx, len, o_f, lse_f, oc, g_c, g_f, o);
    } else {
      if (fused) fine_launch_f32<128, true>(L, q, k, v, idx, len, o_f, lse_f, oc, g_c, g_f, o);
      else fine_launch_f32<128, false>(L, q, k, v, idx, len, o_f, lse_f, oc, g_c, g_f, o);
    }
  }
  return hipGetLastError();
}

}  // namespace vsa
