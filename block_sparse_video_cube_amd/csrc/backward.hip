// Backward of VSA (steps 1 and 4) and the list utilities; the coarse
// attention's backward is with its forward GEMMs.
//
// The pages state that VSA trains end to end through one differentiable
// kernel and that the coarse output takes part in the result, so the pooled
// path also receives gradient (VSA summary page, paperlayer.ai arXiv
// 2505.13389, abstract and section 1; VSA reading notes, key design 1). The
// top-K mask is piecewise constant and is held fixed. The formulas are the
// calculus of softmax attention: with P = exp(s*q.k - LSE),
//   dV = P^T dO, dP = dO V^T, dS = P * (dP - delta), delta = rowsum(dO * O),
//   dQ = s * dS K, dK = s * dS^T Q,
// and the mean-pool spreads dX_c[c] / 64 over the cube's tokens.
//
// The fine backward is deterministic (no atomics): dQ walks each query cube's
// list (q2k), dK/dV walk the transposed lists (k2q) built by the index
// transpose.
#include "vsa_kernels.h"

namespace vsa {

// ------------------------------------------------------------ list helpers
// Index transpose through a key-major bitmask: bit i of row j of `bits`
// (W = ceil(Nc / 32) words per row) is set when query cube i lists key cube
// j. Counting a row's bits gives the length of j's list, and walking them
// writes it in ascending order, so the result is deterministic.
__global__ __launch_bounds__(256) void k2q_zero_kernel(uint32_t* __restrict__ bits, long n) {
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long)gridDim.x * 256) bits[e] = 0u;
}

__global__ __launch_bounds__(256) void k2q_bits_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ len, uint32_t* __restrict__ bits,
                                                       int Nc, int stride, int W) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;   // entry of this head's lists
  const long bh = blockIdx.y;
  if (e >= (long)Nc * stride) return;
  const int i = (int)(e / stride), t = (int)(e - (long)i * stride);
  const long row = bh * Nc + i;
  if (t >= min(max(len[row], 0), stride)) return;
  const int j = idx[row * stride + t];
  if (j < 0 || j >= Nc) return;
  atomicOr(&bits[(bh * Nc + j) * W + (i >> 5)], 1u << (i & 31));
}

// cnt[bh][j + 1] = number of query cubes listing j (cnt[bh][0] is set by the scan).
__global__ __launch_bounds__(256) void k2q_count_kernel(const uint32_t* __restrict__ bits, int32_t* __restrict__ cnt,
                                                        int Nc, int W) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const long bh = blockIdx.y;
  if (j >= Nc) return;
  const uint32_t* r = bits + (bh * Nc + j) * W;
  int c = 0;
  for (int w = 0; w < W; ++w) c += __popc(r[w]);
  cnt[bh * (Nc + 1) + j + 1] = c;
}

// In place: off[bh][0] = 0, off[bh][j+1] = count of j  ->  exclusive offsets.
__global__ __launch_bounds__(256) void k2q_scan_kernel(int32_t* __restrict__ off, int Nc) {
  __shared__ int part[256];
  const long bh = blockIdx.x;
  int32_t* o = off + bh * (Nc + 1);
  const int tid = threadIdx.x;
  const int per = (Nc + 255) / 256;
  const int b0 = tid * per, b1 = min(Nc, b0 + per);
  int s = 0;
  for (int j = b0; j < b1; ++j) s += o[j + 1];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int t = 0; t < 256; ++t) { const int v = part[t]; part[t] = run; run += v; }
  }
  __syncthreads();
  int run = part[tid];
  if (tid == 0) o[0] = 0;
  for (int j = b0; j < b1; ++j) { run += o[j + 1]; o[j + 1] = run; }
}

__global__ __launch_bounds__(256) void k2q_fill_kernel(const uint32_t* __restrict__ bits,
                                                       const int32_t* __restrict__ off, int32_t* __restrict__ k2q,
                                                       int Nc, int stride, int W) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const long bh = blockIdx.y;
  if (j >= Nc) return;
  const uint32_t* r = bits + (bh * Nc + j) * W;
  int32_t* out = k2q + bh * (long)Nc * stride;
  int pos = off[bh * (Nc + 1) + j];
  for (int w = 0; w < W; ++w) {
    uint32_t word = r[w];
    while (word != 0u) {
      out[pos++] = 32 * w + __ffs(word) - 1;
      word &= word - 1u;
    }
  }
}

int k2q_bits_words(int Nc) { return (Nc + 31) / 32; }

hipError_t launch_index_transpose(const Launch& L, const int32_t* idx, const int32_t* len, int32_t* k2q_off,
                                  int32_t* k2q, uint32_t* bits) {
  const int Nc = L.g.Nc, W = k2q_bits_words(Nc);
  const long nbits = (long)L.BH * Nc * W;
  hipLaunchKernelGGL(k2q_zero_kernel, dim3((unsigned)min((nbits + 255) / 256, 65536L)), dim3(256), 0, L.stream,
                     bits, nbits);
  const long entries = (long)Nc * L.stride;
  hipLaunchKernelGGL(k2q_bits_kernel, dim3((unsigned)((entries + 255) / 256), L.BH), dim3(256), 0, L.stream, idx,
                     len, bits, Nc, L.stride, W);
  const dim3 grid((Nc + 255) / 256, L.BH);
  hipLaunchKernelGGL(k2q_count_kernel, grid, dim3(256), 0, L.stream, bits, k2q_off, Nc, W);
  hipLaunchKernelGGL(k2q_scan_kernel, dim3(L.BH), dim3(256), 0, L.stream, k2q_off, Nc);
  hipLaunchKernelGGL(k2q_fill_kernel, grid, dim3(256), 0, L.stream, bits, k2q_off, k2q, Nc, L.stride, W);
  return hipGetLastError();
}

// Lists valid? len in [0, stride], ids in [0, Nc), strictly increasing.
__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ len, int32_t* flag, long rows,
                                                       int Nc, int stride) {
  const long r = (long)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int n = len[r];
  bool ok = n >= 0 && n <= stride;
  if (ok) {
    int prev = -1;
    for (int t = 0; t < n; ++t) {
      const int v = idx[r * stride + t];
      if (v <= prev || v >= Nc) { ok = false; break; }
      prev = v;
    }
  }
  if (!ok) atomicOr(flag, 1);
}

hipError_t launch_validate_lists(const Launch& L, const int32_t* idx, const int32_t* len, int32_t* flag) {
  const long rows = (long)L.BH * L.g.Nc;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, L.stream, idx, len,
                     flag, rows, L.g.Nc, L.stride);
  return hipGetLastError();
}

// ------------------------------------------------------------ fine backward
// dQ: one wave per query cube i, walking q2k[i] (the forward's lists).
//   S^T = K_j Q^T, dP^T = V_j dO_f^T       (A = raster rows of K_j / V_j)
//   P^T = exp2(S^T * s*log2e - LSE*log2e), dS^T = P^T * (dP^T - delta)
//   dQ^T += K_j^T dS^T                      (A = K T-tile of cube j)
// Every lane owns one query column, so LSE / delta are lane scalars.
template <int D>
__global__ __launch_bounds__(64) void fine_bwd_dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ kt, const int32_t* __restrict__ idx, const int32_t* __restrict__ len,
    const float* __restrict__ lse_f, const bf16* __restrict__ dof, const float* __restrict__ delta,
    const float* __restrict__ dqc, bf16* __restrict__ dq, Grid g, int stride, float scale) {
  constexpr int KS = D / 32, DB = D / 16;
  const int lane = threadIdx.x, c16 = lane & 15, grp = lane >> 4;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / g.Nc, i = item - bh * g.Nc;
  const long tok0 = (long)bh * g.N;
  const bf16* Q = q + tok0 * D;
  const bf16* K = k + tok0 * D;
  const bf16* V = v + tok0 * D;
  const bf16* DO = dof + tok0 * D;
  const float sl2 = scale * kLog2e;
  int qrow[4];
  float lse2[4], dl[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    qrow[qb] = cube_row(g, i, qb, c16 >> 2) + (c16 & 3);
    lse2[qb] = lse_f[tok0 + qrow[qb]] * kLog2e;
    dl[qb] = delta[tok0 + qrow[qb]];
  }
  bf16x8 qf[4][KS], df[4][KS];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qb][ks] = *reinterpret_cast<const bf16x8*>(Q + (long)qrow[qb] * D + ks * 32 + grp * 8);
      df[qb][ks] = *reinterpret_cast<const bf16x8*>(DO + (long)qrow[qb] * D + ks * 32 + grp * 8);
    }
  f32x4 acc[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int L = min(max(len[item], 0), stride);
  const int32_t* list = idx + (long)item * stride;
  for (int t = 0; t < L; ++t) {
    const int j = list[t];
    if (j < 0 || j >= g.Nc) continue;
    bf16x8 dsf[4][2];
    {
      f32x4 p[4][4];
      {
        bf16x8 kf[4][KS];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const long r = cube_row(g, j, kb, c16 >> 2) + (c16 & 3);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            kf[kb][ks] = *reinterpret_cast<const bf16x8*>(K + r * D + ks * 32 + grp * 8);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) a = mfma16_bf16(kf[kb][ks], qf[qb][ks], a);
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = __builtin_amdgcn_exp2f(a[r] * sl2 - lse2[qb]);
            p[kb][qb] = a;
          }
      }
      bf16x8 vf[4][KS];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const long r = cube_row(g, j, kb, c16 >> 2) + (c16 & 3);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          vf[kb][ks] = *reinterpret_cast<const bf16x8*>(V + r * D + ks * 32 + grp * 8);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) a = mfma16_bf16(vf[kb][ks], df[qb][ks], a);
#pragma unroll
          for (int r = 0; r < 4; ++r) dsf[qb][kb >> 1][(kb & 1) * 4 + r] = (bf16)(p[kb][qb][r] * (a[r] - dl[qb]));
        }
    }
    const bf16* ktile = kt + ((long)bh * g.Nc + j) * D * kTile;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int sx = 0; sx < 2; ++sx) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ktile + (db * 16 + c16) * kTile + sx * 32 + grp * 8);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) acc[db][qb] = mfma16_bf16(a, dsf[qb][sx], acc[db][qb]);
      }
  }
  // lane holds dQ^T[channel db*16 + 4*grp + r][query qb*16 + c16]
  const float* dqc_i = dqc + ((long)bh * g.Nc + i) * D;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const long n = tok0 + qrow[qb];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = db * 16 + 4 * grp;
      const float4 c4 = *reinterpret_cast<const float4*>(dqc_i + ch);
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
      bf16x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (bf16)(scale * acc[db][qb][r] + cv[r] * (1.0f / kTile));
      *reinterpret_cast<bf16x4*>(dq + n * D + ch) = w;
    }
  }
}

// dK, dV: one wave per key cube j, walking k2q[j].
//   S = Q_i K_j^T, dP = dO_i V_j^T       (A = raster rows of Q_i / dO_i, B = rows of K_j / V_j)
//   lane holds key column kb*16 + c16 and query rows qb*16 + 4*grp + r
//   P = exp2(S * s*log2e - LSE*log2e), dS = P * (dP - delta)
//   dV^T += dO_i^T P,  dK^T += Q_i^T dS  (A = T-tiles of cube i, B = P / dS)
template <int D>
__global__ __launch_bounds__(64) void fine_bwd_dkdv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ qt, const int32_t* __restrict__ k2q_off, const int32_t* __restrict__ k2q,
    const float* __restrict__ lse_f, const bf16* __restrict__ dof, const bf16* __restrict__ doft,
    const float* __restrict__ delta, const float* __restrict__ dkc, const float* __restrict__ dvc,
    bf16* __restrict__ dk, bf16* __restrict__ dv, Grid g, int stride, float scale) {
  constexpr int KS = D / 32, DB = D / 16;
  const int lane = threadIdx.x, c16 = lane & 15, grp = lane >> 4;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = item / g.Nc, j = item - bh * g.Nc;
  const long tok0 = (long)bh * g.N;
  const bf16* Q = q + tok0 * D;
  const bf16* DO = dof + tok0 * D;
  const float sl2 = scale * kLog2e;
  int krow[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) krow[kb] = cube_row(g, j, kb, c16 >> 2) + (c16 & 3);
  bf16x8 kf[4][KS], vf[4][KS];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[kb][ks] = *reinterpret_cast<const bf16x8*>(k + (tok0 + krow[kb]) * D + ks * 32 + grp * 8);
      vf[kb][ks] = *reinterpret_cast<const bf16x8*>(v + (tok0 + krow[kb]) * D + ks * 32 + grp * 8);
    }
  f32x4 adk[DB][4], adv[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      adk[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      adv[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const int32_t* offs = k2q_off + (long)bh * (g.Nc + 1);
  const int t0 = max(offs[j], 0), t1 = min(offs[j + 1], g.Nc * stride);
  const int32_t* list = k2q + (long)bh * g.Nc * stride;
  for (int t = t0; t < t1; ++t) {
    const int i = list[t];
    if (i < 0 || i >= g.Nc) continue;
    // query rows of this lane: qb*16 + 4*grp + r = token (t' = qb, y' = grp, x' = r)
    float lse2[4][4], dl[4][4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const long n = tok0 + cube_row(g, i, qb, grp);
      const float4 l4 = *reinterpret_cast<const float4*>(lse_f + n);
      const float4 d4 = *reinterpret_cast<const float4*>(delta + n);
      lse2[qb][0] = l4.x * kLog2e; lse2[qb][1] = l4.y * kLog2e;
      lse2[qb][2] = l4.z * kLog2e; lse2[qb][3] = l4.w * kLog2e;
      dl[qb][0] = d4.x; dl[qb][1] = d4.y; dl[qb][2] = d4.z; dl[qb][3] = d4.w;
    }
    bf16x8 pb[4][2], sb[4][2];   // [kb][k-step over queries]
    {
      f32x4 p[4][4];   // [qb][kb]
      {
        bf16x8 qf[4][KS];
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          const long r = cube_row(g, i, qb, c16 >> 2) + (c16 & 3);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = *reinterpret_cast<const bf16x8*>(Q + r * D + ks * 32 + grp * 8);
        }
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) a = mfma16_bf16(qf[qb][ks], kf[kb][ks], a);
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = __builtin_amdgcn_exp2f(a[r] * sl2 - lse2[qb][r]);
            p[qb][kb] = a;
          }
      }
      bf16x8 df[4][KS];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const long r = cube_row(g, i, qb, c16 >> 2) + (c16 & 3);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) df[qb][ks] = *reinterpret_cast<const bf16x8*>(DO + r * D + ks * 32 + grp * 8);
      }
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) a = mfma16_bf16(df[qb][ks], vf[kb][ks], a);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pb[kb][qb >> 1][(qb & 1) * 4 + r] = (bf16)p[qb][kb][r];
            sb[kb][qb >> 1][(qb & 1) * 4 + r] = (bf16)(p[qb][kb][r] * (a[r] - dl[qb][r]));
          }
        }
    }
    const bf16* dtile = doft + ((long)bh * g.Nc + i) * D * kTile;
    const bf16* qtile = qt + ((long)bh * g.Nc + i) * D * kTile;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int sx = 0; sx < 2; ++sx) {
        const int off = (db * 16 + c16) * kTile + sx * 32 + grp * 8;
        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dtile + off);
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qtile + off);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          adv[db][kb] = mfma16_bf16(ad, pb[kb][sx], adv[db][kb]);
          adk[db][kb] = mfma16_bf16(aq, sb[kb][sx], adk[db][kb]);
        }
      }
  }
  // lane holds d{K,V}^T[channel db*16 + 4*grp + r][key kb*16 + c16]
  const float* dkc_j = dkc + ((long)bh * g.Nc + j) * D;
  const float* dvc_j = dvc + ((long)bh * g.Nc + j) * D;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const long n = tok0 + krow[kb];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = db * 16 + 4 * grp;
      const float4 k4 = *reinterpret_cast<const float4*>(dkc_j + ch);
      const float4 v4 = *reinterpret_cast<const float4*>(dvc_j + ch);
      const float kcv[4] = {k4.x, k4.y, k4.z, k4.w}, vcv[4] = {v4.x, v4.y, v4.z, v4.w};
      bf16x4 wk, wv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wk[r] = (bf16)(scale * adk[db][kb][r] + kcv[r] * (1.0f / kTile));
        wv[r] = (bf16)(adv[db][kb][r] + vcv[r] * (1.0f / kTile));
      }
      *reinterpret_cast<bf16x4*>(dk + n * D + ch) = wk;
      *reinterpret_cast<bf16x4*>(dv + n * D + ch) = wv;
    }
  }
}

hipError_t launch_fine_bwd(const Launch& L, const bf16* q, const bf16* k, const bf16* v, const bf16* qt,
                           const bf16* kt, const int32_t* idx, const int32_t* len, const int32_t* k2q_off,
                           const int32_t* k2q, const float* lse_f, const bf16* dof, const bf16* doft,
                           const float* delta, const float* dqc, const float* dkc, const float* dvc, bf16* dq,
                           bf16* dk, bf16* dv) {
  const int nitems = L.BH * L.g.Nc;
  if (L.D == 64) {
    hipLaunchKernelGGL((fine_bwd_dq_kernel<64>), dim3(nitems), dim3(64), 0, L.stream, q, k, v, kt, idx, len, lse_f,
                       dof, delta, dqc, dq, L.g, L.stride, L.scale);
    hipLaunchKernelGGL((fine_bwd_dkdv_kernel<64>), dim3(nitems), dim3(64), 0, L.stream, q, k, v, qt, k2q_off, k2q,
                       lse_f, dof, doft, delta, dkc, dvc, dk, dv, L.g, L.stride, L.scale);
  } else {
    hipLaunchKernelGGL((fine_bwd_dq_kernel<128>), dim3(nitems), dim3(64), 0, L.stream, q, k, v, kt, idx, len,
                       lse_f, dof, delta, dqc, dq, L.g, L.stride, L.scale);
    hipLaunchKernelGGL((fine_bwd_dkdv_kernel<128>), dim3(nitems), dim3(64), 0, L.stream, q, k, v, qt, k2q_off,
                       k2q, lse_f, dof, doft, delta, dkc, dvc, dk, dv, L.g, L.stride, L.scale);
  }
  return hipGetLastError();
}

}  // namespace vsa
