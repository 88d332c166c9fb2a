// Steps 2-3 of VSA: dense attention over the pooled cubes, the row-wise
// top-K and the mask-to-index conversion.
//
// VSA summary page (paperlayer.ai, arXiv 2505.13389), section 2 "Methods"
// (coarse stage: cube-level attention, Top-K critical cubes, no token-level
// matrix) and Appendix B (dense block attention, top-k of each row); VSA
// reading notes, key design 1 (A_c, O_c, row Top-K into mask M) and the
// training section (softmax, Top-K and mask-to-index fused in one kernel).
//
// Three kernels per forward call:
//   1. coarse_scores: S = scale * Q_c K_c^T (fp32 MFMA GEMM) into workspace;
//   2. coarse_rows:   one wave per row: row max / sum -> LSE_c, then the exact
//                     top-K by a 4-pass radix select on the order-preserving
//                     integer image of the logits (ties: smaller cube id) and
//                     one ordered pass that writes the ascending index list
//                     (softmax, top-K and mask-to-index in one kernel);
//   3. coarse_gemm:   O_c = exp(S - LSE_c) V_c (an LDS-tiled GEMM, the
//                     softmax applied to the operand as it is staged); for
//                     bf16 problems coarse_pv_bf16 instead, the same product
//                     on bf16 MFMAs with a three-term split of the fp32
//                     operands (fp32-level accuracy).
// The backward of the coarse attention is here too; it shares these GEMMs.
// Selecting on the logits picks the same set as selecting on A_c: the
// softmax is increasing within a row. S_c is Nq x Nk fp32 per (b, h) of
// workspace (Nq query cubes, Nk key blocks; rows padded to a multiple of 4
// floats), written once and read twice (279 MB at the 720p latent).
#include "vsa_kernels.h"
#include "fine_common.h"

namespace vsa {

constexpr int kCoarseMaxCubes = 8192;   // rows of up to 2048 logits in registers, longer ones streamed
constexpr int kRowsInRegisters = 2048;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Order-preserving map of an fp32 value to uint32 (+0 and -0 map alike).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave's 64x64 block of an "NT" product C = A B^T with A [Na][D] and
// B [Nb][D] row-major (fp32 16x16x4 MFMAs, 4x4 blocks). Lane (r = lane%16, g = lane/16)
// holds, for channel group t, the float4 A[row r][16t + 4g .. +3] (and
// likewise B), so four lanes cover 64 contiguous bytes of a row; k-step 4t+e
// contracts channel 16t + 4g + e. With NBUF = 2 channel groups are
// double-buffered in registers (the next group loads while this one's 64
// MFMAs run); NBUF = 1 loads each group just before its MFMAs, 32 registers
// fewer. Rows beyond Na (of A) or Nb (of B) read as zero. acc[i][j][e] is
// C[m0 + 16i + 4g + e][n0 + 16j + r].
template <int D, int NBUF = 2>
__device__ __forceinline__ void nt_block64(const float* __restrict__ A, const float* __restrict__ B, int Na,
                                           int Nb, int m0, int n0, f32x4 acc[4][4]) {
  constexpr int KT = D / 16;
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  float4 av[NBUF][4], bv[NBUF][4];
  auto load = [&](int t, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = m0 + 16 * i + r, rb = n0 + 16 * i + r;
      av[buf][i] = ra < Na ? *reinterpret_cast<const float4*>(A + (long)ra * D + 16 * t + 4 * g)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
      bv[buf][i] = rb < Nb ? *reinterpret_cast<const float4*>(B + (long)rb * D + 16 * t + 4 * g)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (NBUF == 2) load(0, 0);
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    if (NBUF == 1) load(t, 0);
    else if (t + 1 < KT) load(t + 1, (t + 1) % NBUF);
    const int bf = t % NBUF;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = e == 0 ? av[bf][i].x : e == 1 ? av[bf][i].y : e == 2 ? av[bf][i].z : av[bf][i].w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float b = e == 0 ? bv[bf][j].x : e == 1 ? bv[bf][j].y : e == 2 ? bv[bf][j].z : bv[bf][j].w;
          acc[i][j] = mfma16_f32(a, b, acc[i][j]);
        }
      }
  }
}

// S[bh][i][j] = scale * Q_c[i] . K_c[j] over Nq query cubes and Nk key
// blocks; a workgroup of 4 waves owns a 128x128 tile, each wave a 64x64
// quarter.
template <int D>
__global__ __launch_bounds__(256) void coarse_scores_kernel(const float* __restrict__ qc,
                                                            const float* __restrict__ kc, float* __restrict__ s,
                                                            int Nq, int Nk, int ld, float scale) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const Tile3 t = tile3((Nk + 127) / 128, (Nq + 127) / 128);
  const long bh = t.z;
  const int m0 = t.y * 128 + (w >> 1) * 64, n0 = t.x * 128 + (w & 1) * 64;
  if (m0 >= Nq || n0 >= Nk) return;   // wave-uniform; no barrier in this kernel
  f32x4 acc[4][4];
  nt_block64<D>(qc + bh * (long)Nq * D, kc + bh * (long)Nk * D, Nq, Nk, m0, n0, acc);
  float* S = s + bh * (long)Nq * ld;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + 16 * j + r;
      if (col >= Nk) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + 16 * i + 4 * g + e;
        if (row < Nq) S[(long)row * ld + col] = acc[i][j][e] * scale;
      }
    }
}

// The coarse logits of a bf16 problem on bf16 MFMAs, to fp32 accuracy: every
// fp32 operand x is split exactly into three bf16 pieces, x = hi + mid + lo
// (hi = bf16(x), mid = bf16(x - hi), lo = x - hi - mid, which needs no more
// than bf16's 8 significant bits), and the dot product over channels is
// formed from the six piece products whose size exceeds 2^-24 of the whole:
// hi.hi into one accumulator, hi.mid, mid.hi, hi.lo, lo.hi and mid.mid into a
// second (each product of two bf16 values is exact in fp32), the two added at
// the end. Against an fp32 dot product this adds at most 2^-23 of sum |q||k|
// per channel for the dropped products (mid.lo, lo.mid, lo.lo) and the
// rounding of the second accumulator, whose partial sums stay below 2^-7 of
// the first's scale: the error bound grows by under 10% (the oracle's logit
// error bound counts this arithmetic). A workgroup of four waves owns a
// 128 x 128 tile of S, a wave a 64 x 64 quarter as four 32 x 32 MFMA tiles.
// Per k-step of 16 channels the workgroup loads the tile's 128 rows of Q_c
// and of K_c once (coalesced, a row's 64 bytes by four lanes), splits every
// value once, and stages the pieces in LDS (double buffered, one barrier per
// k-step), where each wave reads its MFMA fragments (a row's 8 channels,
// 16 bytes, per lane). S leaves through LDS as whole 16-byte row units. The
// vector memory path bounds this kernel (address and data units about 85%
// busy with per-lane fragment loads and 4-byte stores), so both go in fewer,
// wider accesses. Rows past Nq / Nk are clamped for the loads and not stored.
__device__ __forceinline__ void split3(const float4& x0, const float4& x1, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (bf16)x[e];
    const float r1 = x[e] - (float)hi[e];
    mid[e] = (bf16)r1;
    lo[e] = (bf16)(r1 - (float)mid[e]);
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void coarse_scores_split_kernel(const float* __restrict__ qc,
                                                                    const float* __restrict__ kc,
                                                                    float* __restrict__ s, int Nq, int Nk, int ld,
                                                                    float scale) {
  constexpr int KS = D / 16;        // k-steps of 16 channels
  constexpr int PT = 128 * 16;      // bf16 per piece tile (128 rows x 16 channels)
  constexpr int EP = 72;            // floats per row of a wave's 64 x 64 output tile in LDS
  constexpr int STAGE_B = 2 * 2 * 3 * PT * 2, EPI_B = 4 * 64 * EP * 4;
  __shared__ __attribute__((aligned(16))) char smem[STAGE_B > EPI_B ? STAGE_B : EPI_B];
  bf16* stage = reinterpret_cast<bf16*>(smem);   // [buffer][A, B][hi, mid, lo][row][16 channels]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n32 = lane & 31, hf = lane >> 5;
  const Tile3 t = tile3((Nk + 127) / 128, (Nq + 127) / 128);
  const long bh = t.z;
  const int M0 = t.y * 128, N0 = t.x * 128, wm = (w >> 1) * 64, wn = (w & 1) * 64;
  // Staging role: float4 idx = tid + 256j of the k-step's tile, row idx / 4,
  // channels 4 (idx % 4) .. +3.
  const float* Ar[2];
  const float* Br[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 256 * j, row = idx >> 2, q4 = idx & 3;
    Ar[j] = qc + (bh * Nq + min(M0 + row, Nq - 1)) * (long)D + 4 * q4;
    Br[j] = kc + (bh * Nk + min(N0 + row, Nk - 1)) * (long)D + 4 * q4;
  }
  float4 ra[2], rb[2];
  auto load = [&](int ks) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ra[j] = *reinterpret_cast<const float4*>(Ar[j] + 16 * ks);
      rb[j] = *reinterpret_cast<const float4*>(Br[j] + 16 * ks);
    }
  };
  auto put = [&](bf16* piece0, const float4& x, int idx) {
    const float v[4] = {x.x, x.y, x.z, x.w};
    bf16x4 hi, mid, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = (bf16)v[e];
      const float r1 = v[e] - (float)hi[e];
      mid[e] = (bf16)r1;
      lo[e] = (bf16)(r1 - (float)mid[e]);
    }
    const int at = (idx >> 2) * 16 + (idx & 3) * 4;
    *reinterpret_cast<bf16x4*>(piece0 + at) = hi;
    *reinterpret_cast<bf16x4*>(piece0 + PT + at) = mid;
    *reinterpret_cast<bf16x4*>(piece0 + 2 * PT + at) = lo;
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      put(stage + (buf * 2 + 0) * 3 * PT, ra[j], tid + 256 * j);
      put(stage + (buf * 2 + 1) * 3 * PT, rb[j], tid + 256 * j);
    }
  };
  // Fragment of piece p for the lane's row r of operand ab: channels 8hf .. +7.
  auto frag = [&](int buf, int ab, int p, int r) {
    return *reinterpret_cast<const bf16x8*>(stage + ((buf * 2 + ab) * 3 + p) * PT + r * 16 + 8 * hf);
  };
  f32x16 hh[2][2], xx[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) hh[i][j][e] = xx[i][j][e] = 0.f;
  load(0);
  store(0);
  if (KS > 1) load(1);
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int buf = ks & 1;
    bf16x8 ah[2], am[2], al[2], bh8[2], bm[2], bl[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ra_ = wm + 32 * i + n32, rb_ = wn + 32 * i + n32;
      ah[i] = frag(buf, 0, 0, ra_);
      am[i] = frag(buf, 0, 1, ra_);
      al[i] = frag(buf, 0, 2, ra_);
      bh8[i] = frag(buf, 1, 0, rb_);
      bm[i] = frag(buf, 1, 1, rb_);
      bl[i] = frag(buf, 1, 2, rb_);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        xx[i][j] = mfma32_bf16(am[i], bm[j], xx[i][j]);
        xx[i][j] = mfma32_bf16(al[i], bh8[j], xx[i][j]);
        xx[i][j] = mfma32_bf16(ah[i], bl[j], xx[i][j]);
        xx[i][j] = mfma32_bf16(am[i], bh8[j], xx[i][j]);
        xx[i][j] = mfma32_bf16(ah[i], bm[j], xx[i][j]);
        hh[i][j] = mfma32_bf16(ah[i], bh8[j], hh[i][j]);
      }
    if (ks + 1 < KS) {
      // Buffer buf ^ 1 was last read in step ks - 1, which ended with a
      // barrier. Kept after the MFMAs, which cover the latency of its loads.
      __builtin_amdgcn_sched_barrier(0);
      store(buf ^ 1);
      if (ks + 2 < KS) load(ks + 2);
      __syncthreads();
    }
  }
  // hh[i][j][jj] + xx[i][j][jj] = S[row wm + 32i + 8(jj/4) + 4hf + jj%4][col wn + 32j + n32] / scale
  // (within the tile). Through LDS (every wave is past its last staging read),
  // then out as rows of 16-byte units.
  __syncthreads();
  float* et = reinterpret_cast<float*>(smem) + w * 64 * EP;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj)
        et[(32 * i + 8 * (jj >> 2) + 4 * hf + (jj & 3)) * EP + 32 * j + n32] = (hh[i][j][jj] + xx[i][j][jj]) * scale;
  wave_sync();
  float* S = s + bh * (long)Nq * ld;
  const int c4 = 4 * (lane & 15), col = N0 + wn + c4;
#pragma unroll
  for (int st = 0; st < 16; ++st) {
    const int r = 4 * st + (lane >> 4), row = M0 + wm + r;
    const float4 v = *reinterpret_cast<const float4*>(et + r * EP + c4);
    if (row < Nq && col < ld) *reinterpret_cast<float4*>(S + (long)row * ld + col) = v;   // ld % 4 == 0
  }
}

// C[bh][i][:] = scale * sum_j A[i][j] B[j][:] for i < R, j < Kd, with B
// [Kd][D] and A = M (M is R x Kd) or A = M^T with TRANS_A (M is Kd x R);
// M is fp32 with row pitch ld. With EXP A[i][j] = exp(M[i][j] - lse[i]) (the
// coarse softmax applied as the tile is staged). A workgroup owns 32 rows of C and every channel; k goes in chunks
// of 32 through LDS, double buffered: the A tile row-major and the B tile
// transposed (channel-major), so that for 16x16x4 MFMA k-step s a lane of
// lane group g contracts k = 8g + s and reads its eight A values and eight B
// values as two 16-byte LDS reads each. Wave w owns channels
// [16*CB*w, 16*CB*(w+1)) of both 16-row blocks. Both tiles have rows of
// KC = 32 floats with their 16-byte units XOR-permuted by row / 2 (tslot),
// so the 16-lane reads of 16 consecutive rows fall on distinct banks; the B
// tile is staged with k varying fastest across lanes, and the two lane halves
// of a wave store rows of opposite parity (they swap the components of their
// float4 in pairs), which keeps the transposing stores conflict-free too. At
// 40 KB of LDS four workgroups fit a CU.
template <int D, bool TRANS_A, bool EXP>
__global__ __launch_bounds__(256) void coarse_gemm_kernel(const float* __restrict__ m, const float* __restrict__ lse,
                                                          const float* __restrict__ b, float* __restrict__ c, int R,
                                                          int Kd, int ld, float scale) {
  constexpr int KC = 32;                         // k per chunk = floats per LDS tile row
  constexpr int CB = D / 64;                     // 16-channel blocks per wave
  constexpr int BF4 = KC * D / 4 / 256;          // B float4 loads per thread per chunk
  static_assert(!(TRANS_A && EXP), "the softmax is applied along rows of M only");
  static_assert(KC == 32 && BF4 * 8 * 4 == D, "B staging: 32 k per lane half, 8 channel groups per pass");
  __shared__ __attribute__((aligned(16))) float Al[2][32 * KC];
  __shared__ __attribute__((aligned(16))) float Bl[2][D * KC];
  // Float index of element (row, k) of a tile: 16-byte unit k / 4 of the row
  // is stored at unit (k / 4) ^ (row / 2 mod 8).
  auto tslot = [](int row, int k) { return row * KC + ((((k >> 2) ^ (row >> 1)) & 7) << 2) + (k & 3); };
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const Tile3 t = tile3((R + 31) / 32, 1);
  const long bh = t.z;
  const int r0 = t.x * 32;
  const float* M = m + bh * (long)(TRANS_A ? Kd : R) * ld;
  const float* Bm = b + bh * (long)Kd * D;
  // A staging role: without TRANS_A, row ai of the tile, k = 4aq .. 4aq+3
  // (M[r0 + ai][k0 + 4aq ..]); with TRANS_A, k = ai of the chunk and tile rows
  // 4aq .. 4aq+3 (M[k0 + ai][r0 + 4aq ..]), written transposed.
  const int ai = tid >> 3, aq = tid & 7;
  // B staging role in pass j: k row kap of the chunk, channel group bc4 + 8 j
  // (four channels).
  const int kap = lane & 31, bc4 = (w & 1) + 4 * (w >> 1) + 2 * (lane >> 5);
  const bool arow = r0 + ai < R;
  const float alse = (EXP && arow) ? lse[bh * R + r0 + ai] : 0.f;
  float4 ar, br[BF4];
  auto load = [&](int k0) {
    ar = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!TRANS_A) {
      const int kk = k0 + 4 * aq;
      if (arow && kk < Kd) {
        ar = *reinterpret_cast<const float4*>(M + (long)(r0 + ai) * ld + kk);   // ld % 4 == 0
        if (EXP) {
          ar.x = __expf(ar.x - alse);
          ar.y = kk + 1 < Kd ? __expf(ar.y - alse) : 0.f;
          ar.z = kk + 2 < Kd ? __expf(ar.z - alse) : 0.f;
          ar.w = kk + 3 < Kd ? __expf(ar.w - alse) : 0.f;
        } else {
          if (kk + 1 >= Kd) ar.y = 0.f;
          if (kk + 2 >= Kd) ar.z = 0.f;
          if (kk + 3 >= Kd) ar.w = 0.f;
        }
      }
    } else {
      const int kk = k0 + ai, cc = r0 + 4 * aq;
      if (kk < Kd && cc < R) {
        ar = *reinterpret_cast<const float4*>(M + (long)kk * ld + cc);
        if (cc + 1 >= R) ar.y = 0.f;
        if (cc + 2 >= R) ar.z = 0.f;
        if (cc + 3 >= R) ar.w = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < BF4; ++j) {
      const int c4 = bc4 + 8 * j;
      br[j] = k0 + kap < Kd ? *reinterpret_cast<const float4*>(Bm + (long)(k0 + kap) * D + 4 * c4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store = [&](int bb) {
    if (!TRANS_A) {
      *reinterpret_cast<float4*>(&Al[bb][tslot(ai, 4 * aq)]) = ar;
    } else {
      Al[bb][tslot(4 * aq + 0, ai)] = ar.x;
      Al[bb][tslot(4 * aq + 1, ai)] = ar.y;
      Al[bb][tslot(4 * aq + 2, ai)] = ar.z;
      Al[bb][tslot(4 * aq + 3, ai)] = ar.w;
    }
    const int hb = lane >> 5;   // the upper lane half stores component t ^ 1 in step t
#pragma unroll
    for (int j = 0; j < BF4; ++j) {
      const int c4 = bc4 + 8 * j;
      float4 v = br[j];
      if (hb) v = make_float4(v.y, v.x, v.w, v.z);
      Bl[bb][tslot(4 * c4 + (0 ^ hb), kap)] = v.x;
      Bl[bb][tslot(4 * c4 + (1 ^ hb), kap)] = v.y;
      Bl[bb][tslot(4 * c4 + (2 ^ hb), kap)] = v.z;
      Bl[bb][tslot(4 * c4 + (3 ^ hb), kap)] = v.w;
    }
  };
  f32x4 acc[2][CB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nchunk = (Kd + KC - 1) / KC;
  load(0);
  store(0);
  __syncthreads();
  for (int ch = 0; ch < nchunk; ++ch) {
    const int bb = ch & 1;
    if (ch + 1 < nchunk) load((ch + 1) * KC);
    float av[2][8], bv[CB][8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float4 x0 = *reinterpret_cast<const float4*>(&Al[bb][tslot(16 * rb + r, 8 * g)]);
      const float4 x1 = *reinterpret_cast<const float4*>(&Al[bb][tslot(16 * rb + r, 8 * g + 4)]);
      av[rb][0] = x0.x; av[rb][1] = x0.y; av[rb][2] = x0.z; av[rb][3] = x0.w;
      av[rb][4] = x1.x; av[rb][5] = x1.y; av[rb][6] = x1.z; av[rb][7] = x1.w;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = 16 * (CB * w + cb) + r;
      const float4 x0 = *reinterpret_cast<const float4*>(&Bl[bb][tslot(col, 8 * g)]);
      const float4 x1 = *reinterpret_cast<const float4*>(&Bl[bb][tslot(col, 8 * g + 4)]);
      bv[cb][0] = x0.x; bv[cb][1] = x0.y; bv[cb][2] = x0.z; bv[cb][3] = x0.w;
      bv[cb][4] = x1.x; bv[cb][5] = x1.y; bv[cb][6] = x1.z; bv[cb][7] = x1.w;
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = mfma16_f32(av[rb][st], bv[cb][st], acc[rb][cb]);
    if (ch + 1 < nchunk) {
      store(bb ^ 1);   // bb ^ 1 was last read in chunk ch - 1, which ended with a barrier
      __syncthreads();
    }
  }
  float* C = c + bh * (long)R * D;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = 16 * (CB * w + cb) + r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = r0 + 16 * rb + 4 * g + e;
        if (row < R) C[(long)row * D + col] = scale * acc[rb][cb][e];
      }
    }
}

// The largest key x such that at least k of the wave's keys (one per lane,
// `have` lanes taking part; 1 <= k <= 64) are >= x: the k-th largest key, or
// 0 when fewer than k lanes take part. The 64 keys (0 for the lanes that do
// not take part) are sorted in descending order across the lanes by a
// bitonic network of lane exchanges, and lane k - 1 then holds it. (This
// replaced a 32-step search by bit with ballots, which ran on the scalar
// unit that the whole CU shares; same results, coarse stage 0.8% faster.)
// Every lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t key, bool have, int k) {
  const int lane = threadIdx.x & 63;
  uint32_t v = have ? key : 0u;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int j = size >> 1; j > 0; j >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)v, j, 64);
      const bool desc = (lane & size) == 0;   // blocks of `size` lanes alternate direction
      v = (((lane & j) == 0) == desc) ? max(v, o) : min(v, o);
    }
  }
  return __builtin_amdgcn_readlane(v, k - 1);
}

// Top-K of a row for K <= 64 when few values can be in it (key[t] = the
// order-preserving key of value t*64 + lane, 0 beyond Nk). The K-th largest
// of the 64 lane maxima bounds the K-th largest value from below (K lanes
// hold a value at least that large), so only values at or above it are
// candidates. When there are at most 64 they are compacted one per lane in
// ascending block order (cand: 64 slots of this wave's LDS), the K-th
// largest candidate (the K-th largest value of the row) is found, and every
// candidate above it plus the first ones equal to it (smaller ids win ties)
// are written in that order, i.e. ascending. Returns false, having written
// nothing, when there are more than 64 candidates.
template <int NCH>
__device__ __forceinline__ bool row_topk_few(const uint32_t (&key)[NCH], int Nk, int topk, int stride,
                                             uint64_t* cand, int32_t* __restrict__ out,
                                             int32_t* __restrict__ len_out) {
  const int lane = threadIdx.x & 63;
  const int nused = (Nk + 63) >> 6;
  uint32_t lmax = 0u;
#pragma unroll
  for (int t = 0; t < NCH; ++t)
    if (t < nused) lmax = max(lmax, key[t]);
  const uint32_t thr = wave_kth_largest(lmax, true, topk);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int n = 0;
#pragma unroll
  for (int t = 0; t < NCH; ++t) {
    if (t >= nused) break;
    n += __popcll(__ballot(t * 64 + lane < Nk && key[t] >= thr));
  }
  if (n > 64) return false;
  int pos = 0;
#pragma unroll
  for (int t = 0; t < NCH; ++t) {
    if (t >= nused) break;
    const int j = t * 64 + lane;
    const bool c = j < Nk && key[t] >= thr;
    const uint64_t b = __ballot(c);
    // Every lane writes (no branch): a non-candidate into its own slot past
    // the 64 candidate slots.
    cand[c ? pos + __popcll(b & lt_mask) : 64 + lane] = ((uint64_t)key[t] << 32) | (uint32_t)j;
    pos += __popcll(b);
  }
  wave_sync();
  const bool have = lane < n;
  const uint64_t x = have ? cand[lane] : 0ull;
  wave_sync();
  const uint32_t ck = (uint32_t)(x >> 32);
  const uint32_t kth = wave_kth_largest(ck, have, topk);
  const int above = __popcll(__ballot(have && ck > kth));
  const bool eq = have && ck == kth;
  const int eq_rank = __popcll(__ballot(eq) & lt_mask);
  const bool take = (have && ck > kth) || (eq && eq_rank < topk - above);
  const int opos = __popcll(__ballot(take) & lt_mask);
  if (take) out[opos] = (int32_t)(uint32_t)(x & 0xFFFFFFFFu);
  for (int j = topk + lane; j < stride; j += 64) out[j] = -1;
  if (lane == 0) *len_out = topk;
  return true;
}

// One wave per row: LSE_c, and with topk > 0 the ascending top-K list.
// With K <= 64 it first tries row_topk_few (ballots only); otherwise, or when
// more than 64 values are candidates, selection works on the
// order-preserving integer keys of the logits: a
// radix select finds the key of the K-th largest logit, 8 bits per pass from
// the most significant bit in which the row's keys differ (the bits above it
// are shared by every key, and skipping them keeps the first histogram
// spread over many buckets, so the LDS atomics rarely collide). A pass whose
// chosen bucket is taken whole (its count is the number still needed) ends
// the search: the lower bits cannot change the set. Then every key above the
// bucket and the first (K - #above) keys in it, in ascending key-block order,
// are taken (with the search run to the last bit, the bucket is one key
// value).
template <int NCH>
__global__ __launch_bounds__(256) void coarse_rows_kernel(const float* __restrict__ s, float* __restrict__ lse,
                                                          int32_t* __restrict__ idx, int32_t* __restrict__ len,
                                                          long rows, int Nk, int ld, int topk, int stride) {
  __shared__ __attribute__((aligned(16))) int hist_all[4][256];   // per wave: histogram or 64 candidates
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + w;
  if (row >= rows) return;   // wave-uniform; no block barrier below
  const float* srow = s + row * ld;
  const int nused = (Nk + 63) >> 6;   // register slots holding any key block
  float v[NCH];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < NCH; ++t) {
    const int j = t * 64 + lane;
    const float x = srow[min(j, Nk - 1)];   // unconditional (no branch per slot)
    v[t] = j < Nk ? x : -INFINITY;
    mx = fmaxf(mx, v[t]);
  }
  mx = wave_max(mx);
  float sm = 0.f;
#pragma unroll
  for (int t = 0; t < NCH; ++t) {
    if (t >= nused) break;
    sm += __expf(v[t] - mx);   // exp(-inf) = 0 for padding
  }
  sm = wave_sum(sm);
  if (lane == 0) lse[row] = mx + __logf(sm);
  if (topk <= 0) return;

  int* h = hist_all[w];
  uint32_t key[NCH];
  uint32_t kmin = 0xFFFFFFFFu;
#pragma unroll
  for (int t = 0; t < NCH; ++t) {
    const bool valid = t * 64 + lane < Nk;
    key[t] = valid ? fkey(v[t]) : 0u;
    if (valid) kmin = min(kmin, key[t]);
  }
  // Few candidates (the usual case for K <= 64): selected with ballots alone.
  if (topk <= 64 && row_topk_few<NCH>(key, Nk, topk, stride, reinterpret_cast<uint64_t*>(h),
                                      idx + row * (long)stride, len + row))
    return;
  kmin = wave_min_u32(kmin);
  const uint32_t diff = kmin ^ fkey(mx);
  // Keys matching `prefix` on the bits of `pmask` are the candidates.
  uint32_t prefix = kmin, pmask = 0xFFFFFFFFu;
  int krem = topk;
  int hi = diff == 0u ? -1 : 31 - __clz(diff);   // highest free bit
  if (hi >= 0) {
    pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
    prefix = kmin & pmask;
  }
  while (hi >= 0) {
    const int nb = min(8, hi + 1), shift = hi - nb + 1;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int b = lane; b < 256; b += 64) h[b] = 0;
    wave_sync();
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
      if (t >= nused) break;
      if ((t * 64 + lane) < Nk && (key[t] & pmask) == prefix) atomicAdd(&h[(key[t] >> shift) & dmask], 1);
    }
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
    int found = -1, before = 0, fcount = 0;
    const int cnt[4] = {b3, b2, b1, b0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (found < 0 && acc < krem && acc + cnt[q] >= krem) { found = 4 * lane + 3 - q; before = acc; fcount = cnt[q]; }
      acc += cnt[q];
    }
    const uint64_t bal = __ballot(found >= 0);
    const int src = __ffsll((unsigned long long)bal) - 1;
    const int fb = __shfl(found, src, 64);
    const int fbefore = __shfl(before, src, 64);
    const int fcnt = __shfl(fcount, src, 64);
    prefix |= (uint32_t)fb << shift;
    pmask |= dmask << shift;
    krem -= fbefore;
    hi -= nb;
    wave_sync();
    if (fcnt == krem) break;   // the whole bucket is taken
  }
  // prefix (on the bits of pmask) is the bucket of the K-th largest logit:
  // take every key above it and the first krem in it in ascending order.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* out = idx + row * (long)stride;
  int taken = 0, eq_seen = 0;
#pragma unroll
  for (int t = 0; t < NCH; ++t) {
    if (t >= nused) break;
    const int j = t * 64 + lane;
    const bool valid = j < Nk;
    const bool gt = valid && (key[t] & pmask) > prefix;
    const bool eq = valid && (key[t] & pmask) == prefix;
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

// The rows kernel for rows longer than kRowsInRegisters: the same LSE_c and
// selection (candidates with ballots for K <= 64 when at most 64 values can
// be chosen, else the radix select), with the row read again from memory in
// every pass instead of held in registers. The first read forms each lane's
// running maximum and rescaled exponential sum (so LSE_c takes one pass) and
// the lane's largest and smallest keys (the key map preserves order); with
// K <= 64 the second counts and collects the candidates together.
__global__ __launch_bounds__(256) void coarse_rows_stream_kernel(const float* __restrict__ s, float* __restrict__ lse,
                                                                 int32_t* __restrict__ idx, int32_t* __restrict__ len,
                                                                 long rows, int Nk, int ld, int topk, int stride) {
  __shared__ __attribute__((aligned(16))) int hist_all[4][256];   // per wave: histogram or 64 candidates
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + w;
  if (row >= rows) return;   // wave-uniform; no block barrier below
  const float* srow = s + row * ld;
  const int nused = (Nk + 63) >> 6;
  auto key_at = [&](int t) { const int j = t * 64 + lane; return j < Nk ? fkey(srow[j]) : 0u; };
  float ml = -INFINITY, sl = 0.f;   // this lane's running maximum and sum of exp(x - ml)
  float mn = INFINITY;              // and its minimum (the radix select's lowest key)
  for (int j = lane; j < Nk; j += 64) {
    const float x = srow[j];
    mn = fminf(mn, x);
    if (x > ml) {
      sl = sl * __expf(ml - x) + 1.0f;
      ml = x;
    } else {
      sl += __expf(x - ml);
    }
  }
  const float mx = wave_max(ml);
  const float sm = wave_sum(ml == -INFINITY ? 0.f : sl * __expf(ml - mx));
  if (lane == 0) lse[row] = mx + __logf(sm);
  if (topk <= 0) return;
  int* h = hist_all[w];
  int32_t* out = idx + row * (long)stride;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (topk <= 64) {   // candidates (see row_topk_few)
    const uint32_t lmax = ml == -INFINITY ? 0u : fkey(ml);   // lanes without a value hold key 0
    const uint32_t thr = wave_kth_largest(lmax, true, topk);
    uint64_t* cand = reinterpret_cast<uint64_t*>(h);
    int n = 0;   // candidates seen; the first 64 are kept
    for (int t = 0; t < nused; ++t) {
      const int j = t * 64 + lane;
      const uint32_t kj = key_at(t);
      const bool c = j < Nk && kj >= thr;
      const uint64_t b = __ballot(c);
      const int slot = n + __popcll(b & lt_mask);
      if (c && slot < 64) cand[slot] = ((uint64_t)kj << 32) | (uint32_t)j;
      n += __popcll(b);
    }
    if (n <= 64) {
      wave_sync();
      const bool have = lane < n;
      const uint64_t x = have ? cand[lane] : 0ull;
      wave_sync();
      const uint32_t ck = (uint32_t)(x >> 32);
      const uint32_t kth = wave_kth_largest(ck, have, topk);
      const int above = __popcll(__ballot(have && ck > kth));
      const bool eq = have && ck == kth;
      const int eq_rank = __popcll(__ballot(eq) & lt_mask);
      const bool take = (have && ck > kth) || (eq && eq_rank < topk - above);
      const int opos = __popcll(__ballot(take) & lt_mask);
      if (take) out[opos] = (int32_t)(uint32_t)(x & 0xFFFFFFFFu);
      for (int j = topk + lane; j < stride; j += 64) out[j] = -1;
      if (lane == 0) len[row] = topk;
      return;
    }
  }
  // Radix select (see row_topk), keys recomputed in every pass.
  const uint32_t kmin = wave_min_u32(mn == INFINITY ? 0xFFFFFFFFu : fkey(mn));
  const uint32_t diff = kmin ^ fkey(mx);
  uint32_t prefix = kmin, pmask = 0xFFFFFFFFu;
  int krem = topk;
  int hi = diff == 0u ? -1 : 31 - __clz(diff);
  if (hi >= 0) {
    pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
    prefix = kmin & pmask;
  }
  while (hi >= 0) {
    const int nb = min(8, hi + 1), shift = hi - nb + 1;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int b = lane; b < 256; b += 64) h[b] = 0;
    wave_sync();
    for (int t = 0; t < nused; ++t) {
      const uint32_t k = key_at(t);
      if ((t * 64 + lane) < Nk && (k & pmask) == prefix) atomicAdd(&h[(k >> shift) & dmask], 1);
    }
    wave_sync();
    const int b0 = h[4 * lane], b1 = h[4 * lane + 1], b2 = h[4 * lane + 2], b3 = h[4 * lane + 3];
    const int mine = b0 + b1 + b2 + b3;
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_down(incl, o, 64);
      if (lane + o < 64) incl += t;
    }
    int acc = incl - mine;
    int found = -1, before = 0, fcount = 0;
    const int cnt[4] = {b3, b2, b1, b0};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (found < 0 && acc < krem && acc + cnt[q] >= krem) { found = 4 * lane + 3 - q; before = acc; fcount = cnt[q]; }
      acc += cnt[q];
    }
    const uint64_t bal = __ballot(found >= 0);
    const int src = __ffsll((unsigned long long)bal) - 1;
    const int fb = __shfl(found, src, 64);
    const int fbefore = __shfl(before, src, 64);
    const int fcnt = __shfl(fcount, src, 64);
    prefix |= (uint32_t)fb << shift;
    pmask |= dmask << shift;
    krem -= fbefore;
    hi -= nb;
    wave_sync();
    if (fcnt == krem) break;
  }
  int taken = 0, eq_seen = 0;
  for (int t = 0; t < nused; ++t) {
    const int j = t * 64 + lane;
    const uint32_t k = key_at(t);
    const bool valid = j < Nk;
    const bool gt = valid && (k & pmask) > prefix;
    const bool eq = valid && (k & pmask) == prefix;
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

// C = scale * op(M) B with R output rows and Kd contracted; M is the
// Nq x Nk coarse matrix (pitch coarse_ld(Nk)), see coarse_gemm_kernel.
template <bool TRANS_A, bool EXP>
static void launch_gemm(const Launch& L, const float* m, const float* lse, const float* b, float* c, int R, int Kd,
                        float scale) {
  const int ld = coarse_ld(L.gk.Nc);
  const dim3 grid((unsigned)((R + 31) / 32 * L.BH));
  if (L.D == 64)
    hipLaunchKernelGGL((coarse_gemm_kernel<64, TRANS_A, EXP>), grid, dim3(256), 0, L.stream, m, lse, b, c, R, Kd,
                       ld, scale);
  else
    hipLaunchKernelGGL((coarse_gemm_kernel<128, TRANS_A, EXP>), grid, dim3(256), 0, L.stream, m, lse, b, c, R,
                       Kd, ld, scale);
}
// O_c = exp(S - LSE_c) V_c of a bf16 problem, on bf16 MFMAs (32x32x16, fp32
// accumulation) with every fp32 operand split into a bf16 head and a bf16
// tail (hi = bf16(x), lo = bf16(x - hi); bf16 rounding is within 2^-8 of
// the value rounded) and the product formed as P_hi V_hi + P_hi V_lo +
// P_lo V_hi: the dropped P_lo V_lo and the tails' rounding leave each term
// within 3 * 2^-16 of exact, so O_c keeps near-fp32 accuracy at matrix-core
// rate (three
// bf16 products take less matrix time than one fp32 product, and less than
// the read of S at HBM rate). A workgroup of four waves owns
// 128 rows of O_c, wave w the rows 32w .. 32w+31 (one per lane column) in the
// transposed form O_c^T += V_chunk^T P^T over chunks of 32 key blocks. The
// chunk's V_c rows (fp32, split) form two bf16 row tiles in LDS, double
// buffered with one barrier per chunk, whose transposed A fragments come from
// LDS transpose reads; each lane forms its row's P^T fragments from S
// directly, in the key order those reads deliver (for k-step s2, slot e is
// key 16 s2 + 8(e/4) + 4hf + e%4: two float4 loads). S loads run two chunks
// ahead, V_c one.
// The same kernel without EXP forms C = scale * M B for any fp32 M (the
// coarse backward's dQ_c = s dS K_c): M takes the place of P, B of V_c.
template <int D, bool EXP>
__global__ __launch_bounds__(256, 2) void coarse_pv_bf16_kernel(const float* __restrict__ s,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ vc, float* __restrict__ oc,
                                                               int Nq, int Nk, int ld, float scale) {
  using G = ChunkGeom<D>;
  constexpr int MB = G::MB, U = G::U;
  constexpr int UPT = 32 * U / 256;   // 16-byte units of a V tile staged per thread
  __shared__ __attribute__((aligned(16))) bf16 vt[2][2][32 * D];   // [buffer][hi, lo]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n32 = lane & 31, hf = lane >> 5;
  const Tile3 t = tile3((Nq + 127) / 128, 1);
  const long bh = t.z;
  const int row = t.x * 128 + 32 * w + n32;
  const bool rvalid = row < Nq;
  const float* V = vc + bh * (long)Nk * D;
  const int nch = (Nk + 31) / 32;

  // Every load below is unconditional (addresses clamped into the arrays):
  // the compiler can then count them and waits only for the oldest (its waits
  // for loads under a branch drain every load in flight, the S loads issued
  // two chunks ahead included). Clamped rows and keys are masked or meet P = 0.
  const int kmax = (Nk - 1) & ~3;   // last float4 of a row of S that starts below Nk
  const float* srow = s + (bh * Nq + min(row, Nq - 1)) * (long)ld;
  const float l2 = EXP ? lse[bh * Nq + min(row, Nq - 1)] * kLog2e : 0.f;
  // S of chunk c for this lane: [s2][half] = keys 32c + 16 s2 + 8 half + 4hf .. +3.
  auto load_s = [&](float4 (&x)[2][2], int c) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        x[s2][h] = *reinterpret_cast<const float4*>(srow + min(32 * c + 16 * s2 + 8 * h + 4 * hf, kmax));
  };
  // P^T fragments (head and tail) of chunk c from its S values; keys beyond
  // Nk (only in the last chunk) give 0.
  auto make_p = [&](const float4 (&x)[2][2], int c, bf16x8 (&ph)[2], bf16x8 (&pl)[2]) {
    const bool full = 32 * c + 32 <= Nk;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = 32 * c + 16 * s2 + 8 * h + 4 * hf;
        const float v[4] = {x[s2][h].x, x[s2][h].y, x[s2][h].z, x[s2][h].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv = EXP ? __builtin_amdgcn_exp2f(fmaf(v[e], kLog2e, -l2)) : v[e];
          if (!full && kk + e >= Nk) pv = 0.f;
          const bf16 hi = (bf16)pv;
          ph[s2][4 * h + e] = hi;
          pl[s2][4 * h + e] = (bf16)(pv - (float)hi);
        }
      }
  };
  // V_c rows of chunk c, unit p = j*256 + tid of a tile: row kappa = p / U,
  // channels 8(p % U) .. +7; rows beyond Nk repeat the last one (their P is 0).
  float4 vr[UPT][2];
  auto load_v = [&](int c) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int p = j * 256 + tid, kappa = p / U, u = p % U, key = min(32 * c + kappa, Nk - 1);
      const float4* src = reinterpret_cast<const float4*>(V + (long)key * D + 8 * u);
      vr[j][0] = src[0];
      vr[j][1] = src[1];
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int p = j * 256 + tid, kappa = p / U, u = p % U;
      const float x[8] = {vr[j][0].x, vr[j][0].y, vr[j][0].z, vr[j][0].w,
                          vr[j][1].x, vr[j][1].y, vr[j][1].z, vr[j][1].w};
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = (bf16)x[e];
        lo[e] = (bf16)(x[e] - (float)hi[e]);
      }
      const int at = (kappa * U + (u ^ kswz<U>(kappa))) * 8;
      *reinterpret_cast<bf16x8*>(&vt[buf][0][at]) = hi;
      *reinterpret_cast<bf16x8*>(&vt[buf][1][at]) = lo;
    }
  };
  uint32_t voffs[MB][2][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) rowt_offsets<D>(lane, mb, s2, voffs[mb][s2]);

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0.f;
  float4 sa[2][2], sb[2][2];
  load_s(sa, 0);
  load_s(sb, min(1, nch - 1));
  load_v(0);
  store_v(0);
  load_v(min(1, nch - 1));
  __syncthreads();
  // Chunk c: P from its S (loaded two chunks ago), the next-but-one chunk's S
  // into the same registers, the MFMAs on tiles c % 2, then tiles (c+1) % 2
  // (last read in chunk c - 1, which ended with a barrier) receive chunk
  // c + 1 and the loads of chunk c + 2's V_c go out (chunk indices past the
  // end are clamped: those loads are never used).
  auto step = [&](auto B, float4 (&x)[2][2], int c) {
    constexpr int buf = decltype(B)::value;
    bf16x8 ph[2], pl[2];
    make_p(x, c, ph, pl);
    load_s(x, min(c + 2, nch - 1));
    const char* th = reinterpret_cast<const char*>(vt[buf][0]);
    const char* tl = reinterpret_cast<const char*>(vt[buf][1]);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 ah = rowt_frag(th, voffs[mb][s2][0], voffs[mb][s2][1]);
        const bf16x8 al = rowt_frag(tl, voffs[mb][s2][0], voffs[mb][s2][1]);
        acc[mb] = mfma32_bf16(al, ph[s2], acc[mb]);
        acc[mb] = mfma32_bf16(ah, pl[s2], acc[mb]);
        acc[mb] = mfma32_bf16(ah, ph[s2], acc[mb]);
      }
    store_v(buf ^ 1);
    load_v(min(c + 2, nch - 1));
    __syncthreads();
  };
  // An even number of steps, none of them under a branch (so the compiler
  // keeps every load where it is issued): with an odd chunk count the last
  // step is chunk nch, all of whose keys lie beyond Nk (P = 0).
  for (int c = 0; c < nch; c += 2) {
    step(std::integral_constant<int, 0>{}, sa, c);
    step(std::integral_constant<int, 1>{}, sb, c + 1);
  }
  if (!rvalid) return;
  // acc[mb][jj] = O_c^T[channel 32mb + 8(jj/4) + 4hf + jj%4][row]: four
  // consecutive channels per float4.
  float* orow = oc + (bh * Nq + row) * (long)D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(orow + 32 * mb + 8 * q + 4 * hf) =
          make_float4(acc[mb][4 * q] * scale, acc[mb][4 * q + 1] * scale, acc[mb][4 * q + 2] * scale,
                      acc[mb][4 * q + 3] * scale);
}

int coarse_ld(int Nk) { return (Nk + 3) & ~3; }

// One wave per query cube; each row has Nk key-block logits.
template <int NCH>
static void launch_rows(const Launch& L, const float* s, float* lse, int32_t* idx, int32_t* len) {
  const long rows = (long)L.BH * L.g.Nc;
  hipLaunchKernelGGL((coarse_rows_kernel<NCH>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, L.stream, s, lse,
                     idx, len, rows, L.gk.Nc, coarse_ld(L.gk.Nc), L.topk, L.stride);
}

hipError_t launch_coarse(const Launch& L, const float* qc, const float* kc, const float* vc, float* oc,
                         float* lse, int32_t* idx, int32_t* len, float* s_scratch) {
  const int Nq = L.g.Nc, Nk = L.gk.Nc, ld = coarse_ld(Nk);
  const dim3 tiles((unsigned)((Nk + 127) / 128 * ((Nq + 127) / 128) * L.BH)), block(256);
  if (L.bf16 && L.D == 64)
    hipLaunchKernelGGL((coarse_scores_split_kernel<64>), tiles, block, 0, L.stream, qc, kc, s_scratch, Nq, Nk, ld,
                       L.scale);
  else if (L.bf16)
    hipLaunchKernelGGL((coarse_scores_split_kernel<128>), tiles, block, 0, L.stream, qc, kc, s_scratch, Nq, Nk, ld,
                       L.scale);
  else if (L.D == 64)
    hipLaunchKernelGGL((coarse_scores_kernel<64>), tiles, block, 0, L.stream, qc, kc, s_scratch, Nq, Nk, ld,
                       L.scale);
  else
    hipLaunchKernelGGL((coarse_scores_kernel<128>), tiles, block, 0, L.stream, qc, kc, s_scratch, Nq, Nk, ld,
                       L.scale);
  if (Nk <= 256) launch_rows<4>(L, s_scratch, lse, idx, len);
  else if (Nk <= 512) launch_rows<8>(L, s_scratch, lse, idx, len);
  else if (Nk <= 1024) launch_rows<16>(L, s_scratch, lse, idx, len);
  else if (Nk <= kRowsInRegisters) launch_rows<32>(L, s_scratch, lse, idx, len);
  else {
    const long rows = (long)L.BH * L.g.Nc;
    hipLaunchKernelGGL(coarse_rows_stream_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, L.stream, s_scratch,
                       lse, idx, len, rows, Nk, ld, L.topk, L.stride);
  }
  if (L.bf16) {
    const dim3 grid((unsigned)((Nq + 127) / 128 * L.BH));
    if (L.D == 64)
      hipLaunchKernelGGL((coarse_pv_bf16_kernel<64, true>), grid, block, 0, L.stream, s_scratch, lse, vc, oc, Nq,
                         Nk, ld, 1.0f);
    else
      hipLaunchKernelGGL((coarse_pv_bf16_kernel<128, true>), grid, block, 0, L.stream, s_scratch, lse, vc, oc, Nq,
                         Nk, ld, 1.0f);
  } else {
    launch_gemm<false, true>(L, s_scratch, lse, vc, oc, Nq, Nk, 1.0f);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ backward
// Calculus of the coarse softmax attention (the top-K selection carries no
// gradient): with P = exp(s * Q_c K_c^T - LSE_c) recomputed,
//   dP = dO_c V_c^T, D_i = dO_c[i] . O_c[i], dS = P * (dP - D),
//   dQ_c = s dS K_c, dK_c = s dS^T Q_c, dV_c = P^T dO_c.

// D_i = dO_c[i] . O_c[i]; one wave per row.
template <int D>
__global__ __launch_bounds__(256) void coarse_bwd_delta_kernel(const float* __restrict__ doc,
                                                               const float* __restrict__ oc, float* __restrict__ dc,
                                                               long rows) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float a = 0.f;
#pragma unroll
  for (int d = lane; d < D; d += 64) a += doc[row * D + d] * oc[row * D + d];
  a = wave_sum(a);
  if (lane == 0) dc[row] = a;
}

// P and dS tiles (128x128 per workgroup, 64x64 per wave): the scores GEMM and
// dP = dO_c V_c^T on the same block, then the softmax and its derivative,
// elementwise.
template <int D>
__global__ __launch_bounds__(256, 2) void coarse_bwd_pds_kernel(const float* __restrict__ qc, const float* __restrict__ kc,
                                                             const float* __restrict__ vc, const float* __restrict__ doc,
                                                             const float* __restrict__ lse, const float* __restrict__ dc,
                                                             float* __restrict__ pbuf, float* __restrict__ dsbuf,
                                                             int Nq, int Nk, int ld, float scale) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const Tile3 t = tile3((Nk + 127) / 128, (Nq + 127) / 128);
  const long bh = t.z;
  const int m0 = t.y * 128 + (w >> 1) * 64, n0 = t.x * 128 + (w & 1) * 64;
  if (m0 >= Nq || n0 >= Nk) return;   // wave-uniform; no barrier in this kernel
  const long qbase = bh * (long)Nq * D, kbase = bh * (long)Nk * D;
  f32x4 sacc[4][4], pacc[4][4];
  nt_block64<D>(qc + qbase, kc + kbase, Nq, Nk, m0, n0, sacc);
  // The second product's loads start after the first product's MFMAs, so
  // only one set of operand buffers is live (two waves per SIMD).
  __builtin_amdgcn_sched_barrier(0);
  nt_block64<D, 1>(doc + qbase, vc + kbase, Nq, Nk, m0, n0, pacc);
  float* P = pbuf + bh * (long)Nq * ld;
  float* DS = dsbuf + bh * (long)Nq * ld;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + 16 * i + 4 * g + e;
      if (row >= Nq) continue;
      const float l = lse[bh * Nq + row], dd = dc[bh * Nq + row];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + 16 * j + r;
        if (col >= Nk) continue;
        const float pv = __expf(sacc[i][j][e] * scale - l);
        P[(long)row * ld + col] = pv;
        DS[(long)row * ld + col] = pv * (pacc[i][j][e] - dd);
      }
    }
}

// P and dS of a bf16 problem: S = s Q_c K_c^T and dP = dO_c V_c^T each from
// the exact three-piece split of their fp32 operands (six piece products in
// two accumulators, as the forward's logits: fp32-level accuracy), then
// P = exp(S - LSE_c) and dS = P (dP - delta) elementwise. A workgroup of four
// waves owns a 128 x 64 tile, wave w the rows 32w .. 32w+31 as two 32 x 32
// MFMA tiles. As in the scores kernel, each k-step's operand rows are loaded
// once per workgroup (coalesced), split once and staged in LDS (double
// buffered), and P and dS leave through LDS as 16-byte row units.
template <int D>
__global__ __launch_bounds__(256, 2) void coarse_bwd_pds_split_kernel(
    const float* __restrict__ qc, const float* __restrict__ kc, const float* __restrict__ vc,
    const float* __restrict__ doc, const float* __restrict__ lse, const float* __restrict__ dc,
    float* __restrict__ pbuf, float* __restrict__ dsbuf, int Nq, int Nk, int ld, float scale) {
  constexpr int KS = D / 16;
  constexpr int PA = 128 * 16, PB = 64 * 16;          // bf16 per piece tile of X (128 rows), Y (64 rows)
  constexpr int BUF = 3 * (PA + PB);                  // bf16 per staging buffer
  constexpr int EP = 72;                              // floats per row of a wave's 32 x 64 output tile
  constexpr int STAGE_B = 2 * BUF * 2, EPI_B = 4 * 32 * EP * 4;
  __shared__ __attribute__((aligned(16))) char smem[STAGE_B > EPI_B ? STAGE_B : EPI_B];
  bf16* stage = reinterpret_cast<bf16*>(smem);   // [buffer][X hi, mid, lo][Y hi, mid, lo]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n32 = lane & 31, hf = lane >> 5;
  const Tile3 t = tile3((Nk + 63) / 64, (Nq + 127) / 128);
  const long bh = t.z;
  const int M0 = t.y * 128, N0 = t.x * 64;
  // LSE and delta of this lane's rows M0 + 32w + 8q + 4hf + 0..3 (rows past
  // Nq clamped), loaded first so that their latency hides behind the products.
  float lq[4][4], dq[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const long r = bh * Nq + min(M0 + 32 * w + 8 * q + 4 * hf + e, Nq - 1);
      lq[q][e] = lse[r];
      dq[q][e] = dc[r];
    }
  auto put = [&](bf16* piece0, int pt, const float4& x, int idx) {
    const float v[4] = {x.x, x.y, x.z, x.w};
    bf16x4 hi, mid, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hi[e] = (bf16)v[e];
      const float r1 = v[e] - (float)hi[e];
      mid[e] = (bf16)r1;
      lo[e] = (bf16)(r1 - (float)mid[e]);
    }
    const int at = (idx >> 2) * 16 + (idx & 3) * 4;
    *reinterpret_cast<bf16x4*>(piece0 + at) = hi;
    *reinterpret_cast<bf16x4*>(piece0 + pt + at) = mid;
    *reinterpret_cast<bf16x4*>(piece0 + 2 * pt + at) = lo;
  };
  // out[j] = X Y^T on the wave's rows of X and rows N0 + 32j .. +31 of Y.
  auto nt_split = [&](const float* X, const float* Y, f32x16 (&out)[2]) {
    // Staging role: X float4s tid, tid + 256 (row idx / 4 of 128), Y float4 tid (row idx / 4 of 64).
    const float* Xr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      Xr[j] = X + (bh * Nq + min(M0 + ((tid + 256 * j) >> 2), Nq - 1)) * (long)D + 4 * (tid & 3);
    const float* Yr = Y + (bh * Nk + min(N0 + (tid >> 2), Nk - 1)) * (long)D + 4 * (tid & 3);
    float4 rx[2], ry;
    auto load = [&](int ks) {
      rx[0] = *reinterpret_cast<const float4*>(Xr[0] + 16 * ks);
      rx[1] = *reinterpret_cast<const float4*>(Xr[1] + 16 * ks);
      ry = *reinterpret_cast<const float4*>(Yr + 16 * ks);
    };
    auto store = [&](int buf) {
      bf16* b0 = stage + buf * BUF;
      put(b0, PA, rx[0], tid);
      put(b0, PA, rx[1], tid + 256);
      put(b0 + 3 * PA, PB, ry, tid);
    };
    auto fx = [&](int buf, int p, int r) {
      return *reinterpret_cast<const bf16x8*>(stage + buf * BUF + p * PA + r * 16 + 8 * hf);
    };
    auto fy = [&](int buf, int p, int r) {
      return *reinterpret_cast<const bf16x8*>(stage + buf * BUF + 3 * PA + p * PB + r * 16 + 8 * hf);
    };
    f32x16 hh[2], xx[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) hh[j][e] = xx[j][e] = 0.f;
    load(0);
    store(0);
    if (KS > 1) load(1);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int buf = ks & 1;
      const int rx_ = 32 * w + n32;
      const bf16x8 ah = fx(buf, 0, rx_), am = fx(buf, 1, rx_), al = fx(buf, 2, rx_);
      bf16x8 bh8[2], bm[2], bl[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bh8[j] = fy(buf, 0, 32 * j + n32);
        bm[j] = fy(buf, 1, 32 * j + n32);
        bl[j] = fy(buf, 2, 32 * j + n32);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        xx[j] = mfma32_bf16(am, bm[j], xx[j]);
        xx[j] = mfma32_bf16(al, bh8[j], xx[j]);
        xx[j] = mfma32_bf16(ah, bl[j], xx[j]);
        xx[j] = mfma32_bf16(am, bh8[j], xx[j]);
        xx[j] = mfma32_bf16(ah, bm[j], xx[j]);
        hh[j] = mfma32_bf16(ah, bh8[j], hh[j]);
      }
      if (ks + 1 < KS) {
        __builtin_amdgcn_sched_barrier(0);   // the store's loads were issued a step ago
        store(buf ^ 1);
        if (ks + 2 < KS) load(ks + 2);
      }
      __syncthreads();   // also frees the buffers for the next product or the epilogue
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) out[j] = hh[j] + xx[j];
  };
  f32x16 sv[2], dp[2];
  nt_split(qc, kc, sv);
  nt_split(doc, vc, dp);
  // sv[j][jj], dp[j][jj]: row 32w + 8(jj/4) + 4hf + jj%4, column 32j + n32 of the tile.
  // P, then dS, through the wave's LDS tile and out as 16-byte row units.
  float* et = reinterpret_cast<float*>(smem) + w * 32 * EP;
  const int c4 = 4 * (lane & 15), col = N0 + c4;
  auto emit = [&](float* dst) {
    wave_sync();
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int r = 4 * st + (lane >> 4), row = M0 + 32 * w + r;
      const float4 v = *reinterpret_cast<const float4*>(et + r * EP + c4);
      if (row < Nq && col < ld) *reinterpret_cast<float4*>(dst + (long)row * ld + col) = v;   // ld % 4 == 0
    }
    wave_sync();
  };
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const float pv = __expf(sv[j][jj] * scale - lq[jj >> 2][jj & 3]);
      sv[j][jj] = pv;
      et[(8 * (jj >> 2) + 4 * hf + (jj & 3)) * EP + 32 * j + n32] = pv;
    }
  emit(pbuf + bh * (long)Nq * ld);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      et[(8 * (jj >> 2) + 4 * hf + (jj & 3)) * EP + 32 * j + n32] = sv[j][jj] * (dp[j][jj] - dq[jj >> 2][jj & 3]);
  emit(dsbuf + bh * (long)Nq * ld);
}

// C = scale * M^T B of a bf16 problem (the coarse backward's dK_c = s dS^T Q_c
// and dV_c = P^T dO_c): M is Kd x R with row pitch ld, B is Kd x D, C is
// R x D, all fp32. The products run on bf16 MFMAs with the head / tail split
// of M and B (three products, each term within 3 * 2^-16 of exact). A
// workgroup of four waves owns 128 rows of C, wave w the rows 32w .. 32w+31,
// in the transposed form C^T (D x 32) += B_chunk^T M_chunk over chunks of 32
// k: the chunk's rows of M (the workgroup's 128 columns) and of B (D columns)
// are split into bf16 row tiles in LDS, double buffered with one barrier per
// chunk, and both operands come from them by LDS transpose reads (rows = k;
// both take the same order of k). Loads are unconditional: rows past Kd are
// clamped and their M values zeroed, columns past the row clamped (they only
// reach rows of C that are not stored).
template <int D>
__global__ __launch_bounds__(256, 2) void coarse_tn_bf16_kernel(const float* __restrict__ m,
                                                               const float* __restrict__ b, float* __restrict__ c,
                                                               int R, int Kd, int ld, float scale) {
  using G = ChunkGeom<D>;
  constexpr int MB = G::MB, U = G::U, UM = 16;   // M tiles: 128 columns
  constexpr int UPTB = 32 * U / 256, UPTM = 32 * UM / 256;
  __shared__ __attribute__((aligned(16))) bf16 mt[2][2][32 * 128];   // [buffer][hi, lo]
  __shared__ __attribute__((aligned(16))) bf16 bt[2][2][32 * D];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n32 = lane & 31, hf = lane >> 5;
  const Tile3 t = tile3((R + 127) / 128, 1);
  const long bh = t.z;
  const int r0 = t.x * 128;
  const float* Mh = m + bh * (long)Kd * ld;
  const float* Bh = b + bh * (long)Kd * D;
  const int nch = (Kd + 31) / 32;
  float4 vm[UPTM][2], vb[UPTB][2];
  auto load = [&](int ch) {
#pragma unroll
    for (int j = 0; j < UPTM; ++j) {
      const int p = j * 256 + tid, kappa = p / UM, u = p % UM, k = 32 * ch + kappa;
      const float* src = Mh + (long)min(k, Kd - 1) * ld;
      const int x0 = min(r0 + 8 * u, ld - 4), x1 = min(r0 + 8 * u + 4, ld - 4);
      const float4 a0 = *reinterpret_cast<const float4*>(src + x0);
      const float4 a1 = *reinterpret_cast<const float4*>(src + x1);
      const bool in = k < Kd;
      vm[j][0] = in ? a0 : make_float4(0.f, 0.f, 0.f, 0.f);
      vm[j][1] = in ? a1 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < UPTB; ++j) {
      const int p = j * 256 + tid, kappa = p / U, u = p % U;
      const float4* src = reinterpret_cast<const float4*>(Bh + (long)min(32 * ch + kappa, Kd - 1) * D + 8 * u);
      vb[j][0] = src[0];
      vb[j][1] = src[1];
    }
  };
  auto split2 = [](const float4 (&x)[2], bf16x8& hi, bf16x8& lo) {
    const float v[8] = {x[0].x, x[0].y, x[0].z, x[0].w, x[1].x, x[1].y, x[1].z, x[1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = (bf16)v[e];
      lo[e] = (bf16)(v[e] - (float)hi[e]);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < UPTM; ++j) {
      const int p = j * 256 + tid, kappa = p / UM, u = p % UM;
      bf16x8 hi, lo;
      split2(vm[j], hi, lo);
      const int at = (kappa * UM + (u ^ kswz<UM>(kappa))) * 8;
      *reinterpret_cast<bf16x8*>(&mt[buf][0][at]) = hi;
      *reinterpret_cast<bf16x8*>(&mt[buf][1][at]) = lo;
    }
#pragma unroll
    for (int j = 0; j < UPTB; ++j) {
      const int p = j * 256 + tid, kappa = p / U, u = p % U;
      bf16x8 hi, lo;
      split2(vb[j], hi, lo);
      const int at = (kappa * U + (u ^ kswz<U>(kappa))) * 8;
      *reinterpret_cast<bf16x8*>(&bt[buf][0][at]) = hi;
      *reinterpret_cast<bf16x8*>(&bt[buf][1][at]) = lo;
    }
  };
  uint32_t boffs[MB][2][2], moffs[2][2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    rowt_offsets<128>(lane, w, s2, moffs[s2]);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) rowt_offsets<D>(lane, mb, s2, boffs[mb][s2]);
  }
  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0.f;
  load(0);
  store(0);
  load(1);
  __syncthreads();
  // Chunk ch: the MFMAs on tiles ch % 2, then tiles (ch+1) % 2 (last read in
  // chunk ch - 1, which ended with a barrier) receive chunk ch + 1 and the
  // loads of chunk ch + 2 go out. An even number of steps, none under a
  // branch; chunks past the last one load zeroed rows of M (so a step past
  // the last chunk adds nothing).
  auto step = [&](auto BUF, int ch) {
    constexpr int buf = decltype(BUF)::value;
    const char* mh = reinterpret_cast<const char*>(mt[buf][0]);
    const char* ml = reinterpret_cast<const char*>(mt[buf][1]);
    const char* th = reinterpret_cast<const char*>(bt[buf][0]);
    const char* tl = reinterpret_cast<const char*>(bt[buf][1]);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 fmh = rowt_frag(mh, moffs[s2][0], moffs[s2][1]);
      const bf16x8 fml = rowt_frag(ml, moffs[s2][0], moffs[s2][1]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 fbh = rowt_frag(th, boffs[mb][s2][0], boffs[mb][s2][1]);
        const bf16x8 fbl = rowt_frag(tl, boffs[mb][s2][0], boffs[mb][s2][1]);
        acc[mb] = mfma32_bf16(fbl, fmh, acc[mb]);
        acc[mb] = mfma32_bf16(fbh, fml, acc[mb]);
        acc[mb] = mfma32_bf16(fbh, fmh, acc[mb]);
      }
    }
    // The stores wait for loads issued at the end of the previous step: keep
    // them after this step's MFMAs so that those cover the load latency.
    __builtin_amdgcn_sched_barrier(0);
    store(buf ^ 1);
    load(ch + 2);
    __syncthreads();
  };
  for (int ch = 0; ch < nch; ch += 2) {
    step(std::integral_constant<int, 0>{}, ch);
    step(std::integral_constant<int, 1>{}, ch + 1);
  }
  const int row = r0 + 32 * w + n32;
  if (row >= R) return;
  // acc[mb][jj] = C^T[channel 32mb + 8(jj/4) + 4hf + jj%4][row].
  float* crow = c + (bh * R + row) * (long)D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(crow + 32 * mb + 8 * q + 4 * hf) =
          make_float4(acc[mb][4 * q] * scale, acc[mb][4 * q + 1] * scale, acc[mb][4 * q + 2] * scale,
                      acc[mb][4 * q + 3] * scale);
}

hipError_t launch_coarse_bwd(const Launch& L, const float* qc, const float* kc, const float* vc,
                             const float* oc, const float* lse, const float* doc, float* dqc, float* dkc,
                             float* dvc, float* ds_scratch, float* p_scratch, float* dc_scratch) {
  const int Nq = L.g.Nc, Nk = L.gk.Nc, ld = coarse_ld(Nk);
  const long rows = (long)L.BH * Nq;
  const dim3 tiles((unsigned)((Nk + 127) / 128 * ((Nq + 127) / 128) * L.BH));
  const dim3 tiles64((unsigned)((Nk + 63) / 64 * ((Nq + 127) / 128) * L.BH));
  if (L.D == 64) {
    hipLaunchKernelGGL((coarse_bwd_delta_kernel<64>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, L.stream, doc,
                       oc, dc_scratch, rows);
    if (L.bf16)
      hipLaunchKernelGGL((coarse_bwd_pds_split_kernel<64>), tiles64, dim3(256), 0, L.stream, qc, kc, vc, doc, lse,
                         dc_scratch, p_scratch, ds_scratch, Nq, Nk, ld, L.scale);
    else
      hipLaunchKernelGGL((coarse_bwd_pds_kernel<64>), tiles, dim3(256), 0, L.stream, qc, kc, vc, doc, lse,
                         dc_scratch, p_scratch, ds_scratch, Nq, Nk, ld, L.scale);
  } else {
    hipLaunchKernelGGL((coarse_bwd_delta_kernel<128>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, L.stream,
                       doc, oc, dc_scratch, rows);
    if (L.bf16)
      hipLaunchKernelGGL((coarse_bwd_pds_split_kernel<128>), tiles64, dim3(256), 0, L.stream, qc, kc, vc, doc, lse,
                         dc_scratch, p_scratch, ds_scratch, Nq, Nk, ld, L.scale);
    else
      hipLaunchKernelGGL((coarse_bwd_pds_kernel<128>), tiles, dim3(256), 0, L.stream, qc, kc, vc, doc, lse,
                         dc_scratch, p_scratch, ds_scratch, Nq, Nk, ld, L.scale);
  }
  if (L.bf16) {
    const dim3 block(256), gq((unsigned)((Nq + 127) / 128 * L.BH)), gk((unsigned)((Nk + 127) / 128 * L.BH));
    if (L.D == 64) {
      hipLaunchKernelGGL((coarse_pv_bf16_kernel<64, false>), gq, block, 0, L.stream, ds_scratch, nullptr, kc, dqc,
                         Nq, Nk, ld, L.scale);
      hipLaunchKernelGGL((coarse_tn_bf16_kernel<64>), gk, block, 0, L.stream, ds_scratch, qc, dkc, Nk, Nq, ld, L.scale);
      hipLaunchKernelGGL((coarse_tn_bf16_kernel<64>), gk, block, 0, L.stream, p_scratch, doc, dvc, Nk, Nq, ld, 1.0f);
    } else {
      hipLaunchKernelGGL((coarse_pv_bf16_kernel<128, false>), gq, block, 0, L.stream, ds_scratch, nullptr, kc, dqc,
                         Nq, Nk, ld, L.scale);
      hipLaunchKernelGGL((coarse_tn_bf16_kernel<128>), gk, block, 0, L.stream, ds_scratch, qc, dkc, Nk, Nq, ld,
                         L.scale);
      hipLaunchKernelGGL((coarse_tn_bf16_kernel<128>), gk, block, 0, L.stream, p_scratch, doc, dvc, Nk, Nq, ld, 1.0f);
    }
    return hipGetLastError();
  }
  launch_gemm<false, false>(L, ds_scratch, nullptr, kc, dqc, Nq, Nk, L.scale);   // dQ_c = s dS K_c
  launch_gemm<true, false>(L, ds_scratch, nullptr, qc, dkc, Nk, Nq, L.scale);    // dK_c = s dS^T Q_c
  launch_gemm<true, false>(L, p_scratch, nullptr, doc, dvc, Nk, Nq, 1.0f);       // dV_c = P^T dO_c
  return hipGetLastError();
}

}  // namespace vsa
