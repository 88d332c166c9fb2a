// Backward of step 4 (fine block-sparse attention) and of the pooling.
//
// The pages state that VSA trains end to end through one differentiable
// kernel (VSA summary page, paperlayer.ai arXiv 2505.13389, abstract and
// section 2); the top-K mask is piecewise constant and held fixed. The
// formulas are the calculus of softmax attention: with P = exp(s*q.k - LSE),
//   dV = P^T dO, dP = dO V^T, dS = P * (dP - delta), delta = rowsum(dO * O),
//   dQ = s * dS K, dK = s * dS^T Q,
// and the mean-pool spreads dX_c[c] / Bt over the cube's Bt tokens (the
// max-pool variant sends it to the cube's maximum), added here. Key blocks
// may have their own shape (Bk tokens); everything below that says "key
// cube" means a key block then.
//
// A dQ kernel and dK / dV kernels, all deterministic (no atomics), in the
// style of the forward: a workgroup owns one cube (NW = Bt/32 or Bk/32 waves,
// wave w its tokens 32w .. 32w+31, one per lane column of 32x32x16 bf16
// MFMAs; at 128 channels the dK / dV workgroup has a dV wave and a dK wave
// per 32 keys, and 16-token key blocks go two to a workgroup) and walks a
// list of partner cubes in 32-token chunks: row tiles of the partner's
// tensors staged in LDS by direct-to-LDS loads (each wave issues its share;
// later chunks load while this one is computed). The transposed operands
// come from the same row tiles through LDS transpose reads.
//  * dQ, per query cube i over its list of key cubes (the forward's list):
//      S^T = K_c Q^T, dP^T = V_c dO^T        A = K / V row tiles, B = the
//                                            lane's Q / dO row (registers)
//      dS^T = P^T * (dP^T - delta)            LSE and delta are lane scalars
//      dQ^T += K_c^T dS^T                     A = K row tile read transposed, B = dS^T
//  * dK and dV, per key cube j over the query cubes whose lists hold j (the
//    transposed lists), longest list first:
//      S = Q_c K^T, dP = dO_c V^T            A = Q / dO row tiles, B = the
//                                            lane's K / V row (registers)
//      dS = P * (dP - delta)                 LSE and delta per row (query)
//      dV^T += dO_c^T P, dK^T += Q_c^T dS     A = dO / Q row tiles read transposed
#include <type_traits>

#include "fine_common.h"
#include "vsa_kernels.h"

namespace vsa {

// Processing order of the Nc key blocks of every (b, h) for the dK / dV
// kernel: descending length of their transposed lists, ties by block id, so
// the longest walks start first. One workgroup per (b, h): a bitonic sort of
// ((Nq - count) << 32 | block) keys in LDS (a count never exceeds the Nq
// query cubes, so the clamp at 0 only orders malformed offsets).
__global__ __launch_bounds__(1024) void order_by_count_kernel(const int32_t* __restrict__ k2q_off,
                                                              int32_t* __restrict__ order, int Nc, int Nq,
                                                              int pow2) {
  __shared__ unsigned long long key[kMaxSortKeys];
  const long bh = blockIdx.x;
  const int32_t* off = k2q_off + bh * (Nc + 1);
  for (int e = threadIdx.x; e < pow2; e += 1024) {
    unsigned long long kv = ~0ull;
    if (e < Nc) {
      const int cnt = max(off[e + 1] - off[e], 0);
      kv = ((unsigned long long)(uint32_t)max(Nq - cnt, 0) << 32) | (uint32_t)e;
    }
    key[e] = kv;
  }
  __syncthreads();
  for (int kk = 2; kk <= pow2; kk <<= 1)
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int e = threadIdx.x; e < pow2; e += 1024) {
        const int p = e ^ jj;
        if (p > e) {
          const unsigned long long x = key[e], y = key[p];
          const bool up = (e & kk) == 0;
          if ((x > y) == up) { key[e] = y; key[p] = x; }
        }
      }
      __syncthreads();
    }
  for (int e = threadIdx.x; e < Nc; e += 1024) order[bh * Nc + e] = (int32_t)(key[e] & 0xffffffffu);
}

// Two waves per SIMD (the register budget of 256 per lane holds the whole
// working set without spills at either head dim).
template <int D, int NW, bool KPAIR>
__global__ __launch_bounds__(64 * NW, 2) void fine_bwd_dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ len, const int32_t* __restrict__ order,
    const float* __restrict__ lse_f, const bf16* __restrict__ dof, const float* __restrict__ delta,
    const float* __restrict__ dqc, const uint8_t* __restrict__ qarg, bf16* __restrict__ dq, Grid g, Grid gk,
    int stride, float scale) {
  using G = ChunkGeom<D>;
  // Three K stages (chunk c for S, c - 1 for the dQ MFMAs, c + 1 loading) and
  // two V stages (c for dP, c + 1 loading): 40 KB at 128 channels.
  __shared__ __attribute__((aligned(16))) bf16 rk[3][G::RUNITS * 8];
  __shared__ __attribute__((aligned(16))) bf16 rv[2][G::RUNITS * 8];

  const int lane = threadIdx.x & 63, n32 = lane & 31, hf = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = slot / g.Nc;
  const int i = order != nullptr ? order[slot] : slot - bh * g.Nc;
  const int item = bh * g.Nc + i;
  const long tok0 = (long)bh * g.N;
  // Lists are validated by contract; the clamps only keep a malformed list
  // from reading outside the tensors.
  const int L = min(max(len[item], 0), stride);
  const int32_t* list = idx + (long)item * stride;

  // This lane's query: in-cube token 32wv + n32 of cube i.
  const long n = tok0 + cube_token(g, i, 32 * wv + n32);
  bf16x8 qf[G::KS], df[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    qf[ks] = *reinterpret_cast<const bf16x8*>(q + n * D + ks * 16 + hf * 8);
    df[ks] = *reinterpret_cast<const bf16x8*>(dof + n * D + ks * 16 + hf * 8);
  }
  const float sl2 = scale * kLog2e;
  const float lse2 = lse_f[n] * kLog2e, dl = delta[n];
  f32x16 acc[G::MB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0.f;

  // Key chunks: key block list[c >> ksh], its chunk h = c & kmask; 16-token
  // key blocks go two to a chunk (entries 2c, 2c + 1; the upper half of the
  // last chunk of an odd list repeats the lower block and is masked).
  constexpr bool kpair = KPAIR;   // gk.B == 16
  const int ksh = kpair ? 0 : chunk_shift(gk), kmask = (1 << ksh) - 1;
  uint32_t roff[G::RINS / NW];
  row_tile_offsets<D, NW>(gk, wv, lane, roff, kpair ? 15 : 31);
  uint32_t toffs[G::MB][2][2];   // transposed reads of the K row tile (dQ^T += K^T dS^T)
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) rowt_offsets<D>(lane, mb, s2, toffs[mb][s2]);
  // Bytes from a key block's first row to the first row of its chunk h.
  auto chunk_bytes = [&](int h) { return (uint32_t)(chunk_first(gk, h) * D) * 2u; };
  const char* Kb = reinterpret_cast<const char*>(k + tok0 * D);
  const char* Vb = reinterpret_cast<const char*>(v + tok0 * D);
  // Byte offsets of the list's cubes, 64 entries at a time, one per lane.
  uint32_t rcube = 0;
  auto cubes = [&](int t0) {
    const int t = t0 + lane;
    int j = t < L ? list[t] : 0;
    j = (j >= 0 && j < gk.Nc) ? j : 0;
    rcube = (uint32_t)cube_first(gk, j) * (uint32_t)(D * 2);
  };
  const uint32_t rkb = lds_addr(rk), rvb = lds_addr(rv);
  auto issue = [&](int c) {
    const int e = kpair ? 2 * c : c >> ksh, h = kpair ? 0 : c & kmask, sk = c % 3, sv = c & 1;
    if ((e & 63) == 0 && h == 0) cubes(e);
    const uint32_t rc = __builtin_amdgcn_readlane(rcube, e & 63) + chunk_bytes(h);
    if constexpr (kpair) {   // entries e, e + 1 share a block of 64 (e is even)
      const uint32_t rc1 = __builtin_amdgcn_readlane(rcube, min(e + 1, L - 1) & 63);
      issue_row_tile2<D, NW>(uniform_ptr(Kb + rc), uniform_ptr(Kb + rc1), roff, rkb + sk * (G::RUNITS * 16), wv);
      issue_row_tile2<D, NW>(uniform_ptr(Vb + rc), uniform_ptr(Vb + rc1), roff, rvb + sv * (G::RUNITS * 16), wv);
      return;
    }
    issue_row_tile<D, NW>(uniform_ptr(Kb + rc), roff, rkb + sk * (G::RUNITS * 16), wv);
    issue_row_tile<D, NW>(uniform_ptr(Vb + rc), roff, rvb + sv * (G::RUNITS * 16), wv);
  };

  // Step c: wait for this wave's loads of chunk c, barrier (every wave's share
  // is in LDS; every wave is done with the stages chunk c + 1 refills: K of
  // c - 2, V of c - 1), issue chunk c + 1, then: the score MFMAs of chunk c;
  // its dP MFMAs, with P = 2^(s*c - LSE) formed one slice per MFMA once the
  // scores are in; and the dQ MFMAs of chunk c - 1 (dS formed in step c - 1,
  // K of c - 1 still in its stage), with dS of chunk c formed one slice per
  // MFMA. Softmax and dS work thus run under the MFMAs of the same wave.
  const int nch = kpair ? (L + 1) >> 1 : L << ksh;
  const bool khalf = kpair && (L & 1);   // keys 16-31 of the last chunk absent
  bf16x8 dsa[2], dsb[2];   // dS of a chunk, as the B operand of its dQ MFMAs
  // The loop is unrolled by six (both stage counts divide it) so that every
  // stage, and with it every LDS address, is a compile-time constant. A step
  // is a sequence of slots, one MFMA each: the score MFMAs, the dP MFMAs (with
  // the exponentials), the dQ MFMAs of chunk c - 1 (with dS of chunk c); each
  // slot's LDS fragment is read three slots ahead, so that few are live. DQ:
  // there is a chunk c - 1.
  auto step = [&](auto PP, auto DQ, const bf16x8 (&dprev)[2], bf16x8 (&dcur)[2], int c) {
    constexpr int p = decltype(PP)::value;
    constexpr bool kDq = decltype(DQ)::value;
    constexpr int sk = p % 3, sv = p % 2, skp = (p + 2) % 3;   // K stage of c, V stage of c, K stage of c - 1
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (c + 1 < nch) issue(c + 1);
    constexpr int NS = G::KS, NT = 2 * G::MB, NSLOT = 2 * NS + NT, LA = 3;
    constexpr int PER = 16 / NS, PT = 16 / NT;   // exponentials per dP slot, dS values per dQ slot
    const char* ktp = reinterpret_cast<const char*>(rk[skp]);
    bf16x8 kf[NS], vf[NS], tf[NT];
    auto fetch = [&](int j) {
      if (j < NS) kf[j] = row_frag<D>(rk[sk], n32, hf, j);
      else if (j < 2 * NS) vf[j - NS] = row_frag<D>(rv[sv], n32, hf, j - NS);
      else if (kDq) {
        const int t = j - 2 * NS, s2 = t / G::MB, mb = t % G::MB;
        tf[t] = rowt_frag(ktp, toffs[mb][s2][0], toffs[mb][s2][1]);
      }
    };
    f32x16 sx, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) { sx[e] = 0.f; dp[e] = 0.f; }
#pragma unroll
    for (int j = 0; j < LA; ++j) fetch(j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
      if (j + LA < NSLOT) fetch(j + LA);
      if (j < NS) {
        sx = mfma32_bf16(kf[j], qf[j], sx);
        if (j == NS - 1 && kpair && khalf && c == nch - 1) {   // accumulator entries 8-15 hold keys 16-31
#pragma unroll
          for (int e = 8; e < 16; ++e) sx[e] = -INFINITY;
        }
      } else if (j < 2 * NS) {
        dp = mfma32_bf16(vf[j - NS], df[j - NS], dp);
#pragma unroll
        for (int r = 0; r < PER; ++r) {
          const int e = (j - NS) * PER + r;
          sx[e] = __builtin_amdgcn_exp2f(sx[e] * sl2 - lse2);   // P
        }
      } else {
        const int t = j - 2 * NS, s2 = t / G::MB, mb = t % G::MB;
        if (kDq) acc[mb] = mfma32_bf16(tf[t], dprev[s2], acc[mb]);
#pragma unroll
        for (int r = 0; r < PT; ++r) {
          const int e = t * PT + r;
          dcur[e >> 3][e & 7] = (bf16)(sx[e] * (dp[e] - dl));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using T1 = std::true_type;
  using F0 = std::false_type;
  // Step c writes dS of chunk c into dsa (c even) or dsb (c odd).
  if (nch > 0) {
    issue(0);
    step(I0(), F0(), dsb, dsa, 0);
  }
  int c = 1;
  for (; c + 6 <= nch; c += 6) {
    step(I1(), T1(), dsa, dsb, c);
    step(I2(), T1(), dsb, dsa, c + 1);
    step(I3(), T1(), dsa, dsb, c + 2);
    step(I4(), T1(), dsb, dsa, c + 3);
    step(I5(), T1(), dsa, dsb, c + 4);
    step(I0(), T1(), dsb, dsa, c + 5);
  }
  if (c < nch) {
    step(I1(), T1(), dsa, dsb, c);
    if (c + 1 < nch) {
      step(I2(), T1(), dsb, dsa, c + 1);
      if (c + 2 < nch) {
        step(I3(), T1(), dsa, dsb, c + 2);
        if (c + 3 < nch) {
          step(I4(), T1(), dsb, dsa, c + 3);
          if (c + 4 < nch) step(I5(), T1(), dsa, dsb, c + 4);
        }
      }
    }
  }
  if (nch > 0) {   // the dQ MFMAs of the last chunk (its dS and K stage)
    const int cl = nch - 1;
    const char* ktl = reinterpret_cast<const char*>(rk[cl % 3]);
    const bf16x8(&dl_)[2] = (cl & 1) ? dsb : dsa;
#pragma unroll
    for (int t = 0; t < 2 * G::MB; ++t) {
      const int s2 = t / G::MB, mb = t % G::MB;
      acc[mb] = mfma32_bf16(rowt_frag(ktl, toffs[mb][s2][0], toffs[mb][s2][1]), dl_[s2], acc[mb]);
    }
  }

  // lane holds dQ^T[channel 32mb + 8(jj/4) + 4hf + jj%4][its query]; the
  // pooled gradient goes to every token (mean) or to the cube's maximum. The
  // pooling mode is decided outside the loops so that all of the epilogue's
  // loads are issued before the first use; the bf16 result then goes through
  // this wave's chunk stage so that the stores cover whole 16-byte units of
  // token rows.
  const float* dqc_i = dqc + ((long)bh * g.Nc + i) * D;
  const uint8_t* qarg_i = qarg != nullptr ? qarg + ((long)bh * g.Nc + i) * D : nullptr;
  const int lq = 32 * wv + n32;   // the query's position in its cube
  const float inv_b = 1.0f / (float)g.B;
  __syncthreads();   // every wave is done with the chunk stages
  bf16* tile = wv < 3 ? rk[wv] : rv[wv - 3];
  auto finish = [&](auto MAXP) {
    constexpr bool kMax = decltype(MAXP)::value;
    float4 c4[G::MB][4];
    uchar4 a4[G::MB][4];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int ch = 32 * mb + 8 * jq + 4 * hf;
        c4[mb][jq] = *reinterpret_cast<const float4*>(dqc_i + ch);
        if (kMax) a4[mb][jq] = *reinterpret_cast<const uchar4*>(qarg_i + ch);
      }
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const float cv[4] = {c4[mb][jq].x, c4[mb][jq].y, c4[mb][jq].z, c4[mb][jq].w};
        const int av[4] = {a4[mb][jq].x, a4[mb][jq].y, a4[mb][jq].z, a4[mb][jq].w};
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pg = kMax ? (av[r] == lq ? cv[r] : 0.f) : cv[r] * inv_b;
          w[r] = (bf16)(scale * acc[mb][4 * jq + r] + pg);
        }
        *reinterpret_cast<bf16x4*>(tile + (n32 * G::U + ((4 * mb + jq) ^ kswz<G::U>(n32))) * 8 + 4 * hf) = w;
      }
  };
  if (qarg_i != nullptr) finish(std::true_type());
  else finish(std::false_type());
  constexpr int RPI = 64 / G::U, NIT = 32 / RPI;   // token rows per instruction, instructions per tile
  const int u = lane % G::U, r0 = lane / G::U;
  bf16x8 out[NIT];
#pragma unroll
  for (int t = 0; t < NIT; ++t) {
    const int row = t * RPI + r0;
    out[t] = *reinterpret_cast<const bf16x8*>(tile + (row * G::U + (u ^ kswz<G::U>(row))) * 8);
  }
#pragma unroll
  for (int t = 0; t < NIT; ++t) {
    const int row = t * RPI + r0;
    *reinterpret_cast<bf16x8*>(dq + (tok0 + cube_token(g, i, 32 * wv + row)) * D + u * 8) = out[t];
  }
}

// The pooled gradient of every channel a lane holds in the accumulator
// layout (channel 32mb + 8jq + 4hf + r at out[mb][4jq + r]), for token
// position l. The pooling mode is decided once, outside the loops, so that all
// loads are issued before the first use.
template <int MB>
__device__ __forceinline__ void pooled_grads(const float* dxc, const uint8_t* arg, int hf, int l, float inv_b,
                                             float out[MB][16]) {
  float4 c4[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) c4[mb][jq] = *reinterpret_cast<const float4*>(dxc + 32 * mb + 8 * jq + 4 * hf);
  if (arg == nullptr) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        out[mb][4 * jq + 0] = c4[mb][jq].x * inv_b;
        out[mb][4 * jq + 1] = c4[mb][jq].y * inv_b;
        out[mb][4 * jq + 2] = c4[mb][jq].z * inv_b;
        out[mb][4 * jq + 3] = c4[mb][jq].w * inv_b;
      }
  } else {
    uchar4 a4[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) a4[mb][jq] = *reinterpret_cast<const uchar4*>(arg + 32 * mb + 8 * jq + 4 * hf);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        out[mb][4 * jq + 0] = a4[mb][jq].x == l ? c4[mb][jq].x : 0.f;
        out[mb][4 * jq + 1] = a4[mb][jq].y == l ? c4[mb][jq].y : 0.f;
        out[mb][4 * jq + 2] = a4[mb][jq].z == l ? c4[mb][jq].z : 0.f;
        out[mb][4 * jq + 3] = a4[mb][jq].w == l ? c4[mb][jq].w : 0.f;
      }
  }
}

// In both dK / dV kernels g is the grid of key blocks (the workgroup's own
// tokens) and gq the grid of query cubes (the partners walked).
//
// The keys a dK / dV workgroup owns and the query cubes it walks. Ordinary
// blocks: key block j (its slot, through `order` when given), lane n32 of key
// wave kw is the block's token 32 kw + n32, and the list is j's transposed
// list. KPAIR (16-token key blocks, two per 32-key MFMA column block): blocks
// 2P and 2P + 1, lane n32 is token n32 % 16 of block 2P + n32 / 16, and the
// list is the union of the two transposed lists (k2q_pair_kernel), each entry
// a query cube with bit 24 (listed by 2P) and bit 25 (by 2P + 1) set.
struct KeyWalk {
  int bh, j, lk, L;
  bool own;   // the lane's key block exists (the last pair of an odd Nk has one)
  const int32_t* list;
};
template <bool KPAIR>
__device__ __forceinline__ KeyWalk key_walk(const Grid& g, const Grid& gq, const int32_t* k2q_off,
                                            const int32_t* k2q, const int32_t* order, const int32_t* plen,
                                            int stride, int kw, int n32) {
  KeyWalk w;
  const int slot = xcd_remap(blockIdx.x, gridDim.x);
  const int cap = gq.Nc * stride;
  if constexpr (KPAIR) {
    const int npairs = (g.Nc + 1) >> 1;
    w.bh = slot / npairs;
    const int P = slot - w.bh * npairs;
    const int32_t* offs = k2q_off + (long)w.bh * (g.Nc + 1);
    const int t0 = min(max(offs[2 * P], 0), cap);
    w.L = min(max(plen[(long)w.bh * npairs + P], 0), cap - t0);
    w.list = k2q + (long)w.bh * cap + t0;
    const int jl = 2 * P + (n32 >> 4);
    w.own = jl < g.Nc;
    w.j = w.own ? jl : 2 * P;
    w.lk = n32 & 15;
  } else {
    w.bh = slot / g.Nc;
    w.j = order != nullptr ? order[slot] : slot - w.bh * g.Nc;
    const int32_t* offs = k2q_off + (long)w.bh * (g.Nc + 1);
    const int t0 = min(max(offs[w.j], 0), cap), t1 = min(max(offs[w.j + 1], t0), cap);
    w.list = k2q + (long)w.bh * cap + t0;
    w.L = t1 - t0;
    w.own = true;
    w.lk = 32 * kw + n32;
  }
  return w;
}
//
// dK and dV at 64 channels: every wave computes both for its 32 keys. With
// two or more waves per workgroup the kernel is held to 168 registers, three
// waves per SIMD (measured 4% faster on the training workload than two, at
// one spilled register); a one-wave workgroup's LDS stages allow no more than
// about two per SIMD, so it keeps the 256-register budget. (At 128 channels
// the two accumulators, 128 registers, and the lane's K and V rows do not fit
// 256 registers without spills; the warp-specialized kernel below splits the
// roles over the waves instead.)
template <int D, int NW, bool KPAIR>
__global__ __launch_bounds__(64 * NW, NW == 1 ? 2 : 3) void fine_bwd_dkdv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ k2q_off,
    const int32_t* __restrict__ k2q, const int32_t* __restrict__ order, const int32_t* __restrict__ plen,
    const float* __restrict__ lse_f,
    const bf16* __restrict__ dof, const float* __restrict__ delta, const float* __restrict__ dkc,
    const float* __restrict__ dvc, const uint8_t* __restrict__ karg, const uint8_t* __restrict__ varg,
    bf16* __restrict__ dk, bf16* __restrict__ dv, Grid g, Grid gq, int stride, float scale) {
  using G = ChunkGeom<D>;
  __shared__ __attribute__((aligned(16))) bf16 rq[2][G::RUNITS * 8];
  __shared__ __attribute__((aligned(16))) bf16 rd[2][G::RUNITS * 8];
  // LSE (log2 units after the load) and delta of the chunk's 32 query rows.
  __shared__ __attribute__((aligned(16))) float rls[2][32];
  __shared__ __attribute__((aligned(16))) float rdl[2][32];

  const int lane = threadIdx.x & 63, n32 = lane & 31, hf = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const KeyWalk kwk = key_walk<KPAIR>(g, gq, k2q_off, k2q, order, plen, stride, wv, n32);
  const int bh = kwk.bh, j = kwk.j, L = kwk.L;
  const int32_t* list = kwk.list;
  const long tok0 = (long)bh * g.N;

  // This lane's key: token lk of key block j.
  const long n = tok0 + cube_token(g, j, kwk.lk);
  bf16x8 kf[G::KS], vf[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    kf[ks] = *reinterpret_cast<const bf16x8*>(k + n * D + ks * 16 + hf * 8);
    vf[ks] = *reinterpret_cast<const bf16x8*>(v + n * D + ks * 16 + hf * 8);
  }
  const float sl2 = scale * kLog2e;
  f32x16 adk[G::MB], adv[G::MB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) { adk[mb][e] = 0.f; adv[mb][e] = 0.f; }

  // Query chunks: query cube list[c >> qsh], its chunk h = c & qmask.
  const int qsh = chunk_shift(gq), qmask = (1 << qsh) - 1;
  uint32_t roff[G::RINS / NW];
  row_tile_offsets<D, NW>(gq, wv, lane, roff);
  uint32_t toffs[G::MB][2][2];   // transposed reads of the Q / dO row tiles
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) rowt_offsets<D>(lane, mb, s2, toffs[mb][s2]);
  const char* Qb = reinterpret_cast<const char*>(q + tok0 * D);
  const char* Db = reinterpret_cast<const char*>(dof + tok0 * D);
  const char* Lb = reinterpret_cast<const char*>(lse_f + tok0);
  const char* Eb = reinterpret_cast<const char*>(delta + tok0);
  // Per lane, for 64 list entries at a time: the partner cube's first row.
  int rcube = 0, rflag = 3;
  auto cubes = [&](int e0) {
    const int t = e0 + lane;
    int ii = t < L ? list[t] : 0;
    if constexpr (KPAIR) {
      rflag = (ii >> 24) & 3;
      ii &= 0xFFFFFF;
    }
    ii = (ii >= 0 && ii < gq.Nc) ? ii : 0;
    rcube = cube_first(gq, ii);
  };
  const uint32_t rqb = lds_addr(rq), rdb = lds_addr(rd), rlb = lds_addr(rls), reb = lds_addr(rdl);
  // Rows 4t .. 4t+3 of a chunk are consecutive in memory (Cw >= 4): lane t
  // < 8 of wave 0 moves them for LSE (and delta) with one 16-byte load.
  const uint32_t soff = (uint32_t)chunk_row(gq, 4 * (lane & 7)) * 4u;
  auto issue = [&](int c) {
    const int e = c >> qsh, h = c & qmask, st = c & 1;
    if ((e & 63) == 0 && h == 0) cubes(e);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane(rcube, e & 63) + (uint32_t)chunk_first(gq, h);
    const uint32_t rc = r0 * (uint32_t)(D * 2);
    issue_row_tile<D, NW>(uniform_ptr(Qb + rc), roff, rqb + st * (G::RUNITS * 16), wv);
    issue_row_tile<D, NW>(uniform_ptr(Db + rc), roff, rdb + st * (G::RUNITS * 16), wv);
    if (wv == 0 && lane < 8) {
      dma16(uniform_ptr(Lb + r0 * 4u), soff, rlb + st * 128);
      dma16(uniform_ptr(Eb + r0 * 4u), soff, reb + st * 128);
    }
  };

  const int nch = L << qsh;
  if (nch > 0) issue(0);
  for (int c = 0; c < nch; ++c) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    // Whether the query cube of chunk c is listed by this lane's key block
    // (read before issue(c + 1) may refresh the entries).
    const bool kvalid = !KPAIR || ((__builtin_amdgcn_readlane(rflag, (c >> qsh) & 63) >> (n32 >> 4)) & 1);
    if (c + 1 < nch) issue(c + 1);
    const int st = c & 1;
    // LSE and delta of the accumulator rows this lane holds: rows 8m + 4hf + r.
    f32x16 sx, dp;
#pragma unroll
    for (int e = 0; e < 16; ++e) { sx[e] = 0.f; dp[e] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) {
      sx = mfma32_bf16(row_frag<D>(rq[st], n32, hf, ks), kf[ks], sx);
      dp = mfma32_bf16(row_frag<D>(rd[st], n32, hf, ks), vf[ks], dp);
    }
    // LSE (to log2 units) and delta of the accumulator rows this lane holds
    // (rows 8m + 4hf + r), read four at a time where they are used.
    bf16x8 pf[2], sf[2];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float4 a = *reinterpret_cast<const float4*>(&rls[st][8 * m + 4 * hf]);
      const float4 b = *reinterpret_cast<const float4*>(&rdl[st][8 * m + 4 * hf]);
      const float la[4] = {a.x, a.y, a.z, a.w}, db[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * m + r;
        float p = __builtin_amdgcn_exp2f(sx[e] * sl2 - la[r] * kLog2e);
        if constexpr (KPAIR) p = kvalid ? p : 0.f;
        pf[e >> 3][e & 7] = (bf16)p;
        sf[e >> 3][e & 7] = (bf16)(p * (dp[e] - db[r]));
      }
    }
    const char* qtile = reinterpret_cast<const char*>(rq[st]);
    const char* dtile = reinterpret_cast<const char*>(rd[st]);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb) {
        adv[mb] = mfma32_bf16(rowt_frag(dtile, toffs[mb][s2][0], toffs[mb][s2][1]), pf[s2], adv[mb]);
        adk[mb] = mfma32_bf16(rowt_frag(qtile, toffs[mb][s2][0], toffs[mb][s2][1]), sf[s2], adk[mb]);
      }
  }

  // lane holds d{K,V}^T[channel 32mb + 8(jj/4) + 4hf + jj%4][its key]
  const long cj = ((long)bh * g.Nc + j) * D;
  const uint8_t* karg_j = karg != nullptr ? karg + cj : nullptr;
  const uint8_t* varg_j = varg != nullptr ? varg + cj : nullptr;
  const int lk = kwk.lk;   // the key's position in its block
  const float inv_b = 1.0f / (float)g.B;
  if (!kwk.own) return;   // no barrier below
  float kcv[G::MB][16], vcv[G::MB][16];
  pooled_grads<G::MB>(dkc + cj, karg_j, hf, lk, inv_b, kcv);
  pooled_grads<G::MB>(dvc + cj, varg_j, hf, lk, inv_b, vcv);
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const int ch = 32 * mb + 8 * jq + 4 * hf;
      bf16x4 wk, wvv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        wk[r] = (bf16)(scale * adk[mb][4 * jq + r] + kcv[mb][4 * jq + r]);
        wvv[r] = (bf16)(adv[mb][4 * jq + r] + vcv[mb][4 * jq + r]);
      }
      *reinterpret_cast<bf16x4*>(dk + n * D + ch) = wk;
      *reinterpret_cast<bf16x4*>(dv + n * D + ch) = wvv;
    }
}

// dK and dV at 128 channels, warp-specialized: a workgroup of 2 NW waves owns
// a key block. Per 32-key group, a dV wave forms S = Q_c K^T and P (the
// lane's K row in registers), hands P (bf16, the values dV is formed with) to
// its partner dK wave through LDS and accumulates dV^T += dO_c^T P; the dK
// wave forms dP = dO_c V^T (the lane's V row in registers), dS = P * (dP -
// delta) with its partner's P, and accumulates dK^T += Q_c^T dS. Both do 16
// MFMAs per chunk and each keeps one row operand and one accumulator array,
// so the working set fits two waves per SIMD. The dK waves run one chunk
// behind (they need that chunk's P) and chunks load two ahead, so Q / dO /
// LSE / delta chunks have four LDS stages and P two slots. The roles swap
// with the workgroup's parity, so that the two workgroups sharing a CU tend
// to put a wave of each role on every SIMD.
template <int D, int NW, bool KPAIR>
__global__ __launch_bounds__(128 * NW, 2) void fine_bwd_dkdv_ws_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ k2q_off,
    const int32_t* __restrict__ k2q, const int32_t* __restrict__ order, const int32_t* __restrict__ plen,
    const float* __restrict__ lse_f,
    const bf16* __restrict__ dof, const float* __restrict__ delta, const float* __restrict__ dkc,
    const float* __restrict__ dvc, const uint8_t* __restrict__ karg, const uint8_t* __restrict__ varg,
    bf16* __restrict__ dk, bf16* __restrict__ dv, Grid g, Grid gq, int stride, float scale) {
  using G = ChunkGeom<D>;
  constexpr int NWT = 2 * NW;   // waves in the workgroup
  constexpr int QST = 4;        // stages of the Q / dO / LSE / delta chunks
  static_assert(G::RINS % NWT == 0, "every wave issues whole 1 KB loads");
  __shared__ __attribute__((aligned(16))) bf16 rq[QST][G::RUNITS * 8];
  __shared__ __attribute__((aligned(16))) bf16 rd[QST][G::RUNITS * 8];
  __shared__ __attribute__((aligned(16))) float rls[QST][32];
  __shared__ __attribute__((aligned(16))) float rdl[QST][32];
  // P of each dV wave's chunk, lane-major: [slot][key group][half][lane].
  __shared__ __attribute__((aligned(16))) bf16x8 xp[2][NW][2][64];

  const int lane = threadIdx.x & 63, n32 = lane & 31, hf = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = wv % NW;                                     // keys 32kw .. 32kw + 31
  const bool isk = ((wv / NW) ^ (int)(blockIdx.x & 1)) != 0;  // this wave computes dK (else dV)
  const KeyWalk kwk = key_walk<KPAIR>(g, gq, k2q_off, k2q, order, plen, stride, kw, n32);
  const int bh = kwk.bh, j = kwk.j, L = kwk.L;
  const int32_t* list = kwk.list;
  const long tok0 = (long)bh * g.N;

  // This lane's key: token lk of key block j. A dV wave keeps its K row (the
  // B operand of S = Q K^T), a dK wave its V row (of dP = dO V^T).
  const long n = tok0 + cube_token(g, j, kwk.lk);
  bf16x8 kv[G::KS];
  const bf16* kvrow = (isk ? v : k) + n * D;
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) kv[ks] = *reinterpret_cast<const bf16x8*>(kvrow + ks * 16 + hf * 8);
  const float sl2 = scale * kLog2e;
  f32x16 acc[G::MB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0.f;

  const int qsh = chunk_shift(gq), qmask = (1 << qsh) - 1;
  uint32_t roff[G::RINS / NWT];
  row_tile_offsets<D, NWT>(gq, wv, lane, roff);
  uint32_t toffs[G::MB][2][2];   // transposed reads of the Q / dO row tiles
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) rowt_offsets<D>(lane, mb, s2, toffs[mb][s2]);
  const char* Qb = reinterpret_cast<const char*>(q + tok0 * D);
  const char* Db = reinterpret_cast<const char*>(dof + tok0 * D);
  const char* Lb = reinterpret_cast<const char*>(lse_f + tok0);
  const char* Eb = reinterpret_cast<const char*>(delta + tok0);
  int rcube = 0, rflag = 3;
  auto cubes = [&](int e0) {
    const int t = e0 + lane;
    int ii = t < L ? list[t] : 0;
    if constexpr (KPAIR) {
      rflag = (ii >> 24) & 3;
      ii &= 0xFFFFFF;
    }
    ii = (ii >= 0 && ii < gq.Nc) ? ii : 0;
    rcube = cube_first(gq, ii);
  };
  const uint32_t rqb = lds_addr(rq), rdb = lds_addr(rd), rlb = lds_addr(rls), reb = lds_addr(rdl);
  const uint32_t soff = (uint32_t)chunk_row(gq, 4 * (lane & 7)) * 4u;
  // Query chunks: query cube list[c >> qsh], its chunk h = c & qmask, into
  // stage c % QST.
  auto issue = [&](int c) {
    const int e = c >> qsh, h = c & qmask, st = c % QST;
    if ((e & 63) == 0 && h == 0) cubes(e);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane(rcube, e & 63) + (uint32_t)chunk_first(gq, h);
    const uint32_t rc = r0 * (uint32_t)(D * 2);
    issue_row_tile<D, NWT>(uniform_ptr(Qb + rc), roff, rqb + st * (G::RUNITS * 16), wv);
    issue_row_tile<D, NWT>(uniform_ptr(Db + rc), roff, rdb + st * (G::RUNITS * 16), wv);
    if (wv == 0 && lane < 8) {
      dma16(uniform_ptr(Lb + r0 * 4u), soff, rlb + st * 128);
      dma16(uniform_ptr(Eb + r0 * 4u), soff, reb + st * 128);
    }
  };

  // Iteration c: the dV waves work on chunk c, the dK waves on chunk c - 1.
  // At its top every wave's loads of chunk c have landed and the P of chunk
  // c - 1 is in LDS (each wave waits for its own loads and LDS writes, then
  // the barrier); chunk c + 2 is then issued into the stage chunk c - 2 used.
  // Wave 0 also issues the LSE and delta loads (two more per chunk).
  const int nch = L << qsh;
  constexpr int RPW = G::RINS / NWT;   // loads per wave per row tile
  // Whether the query cube of chunk c is listed by this lane's key block,
  // read while c's block of 64 list entries is the one loaded (an issue()
  // may refresh it for a later chunk).
  auto kflag = [&](int c) {
    return !KPAIR || ((__builtin_amdgcn_readlane(rflag, (c >> qsh) & 63) >> (n32 >> 4)) & 1);
  };
  bool kvalid_next = true;
  if (nch > 0) {
    issue(0);
    kvalid_next = kflag(0);
  }
  if (nch > 1) issue(1);
  // The first chunks' loads were issued back to back, so waiting for all of
  // them here costs little, and it lets the compiler count the K / V rows as
  // arrived (it would otherwise wait for them, and for every load in flight,
  // before each chunk's MFMAs).
  vm_settled();
  // Iteration c of the walk. Its LDS stage U = c % QST is a compile-time
  // constant (the walk below is unrolled by QST), so every LDS address is a
  // constant offset from a loop-invariant lane address; the role is one too,
  // so each role runs its own copy of the loop and its accumulator stays in
  // place across iterations.
  static_assert(QST == 4, "the walk is unrolled by four");
  auto iter = [&](auto role, auto stage, int c) {
    constexpr bool ISK = decltype(role)::value;
    constexpr int U = decltype(stage)::value;
    // Chunk c has landed once only chunk c + 1's loads may be outstanding.
    if (c + 1 < nch) {
      if (wv == 0) wait_vmcnt<2 * RPW + 2>();
      else wait_vmcnt<2 * RPW>();
    } else {
      wait_vmcnt<0>();
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    const bool kvalid = kvalid_next;
    if (c + 1 < nch) kvalid_next = kflag(c + 1);   // chunk c + 1 was issued before chunk c + 2
    if (c + 2 < nch) issue(c + 2);
    if constexpr (!ISK) {
      if (c < nch) {
        constexpr int st = U;
        float lse2[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 a = *reinterpret_cast<const float4*>(&rls[st][8 * m + 4 * hf]);
          lse2[4 * m + 0] = a.x * kLog2e; lse2[4 * m + 1] = a.y * kLog2e;
          lse2[4 * m + 2] = a.z * kLog2e; lse2[4 * m + 3] = a.w * kLog2e;
        }
        f32x16 sx;
#pragma unroll
        for (int e = 0; e < 16; ++e) sx[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) sx = mfma32_bf16(row_frag<D>(rq[st], n32, hf, ks), kv[ks], sx);
#pragma unroll
        for (int e = 0; e < 16; ++e) sx[e] = __builtin_amdgcn_exp2f(sx[e] * sl2 - lse2[e]);   // P
        if constexpr (KPAIR) {
          if (!kvalid) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sx[e] = 0.f;
          }
        }
        bf16x8 pf[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) pf[e >> 3][e & 7] = (bf16)sx[e];
        xp[U & 1][kw][0][lane] = pf[0];
        xp[U & 1][kw][1][lane] = pf[1];
        const char* dtile = reinterpret_cast<const char*>(rd[st]);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int mb = 0; mb < G::MB; ++mb)
            acc[mb] = mfma32_bf16(rowt_frag(dtile, toffs[mb][s2][0], toffs[mb][s2][1]), pf[s2], acc[mb]);
        __builtin_amdgcn_s_setprio(0);
      }
    } else {
      (void)kvalid;
      if (c > 0) {   // chunk c - 1: its stage and P slot
        constexpr int st = (U + QST - 1) % QST, slot = (U + 1) & 1;
        f32x16 dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) dp[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) dp = mfma32_bf16(row_frag<D>(rd[st], n32, hf, ks), kv[ks], dp);
        bf16x8 sf[2];
        const bf16x8 pp[2] = {xp[slot][kw][0][lane], xp[slot][kw][1][lane]};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float4 b = *reinterpret_cast<const float4*>(&rdl[st][8 * t + 4 * hf]);
          const float d4[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * t + r;
            sf[e >> 3][e & 7] = (bf16)((float)pp[e >> 3][e & 7] * (dp[e] - d4[r]));
          }
        }
        const char* qtile = reinterpret_cast<const char*>(rq[st]);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int mb = 0; mb < G::MB; ++mb)
            acc[mb] = mfma32_bf16(rowt_frag(qtile, toffs[mb][s2][0], toffs[mb][s2][1]), sf[s2], acc[mb]);
        __builtin_amdgcn_s_setprio(0);
      }
    }
  };
  // Both roles run iterations 0 .. nch, one barrier each.
  auto walk = [&](auto role) {
    for (int c = 0; c <= nch; c += QST) {
      iter(role, std::integral_constant<int, 0>{}, c);
      if (c + 1 <= nch) iter(role, std::integral_constant<int, 1>{}, c + 1);
      if (c + 2 <= nch) iter(role, std::integral_constant<int, 2>{}, c + 2);
      if (c + 3 <= nch) iter(role, std::integral_constant<int, 3>{}, c + 3);
    }
  };
  if (isk) walk(std::true_type{});
  else walk(std::false_type{});

  // lane holds d{K,V}^T[channel 32mb + 8(jj/4) + 4hf + jj%4][its key]
  const long cj = ((long)bh * g.Nc + j) * D;
  const uint8_t* arg_j = isk ? (karg != nullptr ? karg + cj : nullptr) : (varg != nullptr ? varg + cj : nullptr);
  const float* xc = (isk ? dkc : dvc) + cj;
  bf16* out = isk ? dk : dv;
  const float sc = isk ? scale : 1.0f;
  const int lk = kwk.lk;   // the key's position in its block
  const float inv_b = 1.0f / (float)g.B;
  if (!kwk.own) return;   // no barrier below
  float cv[G::MB][16];
  pooled_grads<G::MB>(xc, arg_j, hf, lk, inv_b, cv);
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      bf16x4 w4;
#pragma unroll
      for (int r = 0; r < 4; ++r) w4[r] = (bf16)(sc * acc[mb][4 * jq + r] + cv[mb][4 * jq + r]);
      *reinterpret_cast<bf16x4*>(out + n * D + 32 * mb + 8 * jq + 4 * hf) = w4;
    }
}

hipError_t launch_order_by_count(const Launch& L, const int32_t* k2q_off, int32_t* order) {
  int pow2 = 1;
  while (pow2 < L.gk.Nc) pow2 <<= 1;
  if (pow2 > kMaxSortKeys) return hipErrorInvalidValue;
  hipLaunchKernelGGL(order_by_count_kernel, dim3(L.BH), dim3(1024), 0, L.stream, k2q_off, order, L.gk.Nc, L.g.Nc,
                     pow2);
  return hipGetLastError();
}

// dQ: one workgroup of Bt/32 waves per query cube.
template <int D, int NW>
static void launch_dq(const Launch& L, const bf16* q, const bf16* k, const bf16* v, const int32_t* idx,
                      const int32_t* len, const int32_t* qorder, const float* lse_f, const bf16* dof,
                      const float* delta, const float* dqc, const uint8_t* qarg, bf16* dq) {
  if (L.gk.B == 16)
    hipLaunchKernelGGL((fine_bwd_dq_kernel<D, NW, true>), dim3(L.BH * L.g.Nc), dim3(64 * NW), 0, L.stream, q, k, v,
                       idx, len, qorder, lse_f, dof, delta, dqc, qarg, dq, L.g, L.gk, L.stride, L.scale);
  else
    hipLaunchKernelGGL((fine_bwd_dq_kernel<D, NW, false>), dim3(L.BH * L.g.Nc), dim3(64 * NW), 0, L.stream, q, k, v,
                       idx, len, qorder, lse_f, dof, delta, dqc, qarg, dq, L.g, L.gk, L.stride, L.scale);
}

// dK / dV: one workgroup per key block, Bk/32 waves (64 channels) or 2 Bk/32
// (128 channels, warp-specialized); 16-token key blocks go in pairs (KPAIR),
// one 32-key wave (or two) per pair, over the pairs' union lists.
template <int D, int NW, bool KPAIR>
static void launch_dkdv(const Launch& L, const bf16* q, const bf16* k, const bf16* v, const int32_t* k2q_off,
                        const int32_t* k2q, const int32_t* korder, const int32_t* plen, const float* lse_f,
                        const bf16* dof, const float* delta, const float* dkc, const float* dvc,
                        const uint8_t* karg, const uint8_t* varg, bf16* dk, bf16* dv) {
  const dim3 grid(L.BH * (KPAIR ? (L.gk.Nc + 1) / 2 : L.gk.Nc));
  if constexpr (D == 64)
    hipLaunchKernelGGL((fine_bwd_dkdv_kernel<D, NW, KPAIR>), grid, dim3(64 * NW), 0, L.stream, q, k, v, k2q_off,
                       k2q, korder, plen, lse_f, dof, delta, dkc, dvc, karg, varg, dk, dv, L.gk, L.g, L.stride,
                       L.scale);
  else
    hipLaunchKernelGGL((fine_bwd_dkdv_ws_kernel<D, NW, KPAIR>), grid, dim3(128 * NW), 0, L.stream, q, k, v,
                       k2q_off, k2q, korder, plen, lse_f, dof, delta, dkc, dvc, karg, varg, dk, dv, L.gk, L.g,
                       L.stride, L.scale);
}

template <int D>
static void fine_bwd_launch(const Launch& L, const bf16* q, const bf16* k, const bf16* v, const int32_t* idx,
                            const int32_t* len, const int32_t* qorder, const int32_t* k2q_off, const int32_t* k2q,
                            const int32_t* korder, const float* lse_f, const bf16* dof, const float* delta,
                            const float* dqc, const float* dkc, const float* dvc, bf16* dq, bf16* dk, bf16* dv,
                            const uint8_t* qarg, const uint8_t* karg, const uint8_t* varg, const int32_t* k2u,
                            const int32_t* plen) {
  if (L.g.B == 32) launch_dq<D, 1>(L, q, k, v, idx, len, qorder, lse_f, dof, delta, dqc, qarg, dq);
  else if (L.g.B == 128) launch_dq<D, 4>(L, q, k, v, idx, len, qorder, lse_f, dof, delta, dqc, qarg, dq);
  else launch_dq<D, 2>(L, q, k, v, idx, len, qorder, lse_f, dof, delta, dqc, qarg, dq);
  if (L.gk.B == 16)
    launch_dkdv<D, 1, true>(L, q, k, v, k2q_off, k2u, nullptr, plen, lse_f, dof, delta, dkc, dvc, karg, varg, dk,
                            dv);
  else if (L.gk.B == 32)
    launch_dkdv<D, 1, false>(L, q, k, v, k2q_off, k2q, korder, nullptr, lse_f, dof, delta, dkc, dvc, karg, varg,
                             dk, dv);
  else if (L.gk.B == 128)
    launch_dkdv<D, 4, false>(L, q, k, v, k2q_off, k2q, korder, nullptr, lse_f, dof, delta, dkc, dvc, karg, varg,
                             dk, dv);
  else
    launch_dkdv<D, 2, false>(L, q, k, v, k2q_off, k2q, korder, nullptr, lse_f, dof, delta, dkc, dvc, karg, varg,
                             dk, dv);
}

// fp32 path of the fine backward (fp32 problems, small correctness-first
// shapes), fp32 arithmetic throughout. Each token is handled by TPT = D / 32
// adjacent threads, thread `part` holding channels 32*part .. 32*part+31, so
// that no thread keeps more than 4 x 32 floats; the dot products are summed
// over the TPT threads with lane exchanges. The partner rows are staged in
// LDS up to 32 at a time. The pooled gradient of the token's cube (or key
// block) is added in the epilogue as in the bf16 kernels.
constexpr int kF32Part = 32;   // channels per thread

template <int TPT> __device__ __forceinline__ float part_sum(float x) {
  if (TPT >= 2) x += __shfl_xor(x, 1);
  if (TPT >= 4) x += __shfl_xor(x, 2);
  return x;
}

template <int D>
__global__ __launch_bounds__(512) void fine_bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ len, const float* __restrict__ lse_f,
    const float* __restrict__ dof, const float* __restrict__ delta, const float* __restrict__ dqc,
    const uint8_t* __restrict__ qarg, float* __restrict__ dq, Grid g, Grid gk, int stride, float scale) {
  constexpr int R = 32, C = kF32Part, TPT = D / C;
  __shared__ float ks[R][D];
  __shared__ float vs[R][D];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int tok = tid / TPT, c0 = (tid % TPT) * C;
  const int item = blockIdx.x;
  const int bh = item / g.Nc, i = item - bh * g.Nc;
  const long tok0 = (long)bh * g.N;
  const long n = tok0 + cube_token(g, i, tok);
  float qv[C], dov[C], acc[C];
#pragma unroll
  for (int d = 0; d < C; ++d) { qv[d] = q[n * D + c0 + d]; dov[d] = dof[n * D + c0 + d]; acc[d] = 0.f; }
  const float lse = lse_f[n], dl = delta[n];
  const int L = min(max(len[item], 0), stride);
  const int32_t* list = idx + (long)item * stride;
  const int RS = min(R, gk.B), spb = gk.B / RS;   // rows per stage, stages per key block
  for (int t = 0; t < L * spb; ++t) {
    const int j = list[t / spb], r0 = (t % spb) * RS;
    if (j < 0 || j >= gk.Nc) continue;
    __syncthreads();
    for (int e = tid; e < RS * D; e += nt) {
      const int r = e / D, d = e - r * D;
      const long src = (tok0 + cube_token(gk, j, r0 + r)) * D + d;
      ks[r][d] = k[src];
      vs[r][d] = v[src];
    }
    __syncthreads();
    for (int r = 0; r < RS; ++r) {
      float sc = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < C; ++d) {
        sc = fmaf(qv[d], ks[r][c0 + d], sc);
        dp = fmaf(dov[d], vs[r][c0 + d], dp);
      }
      sc = part_sum<TPT>(sc);
      dp = part_sum<TPT>(dp);
      const float ds = expf(sc * scale - lse) * (dp - dl);
#pragma unroll
      for (int d = 0; d < C; ++d) acc[d] = fmaf(ds, ks[r][c0 + d], acc[d]);
    }
  }
  const long ci = ((long)bh * g.Nc + i) * D + c0;
  const float inv_b = 1.0f / (float)g.B;
#pragma unroll
  for (int d = 0; d < C; ++d) {
    const float pg = qarg == nullptr ? dqc[ci + d] * inv_b : (qarg[ci + d] == tok ? dqc[ci + d] : 0.f);
    dq[n * D + c0 + d] = scale * acc[d] + pg;
  }
}

template <int D>
__global__ __launch_bounds__(512) void fine_bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ k2q_off, const int32_t* __restrict__ k2q, const float* __restrict__ lse_f,
    const float* __restrict__ dof, const float* __restrict__ delta, const float* __restrict__ dkc,
    const float* __restrict__ dvc, const uint8_t* __restrict__ karg, const uint8_t* __restrict__ varg,
    float* __restrict__ dk, float* __restrict__ dv, Grid g, Grid gq, int stride, float scale) {
  constexpr int R = 32, C = kF32Part, TPT = D / C;
  __shared__ float qs[R][D];
  __shared__ float os[R][D];
  __shared__ float ls[R];
  __shared__ float es[R];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int tok = tid / TPT, c0 = (tid % TPT) * C;
  const int item = blockIdx.x;
  const int bh = item / g.Nc, j = item - bh * g.Nc;   // g: key blocks, gq: query cubes
  const long tok0 = (long)bh * g.N;
  const long n = tok0 + cube_token(g, j, tok);
  float kv[C], vv[C], adk[C], adv[C];
#pragma unroll
  for (int d = 0; d < C; ++d) {
    kv[d] = k[n * D + c0 + d];
    vv[d] = v[n * D + c0 + d];
    adk[d] = 0.f;
    adv[d] = 0.f;
  }
  const int cap = gq.Nc * stride;
  const int32_t* offs = k2q_off + (long)bh * (g.Nc + 1);
  const int t0 = min(max(offs[j], 0), cap), t1 = min(max(offs[j + 1], t0), cap);
  const int32_t* list = k2q + (long)bh * cap + t0;
  const int L = t1 - t0;
  const int RS = min(R, gq.B), spc = gq.B / RS;   // rows per stage, stages per query cube
  for (int t = 0; t < L * spc; ++t) {
    const int i = list[t / spc], r0 = (t % spc) * RS;
    if (i < 0 || i >= gq.Nc) continue;
    __syncthreads();
    for (int e = tid; e < RS * D; e += nt) {
      const int r = e / D, d = e - r * D;
      const long src = (tok0 + cube_token(gq, i, r0 + r)) * D + d;
      qs[r][d] = q[src];
      os[r][d] = dof[src];
    }
    for (int r = tid; r < RS; r += nt) {
      const long tq = tok0 + cube_token(gq, i, r0 + r);
      ls[r] = lse_f[tq];
      es[r] = delta[tq];
    }
    __syncthreads();
    for (int r = 0; r < RS; ++r) {
      float sc = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < C; ++d) {
        sc = fmaf(qs[r][c0 + d], kv[d], sc);
        dp = fmaf(os[r][c0 + d], vv[d], dp);
      }
      sc = part_sum<TPT>(sc);
      dp = part_sum<TPT>(dp);
      const float p = expf(sc * scale - ls[r]);
      const float ds = p * (dp - es[r]);
#pragma unroll
      for (int d = 0; d < C; ++d) {
        adv[d] = fmaf(p, os[r][c0 + d], adv[d]);
        adk[d] = fmaf(ds, qs[r][c0 + d], adk[d]);
      }
    }
  }
  const long cj = ((long)bh * g.Nc + j) * D + c0;
  const float inv_b = 1.0f / (float)g.B;
#pragma unroll
  for (int d = 0; d < C; ++d) {
    const float pk = karg == nullptr ? dkc[cj + d] * inv_b : (karg[cj + d] == tok ? dkc[cj + d] : 0.f);
    const float pv = varg == nullptr ? dvc[cj + d] * inv_b : (varg[cj + d] == tok ? dvc[cj + d] : 0.f);
    dk[n * D + c0 + d] = scale * adk[d] + pk;
    dv[n * D + c0 + d] = adv[d] + pv;
  }
}

template <int D>
static void fine_bwd_launch_f32(const Launch& L, const float* q, const float* k, const float* v, const int32_t* idx,
                                const int32_t* len, const int32_t* k2q_off, const int32_t* k2q, const float* lse_f,
                                const float* dof, const float* delta, const float* dqc, const float* dkc,
                                const float* dvc, float* dq, float* dk, float* dv, const uint8_t* qarg,
                                const uint8_t* karg, const uint8_t* varg) {
  constexpr int TPT = D / kF32Part;
  hipLaunchKernelGGL((fine_bwd_dq_f32_kernel<D>), dim3(L.BH * L.g.Nc), dim3(L.g.B * TPT), 0, L.stream, q, k, v, idx,
                     len, lse_f, dof, delta, dqc, qarg, dq, L.g, L.gk, L.stride, L.scale);
  hipLaunchKernelGGL((fine_bwd_dkdv_f32_kernel<D>), dim3(L.BH * L.gk.Nc), dim3(L.gk.B * TPT), 0, L.stream, q, k, v,
                     k2q_off, k2q, lse_f, dof, delta, dkc, dvc, karg, varg, dk, dv, L.gk, L.g, L.stride, L.scale);
}

hipError_t launch_fine_bwd(const Launch& L, const void* q, const void* k, const void* v, const int32_t* idx,
                           const int32_t* len, const int32_t* qorder, const int32_t* k2q_off, const int32_t* k2q,
                           const int32_t* korder, const float* lse_f, const void* dof, const float* delta,
                           const float* dqc, const float* dkc, const float* dvc, void* dq, void* dk, void* dv,
                           const uint8_t* args, int32_t* pairs) {
  // Argmax planes in launch_pool's layout: q (Nq cubes), then k and v (Nk blocks).
  const long qplane = (long)L.BH * L.g.Nc * L.D, kplane = (long)L.BH * L.gk.Nc * L.D;
  const uint8_t* qarg = args;
  const uint8_t* karg = args != nullptr ? args + qplane : nullptr;
  const uint8_t* varg = args != nullptr ? args + qplane + kplane : nullptr;
  if (!L.bf16) {
    const float *fq = (const float*)q, *fk = (const float*)k, *fv = (const float*)v, *fdo = (const float*)dof;
    if (L.D == 64)
      fine_bwd_launch_f32<64>(L, fq, fk, fv, idx, len, k2q_off, k2q, lse_f, fdo, delta, dqc, dkc, dvc, (float*)dq,
                              (float*)dk, (float*)dv, qarg, karg, varg);
    else
      fine_bwd_launch_f32<128>(L, fq, fk, fv, idx, len, k2q_off, k2q, lse_f, fdo, delta, dqc, dkc, dvc, (float*)dq,
                               (float*)dk, (float*)dv, qarg, karg, varg);
    return hipGetLastError();
  }
  const bf16 *bq = (const bf16*)q, *bk = (const bf16*)k, *bv = (const bf16*)v, *bdo = (const bf16*)dof;
  bf16 *bdq = (bf16*)dq, *bdk = (bf16*)dk, *bdv = (bf16*)dv;
  int32_t* k2u = nullptr;
  int32_t* plen = nullptr;
  if (L.gk.B == 16) {
    if (pairs == nullptr) return hipErrorInvalidValue;
    k2u = pairs;
    plen = pairs + (long)L.BH * L.g.Nc * L.stride;
    const hipError_t e = launch_key_pairs(L, k2q_off, k2q, k2u, plen);
    if (e != hipSuccess) return e;
  }
  if (L.D == 64)
    fine_bwd_launch<64>(L, bq, bk, bv, idx, len, qorder, k2q_off, k2q, korder, lse_f, bdo, delta, dqc, dkc, dvc, bdq,
                        bdk, bdv, qarg, karg, varg, k2u, plen);
  else
    fine_bwd_launch<128>(L, bq, bk, bv, idx, len, qorder, k2q_off, k2q, korder, lse_f, bdo, delta, dqc, dkc, dvc,
                         bdq, bdk, bdv, qarg, karg, varg, k2u, plen);
  return hipGetLastError();
}

}  // namespace vsa
