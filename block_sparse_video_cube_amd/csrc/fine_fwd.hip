// Step 4 of VSA: fine block-sparse attention, optionally fused with step 5
// (gated combine + untile) in the epilogue.
//
// VSA summary page (paperlayer.ai, arXiv 2505.13389), section 2 "Methods"
// (fine stage: token attention only inside the selected cubes, expanded to
// 64x64 blocks; gating combines coarse and fine) and Appendix B (token QK,
// mask unselected, softmax, times V; combine, untile); VSA reading notes,
// key designs 2-3. Variable-length lists per query cube: VSA2 abstract.
//
// bf16 kernel: a workgroup of NW = Bt/32 waves owns one query cube of Bt
// tokens (two waves for the default 64-token cube); wave w owns the queries
// 32w .. 32w+31 and walks the cube's list of key blocks (Bk tokens each, Bk/32
// chunks; a key block is the query cube unless the problem gives keys their
// own tile) in 32-key chunks with an online softmax (32x32x16 bf16 MFMAs):
//   S^T = K_chunk Q^T    A = the chunk's K row tile (LDS), B = the lane's Q
//                        row (registers, loaded once);
//   the accumulator gives every lane one query column and 16 of the 32 keys,
//   so the row max and sum are lane-local plus one exchange between the two
//   lane halves, and P^T is already the B operand of
//   O^T += V_chunk^T P^T  A = the chunk's V row tile read transposed (LDS
//                        transpose reads, in the accumulator's row order).
// Chunks go to LDS with direct-to-LDS loads, each wave issuing 1/NW of them,
// several chunks ahead, and all NW waves read them. Every lane ends with O^T for its query column, so the 1/l
// normalisation, LSE and the fused gate epilogue need no data exchange.
#include <type_traits>

#include "fine_common.h"
#include "vsa_kernels.h"

namespace vsa {

// bf16 kernel geometry. A workgroup of NW waves owns one query cube; wave
// w owns the 32 queries 32w .. 32w+31 (one MFMA column block). The cube's
// list is walked in 32-key chunks (Bk/32 per key block); each chunk's K and V
// rows go to LDS once (direct-to-LDS loads, 1/NW issued by each wave) and
// all waves read them. MFMAs are 32x32x16.
template <int D> struct FineCfg {
  static constexpr int KS = D / 16;          // k-steps of S^T = K Q^T
  static constexpr int MB = D / 32;          // 32-channel blocks of O^T
  static constexpr int U = D / 8;            // 16-byte units per key row
  static constexpr int KUNITS = 32 * U;      // 16-byte units per K chunk
  static constexpr int VUNITS = 32 * U;      // 16-byte units per V chunk
  static constexpr int KINS = KUNITS / 64;   // 1 KB direct-to-LDS loads per K chunk
  // LDS stages of K and V chunks. D = 128: (3 + 2) x 8 KB = 40 KB, so four
  // workgroups (two waves per SIMD) fit in the 160 KB of LDS of a CU.
  static constexpr int KST = 3;
  static constexpr int VST = D == 64 ? 3 : 2;
};

// Processing order of the Nq query cubes of every (b, h): ascending by the
// first two key blocks of their lists (ids < Nk; empty positions sort last),
// ties by cube id.
// Query cubes with similar lists then run side by side on an XCD and share
// the key / value blocks in its L2. One workgroup per (b, h): a bitonic sort
// of (signature << 32 | cube) keys in LDS.
__global__ __launch_bounds__(1024) void order_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ len,
                                                     int32_t* __restrict__ order, int Nc, int Nk, int stride,
                                                     int pow2) {
  __shared__ unsigned long long key[kMaxSortKeys];
  const long bh = blockIdx.x;
  for (int e = threadIdx.x; e < pow2; e += 1024) {
    unsigned long long kv = ~0ull;
    if (e < Nc) {
      const long row = bh * Nc + e;
      const int n = min(max(len[row], 0), stride);
      const uint32_t a = n > 0 ? (uint32_t)idx[row * stride] : (uint32_t)Nk;
      const uint32_t b = n > 1 ? (uint32_t)idx[row * stride + 1] : (uint32_t)Nk;
      const uint32_t sig = min(a, (uint32_t)Nk) * (uint32_t)(Nk + 1) + min(b, (uint32_t)Nk);
      kv = ((unsigned long long)sig << 32) | (uint32_t)e;
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

// KSAME: key blocks are the query cubes (gk == g), so a key block has NW
// chunks and its geometry is g's, both known at compile time; otherwise the
// key blocks' grid gk is read at run time. Key blocks of 16 tokens are taken
// two per chunk (list entries 2c and 2c + 1; the upper half of the last
// chunk of an odd list repeats the lower block and is masked out of the
// softmax).
//
// At 64 channels a workgroup of two or more waves is held to three waves per
// SIMD (168 registers; the LDS stages allow it): measured 3-9% faster with key
// blocks of their own shape than two waves per SIMD, the same with the cubes as
// key blocks (which fit 168 registers anyway). A one-wave workgroup cannot
// reach three (its stages' LDS) and keeps the 256-register budget.
template <int D, int NW, bool KSAME, bool FUSED>
__global__ __launch_bounds__(64 * NW, (D == 64 && NW >= 2) ? 3 : 2) void fine_fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ len, const int32_t* __restrict__ order,
    bf16* __restrict__ o_f, float* __restrict__ lse_f, const float* __restrict__ oc, const bf16* __restrict__ gc,
    const bf16* __restrict__ gf, bf16* __restrict__ o, Grid g, Grid gk, int stride, float scale_log2) {
  using C = FineCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 kbuf[C::KST * C::KUNITS * 8];
  __shared__ __attribute__((aligned(16))) bf16 vbuf[C::VST * C::VUNITS * 8];

  const int lane = threadIdx.x & 63, n32 = lane & 31, hf = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
  const int slot = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = slot / g.Nc;
  const int i = order != nullptr ? order[slot] : slot - bh * g.Nc;
  const int item = bh * g.Nc + i;
  const long tok0 = (long)bh * g.N;
  const bf16* Q = q + tok0 * D;
  const bf16* K = k + tok0 * D;
  // Lists are validated by contract; the clamps only keep a malformed list
  // from reading outside the tensors.
  const int L = min(max(len[item], 0), stride);
  const int32_t* list = idx + (long)item * stride;
  const Grid& kg = KSAME ? g : gk;   // grid of the key blocks
  auto cube_at = [&](int t) { const int j = list[t]; return (j >= 0 && j < kg.Nc) ? j : 0; };

  // This lane's query: in-cube token 32wv + n32.
  const int qrow = cube_token(g, i, 32 * wv + n32);
  // B operand of S^T = K Q^T: lane holds Q[q][16ks + 8hf .. +8].
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(Q + (long)qrow * D + ks * 16 + hf * 8);

  f32x16 acc[C::MB];
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0.f;
  float m = 0.f, lsum = 0.f;

  // Loads of chunk c = key block list[c >> ksh], chunk h = c & kmask of it
  // (tokens 32h .. 32h+31; 2^ksh = Bk/32 chunks per block): this wave issues
  // 1/NW of the K rows and of the V rows, both into row tiles. Per-lane byte
  // offsets are fixed for the whole list: unit p = ins*64 + lane is key row
  // kappa = p / U, logical unit (p % U) ^ kswz(kappa), i.e. in-block token
  // 32h + kappa.
  const bool kpair = !KSAME && kg.B == 16;   // two 16-token key blocks per chunk
  const int ksh = kpair ? 0 : chunk_shift(kg), kmask = (1 << ksh) - 1;
  const bf16* V = v + tok0 * D;
  constexpr float kSumCap = 65536.0f;
  f32x16 sxa, sxb;
  bf16x8 pfa[2], pfb[2];
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = {(bf16)1.0f, (bf16)1.0f};
  // Bytes of this lane's LDS fragments within a stage: K row fragment ks,
  // and the two transposed reads of V fragment (mb, s2).
  uint32_t koffs[C::KS], voffs[C::MB][2][2];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) koffs[ks] = (n32 * C::U + ((2 * ks + hf) ^ kswz<C::U>(n32))) * 16;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) rowt_offsets<D>(lane, mb, s2, voffs[mb][s2]);
  // The walk of the list through the stages, from its first loads to the O
  // MFMAs of its last chunk. (Written as a lambda, it compiles to 16 fewer
  // registers than the same code inline, and the 720p forward runs 0.8%
  // faster.)
  auto walk = [&]() {
  constexpr int KPW = C::KINS / NW;   // loads per wave per K (or V) chunk
  const uint32_t kbase = lds_addr(kbuf), vbase = lds_addr(vbuf);
  uint32_t koff[KPW];
  row_tile_offsets<D, NW>(kg, wv, lane, koff, kpair ? 15 : 31);
  // Byte offsets of the list's key blocks, 64 entries at a time, one per
  // lane: kcube = first key row of the block within this head's K (and V). A load
  // reads it with readlane, so the per-chunk address work is scalar and
  // division-free. The block of entries is refreshed when the first chunk of
  // entry 64 * n is loaded; K runs ahead of V, so V keeps its own copy.
  uint32_t kcube = 0, vcube = 0;
  auto cubes_k = [&](int t0) {
    const int t = t0 + lane;
    kcube = (uint32_t)cube_first(kg, t < L ? cube_at(t) : 0) * (uint32_t)(D * 2);
  };
  auto cubes_v = [&](int t0) {
    const int t = t0 + lane;
    vcube = (uint32_t)cube_first(kg, t < L ? cube_at(t) : 0) * (uint32_t)(D * 2);
  };
  // Bytes from a key block's first row to the first row of its chunk h.
  auto chunk_bytes = [&](int h) {
    return (KSAME && NW == 1) ? 0u : (uint32_t)(chunk_first(kg, h) * D) * 2u;
  };
  // First list entry of chunk c and the chunk's part h of it.
  auto entry_of = [&](int c, int& e, int& h) {
    if (KSAME) { e = c / NW; h = c % NW; }
    else if (kpair) { e = 2 * c; h = 0; }
    else { e = c >> ksh; h = c & kmask; }
  };
  auto issue_k = [&](int c) {
    int e, h;
    entry_of(c, e, h);
    if ((e & 63) == 0 && h == 0) cubes_k(e);
    const uint32_t dst = kbase + (c % C::KST) * (C::KUNITS * 16);
    const uint32_t kc = __builtin_amdgcn_readlane(kcube, e & 63);
    const void* src = uniform_ptr(reinterpret_cast<const char*>(K) + kc + chunk_bytes(h));
    if (!KSAME && kpair) {   // entries e, e + 1 share a block of 64 (e is even)
      const uint32_t kc1 = __builtin_amdgcn_readlane(kcube, min(e + 1, L - 1) & 63);
      issue_row_tile2<D, NW>(src, uniform_ptr(reinterpret_cast<const char*>(K) + kc1), koff, dst, wv);
      return;
    }
#pragma unroll
    for (int t = 0; t < KPW; ++t) dma16(src, koff[t], dst + (wv * KPW + t) * 1024);
  };
  auto issue_v = [&](int c) {
    int e, h;
    entry_of(c, e, h);
    if ((e & 63) == 0 && h == 0) cubes_v(e);
    const uint32_t dst = vbase + (c % C::VST) * (C::VUNITS * 16);
    const uint32_t vc = __builtin_amdgcn_readlane(vcube, e & 63);
    const void* src = uniform_ptr(reinterpret_cast<const char*>(V) + vc + chunk_bytes(h));
    if (!KSAME && kpair) {
      const uint32_t vc1 = __builtin_amdgcn_readlane(vcube, min(e + 1, L - 1) & 63);
      issue_row_tile2<D, NW>(src, uniform_ptr(reinterpret_cast<const char*>(V) + vc1), koff, dst, wv);
      return;
    }
#pragma unroll
    for (int t = 0; t < KPW; ++t) dma16(src, koff[t], dst + (wv * KPW + t) * 1024);
  };
  // Keys 16-31 of the last chunk of an odd list of 16-token blocks do not
  // exist: their scores (accumulator entries 8-15) are set to -inf.
  const int nch = KSAME ? NW * L : kpair ? (L + 1) >> 1 : L << ksh;
  const bool khalf = !KSAME && kpair && (L & 1);
  auto mask_tail = [&](f32x16& sx, int c) {
    if (!KSAME && khalf && c == nch - 1) {
#pragma unroll
      for (int e = 8; e < 16; ++e) sx[e] = -INFINITY;
    }
  };
  // S^T (32 keys x 32 queries) of the K chunk at kb: lane holds, at
  // accumulator index jj, key 8*(jj/4) + 4hf + jj%4 of the lane's query.
  // All fragments are read first so that LDS latency is paid once.
  auto scores = [&](const bf16* kb) {
    bf16x8 kf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      kf[ks] = *reinterpret_cast<const bf16x8*>(kb + (n32 * C::U + ((2 * ks + hf) ^ kswz<C::U>(n32))) * 8);
    f32x16 sx;
#pragma unroll
    for (int e = 0; e < 16; ++e) sx[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) sx = mfma32_bf16(kf[ks], qf[ks], sx);
    return sx;
  };
  // Three-stage software pipeline over chunks. Step c issues the score MFMAs
  // of chunk c + 2 and the O MFMAs of chunk c (P of chunk c was formed in
  // step c - 1), and between them, one slice per MFMA, forms P of chunk c + 1
  // from its scores (computed in step c - 1). The softmax work then runs in
  // the shadow of all sixteen MFMAs of the step instead of only the score
  // MFMAs, and none of it waits for an MFMA of the same step.
  //
  // K chunks are loaded KST - 1 steps ahead of their scores (step c issues K
  // of c + KST + 1 into the stage that held K of c + 1), V chunks VST - 1
  // steps ahead of their use (step c issues V of c + VST - 1). At its top
  // step c needs K of c + 2 and V of c; loads retire in order, so only the
  // loads issued in step c - 1 for later chunks (K of c + KST and, with three
  // V stages, V of c + 1) may stay in flight. Each wave waits for its own
  // loads, then a barrier (a bare s_barrier: a fenced one would also wait for
  // the loads in flight) makes every wave's share visible and frees the
  // stages about to be refilled (K of c + 1 and V of c - 1, read in step
  // c - 1).
  //
  // Online softmax against a lazily moved reference max m (log2 units): P =
  // 2^(s*c - m) is formed with the current m, and kept when the lane's sum of
  // the chunk's P is at most 2^16 (so every P is, and bf16 P and the fp32
  // sums keep their relative precision). Otherwise (rare: m starts at the row
  // max of chunk 0) m moves up to the chunk's row max, O (which by then holds
  // chunk c) and l are rescaled, and P is formed again. O and l always share
  // m, so the result is exact whatever the schedule.
  // P of a chunk from its scores sx against m, into pf; returns the lane's
  // row sum of the rounded P (the weights O is formed with).
  auto form_p = [&](const f32x16& sx, bf16x8 (&pf)[2]) {
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      pf[e >> 3][e & 7] = (bf16)__builtin_amdgcn_exp2f(sx[e] * scale_log2 - m);
      pf[e >> 3][(e & 7) + 1] = (bf16)__builtin_amdgcn_exp2f(sx[e + 1] * scale_log2 - m);
      const bf16x2 a = {pf[e >> 3][e & 7], pf[e >> 3][(e & 7) + 1]};
      if (e & 2) l1 = __builtin_amdgcn_fdot2_f32_bf16(a, ones2, l1, false);
      else l0 = __builtin_amdgcn_fdot2_f32_bf16(a, ones2, l0, false);
    }
    return l0 + l1;
  };
  // The lazily moved reference max (see above): P of chunk c + 1 was formed
  // from sx into pn with lane sum lc. Returns the sum to add to l.
  auto settle = [&](const f32x16& sx, bf16x8 (&pn)[2], float lc) {
    if (__any(!(lc <= kSumCap))) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sx[e]);
      const float mq = mx * scale_log2 - m;
      const float shift = fmaxf(fmaxf(mq, __shfl_xor(mq, 32, 64)), 0.0f);
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      m += shift;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) acc[mb] *= alpha;
      lc = form_p(sx, pn);
    }
    return lc;
  };
  if (nch > 0) {
    issue_k(0);
#pragma unroll
    for (int c0 = 0; c0 < C::VST - 1; ++c0)
      if (c0 < nch) issue_v(c0);
#pragma unroll
    for (int c0 = 1; c0 < C::KST; ++c0)
      if (c0 < nch) issue_k(c0);
    wait_vmcnt<0>();
  }
  vm_settled();
  if (nch > 0) {
    __builtin_amdgcn_s_barrier();
    f32x16 s0 = scores(kbuf);
    if (nch > 1) sxa = scores(kbuf + C::KUNITS * 8);
    mask_tail(s0, 0);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s0[e]);
    m = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    lsum = form_p(s0, pfa);
    // K of chunk KST goes into stage 0, which every wave read for S of chunk 0.
    if (NW > 1) __builtin_amdgcn_s_barrier();
    if (C::KST < nch) issue_k(C::KST);
  }
  const char* kbytes = reinterpret_cast<const char*>(kbuf);
  const char* vbytes = reinterpret_cast<const char*>(vbuf);

  // The top of step c: wait for this wave's loads of K of c + 2 and V of c,
  // barrier, then issue the step's loads.
  auto step_top = [&](int c) {
    if (c > 0) {
      const bool kin = c + C::KST < nch;
      const bool vin = C::VST >= 3 && c + C::VST - 2 < nch;
      if (kin && vin) wait_vmcnt<2 * KPW>();
      else if (kin || vin) wait_vmcnt<KPW>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
    }
    if (c + C::VST - 1 < nch) issue_v(c + C::VST - 1);
    if (c + C::KST + 1 < nch) issue_k(c + C::KST + 1);
  };
  // One step with chunks c + 1 and c + 2 in the list; P is its position in
  // the 6-step unrolled block (6 is a multiple of both stage counts, so every
  // stage is a constant and every LDS address a per-lane register plus an
  // immediate). sx: scores of chunk c + 1, sn: receives those of c + 2, pc:
  // P of chunk c, pn: receives P of chunk c + 1.
  static_assert(C::KS == 2 * C::MB, "one O MFMA per score MFMA");
  auto step = [&](auto PP, f32x16& sx, f32x16& sn, bf16x8 (&pc)[2], bf16x8 (&pn)[2], int c) {
    constexpr int p = decltype(PP)::value;
    step_top(c);
    mask_tail(sx, c + 1);
    constexpr uint32_t kst = ((p + 2) % C::KST) * C::KUNITS * 16, vst = (p % C::VST) * C::VUNITS * 16;
    // Slot j: score MFMA j/2 (even j) or O MFMA j/2 (odd j), then 16/NSLOT
    // exponentials of chunk c + 1 (pairs rounded to bf16 and summed). Each
    // slot's LDS fragment is read LA slots ahead, so that few are live.
    constexpr int NSLOT = 2 * C::KS, PER = 16 / NSLOT, LA = 3;
    bf16x8 kf[C::KS], vf[C::MB][2];
    auto fetch = [&](int j) {
      if (j % 2 == 0) {
        kf[j / 2] = *reinterpret_cast<const bf16x8*>(kbytes + kst + koffs[j / 2]);
      } else {
        const int t = j / 2, s2 = t / C::MB, mb = t % C::MB;
        vf[mb][s2] = rowt_frag(vbytes + vst, voffs[mb][s2][0], voffs[mb][s2][1]);
      }
    };
#pragma unroll
    for (int j = 0; j < LA; ++j) fetch(j);
#pragma unroll
    for (int e = 0; e < 16; ++e) sn[e] = 0.f;
    __builtin_amdgcn_sched_barrier(0);
    float l0 = 0.f, l1 = 0.f, pend = 0.f;
#pragma unroll
    for (int j = 0; j < NSLOT; ++j) {
      if (j + LA < NSLOT) fetch(j + LA);
      if (j % 2 == 0) {
        sn = mfma32_bf16(kf[j / 2], qf[j / 2], sn);
      } else {
        const int t = j / 2, s2 = t / C::MB, mb = t % C::MB;
        acc[mb] = mfma32_bf16(vf[mb][s2], pc[s2], acc[mb]);
      }
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int e = j * PER + r;
        const float x = __builtin_amdgcn_exp2f(sx[e] * scale_log2 - m);
        if (e % 2 == 0) {
          pend = x;
        } else {
          pn[e >> 3][(e & 7) - 1] = (bf16)pend;
          pn[e >> 3][e & 7] = (bf16)x;
          const bf16x2 a = {pn[e >> 3][(e & 7) - 1], pn[e >> 3][e & 7]};
          if (e & 2) l1 = __builtin_amdgcn_fdot2_f32_bf16(a, ones2, l1, false);
          else l0 = __builtin_amdgcn_fdot2_f32_bf16(a, ones2, l0, false);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lsum += settle(sx, pn, l0 + l1);
  };
  // One of the last two steps (no chunk c + 2; chunk c + 1 when more): the
  // O MFMAs of chunk c from the V stage of c, known only at run time here.
  auto tail = [&](f32x16& sx, bf16x8 (&pc)[2], bf16x8 (&pn)[2], int c) {
    step_top(c);
    const char* vb = vbytes + (c % C::VST) * (C::VUNITS * 16);
    bf16x8 vf[C::MB][2];
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) vf[mb][s2] = rowt_frag(vb, voffs[mb][s2][0], voffs[mb][s2][1]);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mb = 0; mb < C::MB; ++mb) acc[mb] = mfma32_bf16(vf[mb][s2], pc[s2], acc[mb]);
    if (c + 1 < nch) {
      mask_tail(sx, c + 1);
      lsum += settle(sx, pn, form_p(sx, pn));
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  static_assert(6 % C::KST == 0 && 6 % C::VST == 0, "stages must divide the unroll");
  const int nfull = nch - 2;   // steps with chunks c + 1 and c + 2
  int c = 0;
  for (; c + 6 <= nfull; c += 6) {
    step(I0(), sxa, sxb, pfa, pfb, c);
    step(I1(), sxb, sxa, pfb, pfa, c + 1);
    step(I2(), sxa, sxb, pfa, pfb, c + 2);
    step(I3(), sxb, sxa, pfb, pfa, c + 3);
    step(I4(), sxa, sxb, pfa, pfb, c + 4);
    step(I5(), sxb, sxa, pfb, pfa, c + 5);
  }
  if (c < nfull) {
    step(I0(), sxa, sxb, pfa, pfb, c);
    if (c + 1 < nfull) {
      step(I1(), sxb, sxa, pfb, pfa, c + 1);
      if (c + 2 < nfull) {
        step(I2(), sxa, sxb, pfa, pfb, c + 2);
        if (c + 3 < nfull) {
          step(I3(), sxb, sxa, pfb, pfa, c + 3);
          if (c + 4 < nfull) step(I4(), sxa, sxb, pfa, pfb, c + 4);
        }
      }
    }
  }
  for (c = nfull > 0 ? nfull : 0; c < nch; ++c) {
    if (c & 1) tail(sxb, pfb, pfa, c);
    else tail(sxa, pfa, pfb, c);
  }
  };
  walk();

  // Epilogue: lane holds O^T[channel 32mb + 8(jj/4) + 4hf + jj%4][its query].
  const float lt = lsum + __shfl_xor(lsum, 32, 64);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const long n = tok0 + qrow;
  if (lse_f != nullptr && hf == 0) lse_f[n] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  // The normalised O goes through LDS so that every global access of the
  // epilogue is a whole 16-byte unit of a token row, whole rows per
  // instruction. Written from the accumulator layout (lane: one query, four
  // channels per fragment) and read back by rows, each a plain copy of 32
  // token rows; the rounding to bf16 is the one O_f gets when it is stored.
  // A wave uses the chunk stage of its own index (one stage holds 32 rows of
  // D channels), once every wave is done with the stages.
  constexpr int RPI = 64 / C::U, NIT = 32 / RPI;   // token rows per instruction, instructions per tile
  const int u = lane % C::U, r0 = lane / C::U;      // this lane's unit (channels 8u .. 8u+7) and first row
  long nrow[NIT];
#pragma unroll
  for (int t = 0; t < NIT; ++t) nrow[t] = (tok0 + cube_token(g, i, 32 * wv + t * RPI + r0)) * D + u * 8;
  bf16* tile = wv < C::KST ? kbuf + wv * (C::KUNITS * 8) : vbuf + (wv - C::KST) * (C::VUNITS * 8);
  auto stage_o = [&](bf16x8 (&ofv)[NIT]) {
    // Every wave is past its last read of the chunk stages (each read was
    // consumed by an MFMA before the wave left the loop, and no chunk load is
    // in flight), so a bare barrier frees them; loads the caller issued
    // before it (the gates) stay in flight.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (bf16)(acc[mb][4 * jq + r] * inv);
        *reinterpret_cast<bf16x4*>(tile + (n32 * C::U + ((4 * mb + jq) ^ kswz<C::U>(n32))) * 8 + 4 * hf) = w;
      }
#pragma unroll
    for (int t = 0; t < NIT; ++t) {
      const int row = t * RPI + r0;
      ofv[t] = *reinterpret_cast<const bf16x8*>(tile + (row * C::U + (u ^ kswz<C::U>(row))) * 8);
    }
    if (o_f != nullptr) {
#pragma unroll
      for (int t = 0; t < NIT; ++t) __builtin_nontemporal_store(ofv[t], reinterpret_cast<bf16x8*>(o_f + nrow[t]));
    }
  };
  if constexpr (!FUSED) {
    bf16x8 ofv[NIT];
    stage_o(ofv);
  } else {
    // The gated combine, O_f taken as rounded to bf16 (so the fused output
    // equals the unfused combine of the stored O_f). Which gates exist is
    // decided outside the loops, and O_c and the gates are loaded before O
    // is staged, so that their latency overlaps the staging.
    auto combine = [&](auto HC, auto HF) {
      constexpr bool kHC = decltype(HC)::value, kHF = decltype(HF)::value;
      const float4* ocr = reinterpret_cast<const float4*>(oc + ((long)bh * g.Nc + i) * D + u * 8);
      const float4 oa = ocr[0], ob = ocr[1];
      bf16x8 gcv[NIT], gfv[NIT];
#pragma unroll
      for (int t = 0; t < NIT; ++t) {
        if (kHC) gcv[t] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(gc + nrow[t]));
        if (kHF) gfv[t] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(gf + nrow[t]));
      }
      bf16x8 ofv[NIT];
      stage_o(ofv);
      const float cv[8] = {oa.x, oa.y, oa.z, oa.w, ob.x, ob.y, ob.z, ob.w};
#pragma unroll
      for (int t = 0; t < NIT; ++t) {
        bf16x8 w;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float a = kHC ? (float)gcv[t][r] : 1.f;
          const float b = kHF ? (float)gfv[t][r] : 1.f;
          w[r] = (bf16)(cv[r] * a + (float)ofv[t][r] * b);
        }
        __builtin_nontemporal_store(w, reinterpret_cast<bf16x8*>(o + nrow[t]));
      }
    };
    using T1 = std::true_type;
    using F0 = std::false_type;
    if (gc != nullptr && gf != nullptr) combine(T1(), T1());
    else if (gc != nullptr) combine(T1(), F0());
    else if (gf != nullptr) combine(F0(), T1());
    else combine(F0(), F0());
  }
}

// fp32 path: one thread per query token (a workgroup of Bt threads per query
// cube), K/V rows staged in LDS 32 at a time. Used for fp32 problems (small,
// correctness-first shapes).
template <int D, bool FUSED>
__global__ __launch_bounds__(128) void fine_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ len, float* __restrict__ o_f,
    float* __restrict__ lse_f, const float* __restrict__ oc, const float* __restrict__ gc,
    const float* __restrict__ gf, float* __restrict__ o, Grid g, Grid gk, int stride, float scale) {
  constexpr int R = 32;   // key rows per LDS stage
  __shared__ float ks[R][D];
  __shared__ float vs[R][D];
  const int tid = threadIdx.x, nt = blockDim.x;
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

template <int D, int NW, bool FUSED>
static void fine_launch_bf16_nw(const Launch& L, const void* q, const void* k, const void* v, const int32_t* idx,
                                const int32_t* len, const int32_t* order, void* o_f, float* lse_f, const float* oc,
                                const void* gc, const void* gf, void* o) {
  const int nitems = L.BH * L.g.Nc;
  const bool same = L.g.B == L.gk.B && L.g.lct == L.gk.lct && L.g.lch == L.gk.lch;
  if (same)
    hipLaunchKernelGGL((fine_fwd_bf16_kernel<D, NW, true, FUSED>), dim3(nitems), dim3(64 * NW), 0, L.stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, idx, len, order, (bf16*)o_f, lse_f, oc,
                       (const bf16*)gc, (const bf16*)gf, (bf16*)o, L.g, L.gk, L.stride, L.scale * kLog2e);
  else
    hipLaunchKernelGGL((fine_fwd_bf16_kernel<D, NW, false, FUSED>), dim3(nitems), dim3(64 * NW), 0, L.stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, idx, len, order, (bf16*)o_f, lse_f, oc,
                       (const bf16*)gc, (const bf16*)gf, (bf16*)o, L.g, L.gk, L.stride, L.scale * kLog2e);
}

// Waves per workgroup = cube tokens / 32 (32, 64 or 128 tokens).
template <int D, bool FUSED>
static void fine_launch_bf16(const Launch& L, const void* q, const void* k, const void* v, const int32_t* idx,
                             const int32_t* len, const int32_t* order, void* o_f, float* lse_f, const float* oc, const void* gc,
                             const void* gf, void* o) {
  if (L.g.B == 32) fine_launch_bf16_nw<D, 1, FUSED>(L, q, k, v, idx, len, order, o_f, lse_f, oc, gc, gf, o);
  else if (L.g.B == 128) fine_launch_bf16_nw<D, 4, FUSED>(L, q, k, v, idx, len, order, o_f, lse_f, oc, gc, gf, o);
  else fine_launch_bf16_nw<D, 2, FUSED>(L, q, k, v, idx, len, order, o_f, lse_f, oc, gc, gf, o);
}

template <int D, bool FUSED>
static void fine_launch_f32(const Launch& L, const void* q, const void* k, const void* v, const int32_t* idx,
                            const int32_t* len, void* o_f, float* lse_f, const float* oc, const void* gc,
                            const void* gf, void* o) {
  const int nitems = L.BH * L.g.Nc;
  hipLaunchKernelGGL((fine_fwd_f32_kernel<D, FUSED>), dim3(nitems), dim3(L.g.B), 0, L.stream, (const float*)q,
                     (const float*)k, (const float*)v, idx, len, (float*)o_f, lse_f, oc, (const float*)gc,
                     (const float*)gf, (float*)o, L.g, L.gk, L.stride, L.scale);
}

hipError_t launch_order(const Launch& L, const int32_t* idx, const int32_t* len, int32_t* order) {
  int pow2 = 1;
  while (pow2 < L.g.Nc) pow2 <<= 1;
  if (pow2 > kMaxSortKeys) return hipErrorInvalidValue;
  hipLaunchKernelGGL(order_kernel, dim3(L.BH), dim3(1024), 0, L.stream, idx, len, order, L.g.Nc, L.gk.Nc, L.stride,
                     pow2);
  return hipGetLastError();
}

hipError_t launch_fine_fwd(const Launch& L, const void* q, const void* k, const void* v, const int32_t* idx, const int32_t* len, const int32_t* order, void* o_f, float* lse_f,
                           const float* oc, const void* g_c, const void* g_f, void* o) {
  const bool fused = oc != nullptr;
  if (L.bf16) {
    if (L.D == 64) {
      if (fused) fine_launch_bf16<64, true>(L, q, k, v, idx, len, order, o_f, lse_f, oc, g_c, g_f, o);
      else fine_launch_bf16<64, false>(L, q, k, v, idx, len, order, o_f, lse_f, oc, g_c, g_f, o);
    } else {
      if (fused) fine_launch_bf16<128, true>(L, q, k, v, idx, len, order, o_f, lse_f, oc, g_c, g_f, o);
      else fine_launch_bf16<128, false>(L, q, k, v, idx, len, order, o_f, lse_f, oc, g_c, g_f, o);
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
