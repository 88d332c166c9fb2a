// Device helpers shared by the fine-stage kernels (forward and backward):
// direct-to-LDS loads of 32-token chunks, and the LDS layouts they fill.
//
// A chunk is tokens 32h .. 32h+31 of a cube in cube order (a cube of Bt
// tokens has Bt/32 chunks). In LDS a chunk of one tensor (D channels) is a
// row tile: 32 token rows of U = D/8 16-byte units; row kappa is in-cube token
// 32h + kappa, and its logical unit u (channels 8u .. 8u+7) sits at unit
// u ^ kswz(kappa), which spreads the tile's readers over the LDS banks. It
// is loaded from the token tensor, read directly as the A operand of a
// 32x32x16 MFMA (rows = tokens, k = channels) and, by LDS transpose reads,
// as the A operand with k = tokens (rows = channels).
#pragma once

#include "vsa_common.h"

namespace vsa {

template <int D> struct ChunkGeom {
  static constexpr int KS = D / 16;          // k-steps over channels
  static constexpr int MB = D / 32;          // 32-channel blocks
  static constexpr int U = D / 8;            // 16-byte units per token row
  static constexpr int RUNITS = 32 * U;      // 16-byte units per row tile
  static constexpr int RINS = RUNITS / 64;   // 1 KB loads per row tile
};

// The unit swizzle of row kappa: an XOR mask linear in kappa's low four bits,
// chosen (by an exhaustive search over such masks against a model of the LDS
// banks) so that both readers of a row tile are free of bank conflicts: the
// 16-byte row reads (16 consecutive rows at one logical unit) and the
// transpose reads (8 rows x 4 consecutive units per instruction).
template <int U> __device__ __forceinline__ int kswz(int kappa) {
  static_assert(U == 8 || U == 16, "row tiles of 64 or 128 channels");
  const int b0 = kappa & 1, b1 = (kappa >> 1) & 1, b2 = (kappa >> 2) & 1, b3 = (kappa >> 3) & 1;
  if (U == 16) return (b0 * 4) ^ (b1 * 10) ^ b2 ^ (b3 * 2);
  return (b0 * 2) ^ (b1 * 4) ^ b2 ^ (b3 * 2);
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes land at LDS byte
// address lds + 16*l. Issued as inline assembly so that the compiler does not
// treat later LDS reads of other stages as dependent on it; completion is
// tracked by the vector-memory counter and waited for explicitly (wait_vmcnt).
// M0 is a register the compiler reserves, so it cannot be declared clobbered;
// the build (build.py, check_m0) inspects the generated assembly of every
// kernel that issues these loads and fails if the compiler uses M0 anywhere
// else in it, so nothing can depend on M0 across this statement.
// The address is a wave-uniform base (SGPRs) plus a per-lane 32-bit byte
// offset, so issuing a load costs no vector instructions.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
// A pointer the compiler may keep in scalar registers (all lanes agree).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const unsigned long long b = (unsigned long long)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return (const void*)(((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A wait for all vector-memory loads that the compiler itself sees. Its count
// of outstanding loads ignores the direct-to-LDS loads above (inline
// assembly), and where it cannot prove that registers loaded earlier (a
// wave's Q fragments, say) have arrived it waits for them before their next
// use, with counts that then also drain the direct-to-LDS loads in flight.
// Placed where every load has already been waited for, this costs nothing and
// marks those registers as arrived for the code that follows.
__device__ __forceinline__ void vm_settled() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Per-lane byte offsets (within a chunk) of wave wv's share of a row tile's
// loads when NW waves share them: load t of the wave is unit
// p = (wv*RINS/NW + t)*64 + lane. With rmask = 15 the chunk is two 16-token
// blocks (rows 0-15 and 16-31, each load within one of them) and offsets are
// taken from the first row of the row's own block.
template <int D, int NW> __device__ __forceinline__ void row_tile_offsets(const Grid& g, int wv, int lane,
                                                                          uint32_t* off, int rmask = 31) {
  using G = ChunkGeom<D>;
  static_assert(G::RINS % NW == 0, "every wave issues whole 1 KB loads");
#pragma unroll
  for (int t = 0; t < G::RINS / NW; ++t) {
    const int p = (wv * (G::RINS / NW) + t) * 64 + lane, kappa = p / G::U;
    const int u = (p % G::U) ^ kswz<G::U>(kappa);
    off[t] = (uint32_t)(chunk_row(g, kappa & rmask) * D + u * 8) * 2u;
  }
}
// Whether load t of wave wv (NW waves sharing a row tile) fills rows 16-31
// (a load covers 64 / U consecutive rows, never both halves).
template <int D, int NW> __device__ __forceinline__ bool row_tile_upper(int wv, int t) {
  using G = ChunkGeom<D>;
  return (wv * (G::RINS / NW) + t) * 64 / G::U >= 16;
}
// Issue wave wv's share of a row tile: src = first row of the chunk, dst =
// LDS byte address of the tile.
template <int D, int NW> __device__ __forceinline__ void issue_row_tile(const void* src, const uint32_t* off,
                                                                       uint32_t dst, int wv) {
  using G = ChunkGeom<D>;
#pragma unroll
  for (int t = 0; t < G::RINS / NW; ++t) dma16(src, off[t], dst + (wv * (G::RINS / NW) + t) * 1024);
}
// The same for a chunk made of two 16-token blocks: rows 0-15 from srcA,
// rows 16-31 from srcB (offsets from row_tile_offsets with rmask = 15).
template <int D, int NW> __device__ __forceinline__ void issue_row_tile2(const void* srcA, const void* srcB,
                                                                        const uint32_t* off, uint32_t dst, int wv) {
  using G = ChunkGeom<D>;
#pragma unroll
  for (int t = 0; t < G::RINS / NW; ++t)
    dma16(row_tile_upper<D, NW>(wv, t) ? srcB : srcA, off[t], dst + (wv * (G::RINS / NW) + t) * 1024);
}
// A operand fragment of a row tile (rows = tokens, k-step ks over channels).
template <int D> __device__ __forceinline__ bf16x8 row_frag(const bf16* tile, int n32, int hf, int ks) {
  using G = ChunkGeom<D>;
  return *reinterpret_cast<const bf16x8*>(tile + (n32 * G::U + ((2 * ks + hf) ^ kswz<G::U>(n32))) * 8);
}
// Transposed A fragments straight from a row tile, by the LDS transpose read
// ds_read_b64_tr_b16. Within each group of 16 lanes, that read hands output
// lane t the element t % 4 of the 8 bytes source lane 4e + t / 4 addressed,
// as its element e. So if source lane 4e + j reads row r0 + e at channels
// c0 + 4j .. +3, output lane t receives channel c0 + t of rows r0 .. r0 + 3.
// For the A operand of O^T-style products (A[m = channel 32mb + lane%32][k =
// slot 16s2 + 8hf + e], whose B operand is a 32x32 accumulator), slot e of
// lane half hf must hold row 16s2 + 8(e/4) + 4hf + e%4 (the order in which a
// 32x32 accumulator holds its rows): two reads, rows 16s2 + 4hf + 0..3 and
// 16s2 + 8 + 4hf + 0..3. rowt_offsets gives each lane's two byte offsets
// (within a tile) for fragment (mb, s2); rowt_frag performs the reads.
typedef short tr16x4 __attribute__((ext_vector_type(4)));
template <int D> __device__ __forceinline__ void rowt_offsets(int lane, int mb, int s2, uint32_t off[2]) {
  using G = ChunkGeom<D>;
  const int g16 = lane >> 4, s = lane & 15, e = s >> 2, j = s & 3;
  const int hf = g16 >> 1, ch = 32 * mb + 16 * (g16 & 1) + 4 * j;
  const int u = ch >> 3, within = (ch & 7) * 2;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = 16 * s2 + 8 * half + 4 * hf + e;
    off[half] = (uint32_t)((r * G::U + (u ^ kswz<G::U>(r))) * 16 + within);
  }
}
__device__ __forceinline__ bf16x8 rowt_frag(const char* tile, uint32_t off0, uint32_t off1) {
  typedef __attribute__((address_space(3))) tr16x4 lds_tr;
  const tr16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr*)(tile + off0));
  const tr16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr*)(tile + off1));
  const tr16x4 v[2] = {a, b};
  bf16x8 r;
  __builtin_memcpy(&r, v, sizeof(r));
  return r;
}

}  // namespace vsa
