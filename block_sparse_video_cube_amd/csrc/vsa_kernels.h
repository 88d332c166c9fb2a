// Internal launchers of the VSA HIP kernels (not part of the C ABI).
#pragma once

#include "vsa_common.h"

namespace vsa {

// Launch context shared by the launchers: one problem, one stream.
struct Launch {
  Grid g;          // query cubes (and every per-token or per-query-cube array)
  Grid gk;         // key blocks (K, V and their pooled values); equal to g unless
                   // the problem gives key blocks their own shape
  int BH;          // B * heads
  int D;           // head_dim (64 or 128)
  bool bf16;       // dtype of raster tensors
  float scale;     // softmax scale (resolved, > 0)
  int topk;        // > 0: top-K mode
  int stride;      // idx row stride
  bool pool_max;   // max pooling instead of mean (the ablation variant)
  hipStream_t stream;
};

// Pooled q (query cubes) and k, v (key blocks), fp32, each may be null = not
// written; with max pooling, the in-cube index of each (cube, channel)
// maximum (args: q, k, v planes of B*heads*Nq*D, B*heads*Nk*D and
// B*heads*Nk*D bytes; may be null).
hipError_t launch_pool(const Launch& L, const void* q, const void* k, const void* v, float* qc, float* kc,
                       float* vc, uint8_t* args = nullptr);

// Raster <-> cube-major copy of one token tensor (D channels, problem dtype).
hipError_t launch_relayout(const Launch& L, const void* src, void* dst, bool to_tiled);
hipError_t launch_crop_pad(const Launch& L, const void* src, void* dst, int ts, int hs, int ws, bool to_small);

// 256-token tiles as 128-token halves (half_grid): S is L with g and / or
// gk replaced by their half grids and stride doubled when key blocks are
// split. Lists of the query halves (idx2 [BH, S.g.Nc, S.stride], len2) from
// the cubes' lists; per-half copies of per-cube rows (D fp32 values, times
// mul; either of src / asrc may be null) and max-pool argmax bytes.
hipError_t launch_split_lists(const Launch& L, const Launch& S, const int32_t* idx, const int32_t* len, int32_t* idx2,
                              int32_t* len2);
hipError_t launch_split_rows(const Launch& L, const Grid& g, const Grid& g2, const float* src, float* dst,
                             const uint8_t* asrc, uint8_t* adst, float mul);

int coarse_max_cubes();
// Keys of the bitonic order sorts (one workgroup per (b, h), keys in LDS):
// the largest cube or key-block count per (b, h).
constexpr int kMaxSortKeys = 8192;
// Row pitch (floats) of the coarse logits: Nk rounded up to a multiple of 4.
int coarse_ld(int Nk);
// s_scratch: B*heads*Nq*coarse_ld(Nk) fp32 (the coarse logits).
hipError_t launch_coarse(const Launch& L, const float* qc, const float* kc, const float* vc, float* oc,
                         float* lse, int32_t* idx, int32_t* len, float* s_scratch);

// Processing order of query cubes (BH*Nq int32) from their lists.
hipError_t launch_order(const Launch& L, const int32_t* idx, const int32_t* len, int32_t* order);

// Fine forward. For bf16, `order` (may be null = cube order) is the
// processing order from launch_order. When oc is not null the kernel also
// forms o = O_c * g_c + O_f * g_f (gates may be null = ones) and writes it to
// `o`; o_f / lse_f may then be null (not written).
hipError_t launch_fine_fwd(const Launch& L, const void* q, const void* k, const void* v, const int32_t* idx,
                           const int32_t* len, const int32_t* order, void* o_f, float* lse_f,
                           const float* oc, const void* g_c, const void* g_f, void* o);

hipError_t launch_combine(const Launch& L, const float* oc, const void* of, const void* gc, const void* gf,
                          void* o);
hipError_t launch_combine_bwd(const Launch& L, const void* d_o, const float* oc, const void* of,
                              const void* gc, const void* gf, void* dgc, void* dgf, void* dof,
                              float* delta, float* doc);

// bits: B*heads*Nk*k2q_bits_words(Nq) uint32 of scratch; k2q_off has
// B*heads*(Nk+1) entries, k2q B*heads*Nq*stride.
int k2q_bits_words(int Nq);
hipError_t launch_index_transpose(const Launch& L, const int32_t* idx, const int32_t* len, int32_t* k2q_off,
                                  int32_t* k2q, uint32_t* bits);
// Scratch: ds / p B*heads*Nq*coarse_ld(Nk) fp32, dc B*heads*Nq fp32.
hipError_t launch_coarse_bwd(const Launch& L, const float* qc, const float* kc, const float* vc,
                             const float* oc, const float* lse, const float* doc, float* dqc, float* dkc,
                             float* dvc, float* ds_scratch, float* p_scratch, float* dc_scratch);
// Key blocks of every (b, h) (BH*Nk int32) ordered by descending
// transposed-list length.
hipError_t launch_order_by_count(const Launch& L, const int32_t* k2q_off, int32_t* order);
// Union lists of pairs of 16-token key blocks (2P, 2P + 1) from the
// transposed lists: pair P's entries at k2u[bh][k2q_off[bh][2P] ...], count
// in plen[bh][P]; each entry a query cube with bit 24 (listed by block 2P)
// and bit 25 (by 2P + 1). k2u: B*heads*Nq*stride, plen: B*heads*ceil(Nk/2).
hipError_t launch_key_pairs(const Launch& L, const int32_t* k2q_off, const int32_t* k2q, int32_t* k2u,
                            int32_t* plen);
// Fine backward: dq over the forward lists (qorder from launch_order, may be
// null), dk / dv over the transposed lists (korder from
// launch_order_by_count, may be null); token tensors in the problem's dtype
// (bf16: MFMA kernels; fp32: one thread per token). The pooled gradients dqc
// / dkc / dvc are spread over their cubes (mean pooling), or go to the maxima
// given by args (max pooling; layout of launch_pool's args). With 16-token
// key blocks and bf16, `pairs` is scratch for launch_key_pairs (k2u, then
// plen), else unused.
hipError_t launch_fine_bwd(const Launch& L, const void* q, const void* k, const void* v, const int32_t* idx,
                           const int32_t* len, const int32_t* qorder, const int32_t* k2q_off, const int32_t* k2q,
                           const int32_t* korder, const float* lse_f, const void* dof, const float* delta,
                           const float* dqc, const float* dkc, const float* dvc, void* dq, void* dk, void* dv,
                           const uint8_t* args, int32_t* pairs);

hipError_t launch_validate_lists(const Launch& L, const int32_t* idx, const int32_t* len, int32_t* flag);

}  // namespace vsa
