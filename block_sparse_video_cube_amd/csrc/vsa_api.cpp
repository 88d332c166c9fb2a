// C ABI of the VSA operator: validation, buffer layouts, kernel sequencing.
// Declarations and contracts: include/vsa.h.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/vsa.h"
#include "vsa_kernels.h"

using namespace vsa;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Dims {
  long BH, N, Nq, Nk, Bk, D, stride;   // Nq query cubes, Nk key blocks of Bk tokens per (b, h)
  size_t elem;  // bytes per raster element
  // The fine kernels' view (256-token cubes / key blocks as 128-token halves):
  bool qsplit, ksplit;
  long Nq2, Nk2, stride2;
};

// A cube side: a power of two in [1, 128].
inline bool pow2_side(int v) { return v > 0 && v <= 128 && (v & (v - 1)) == 0; }

// Host-side validation of the problem; fills the launch context.
vsa_status check_problem(const vsa_problem* p, Launch* L, Dims* d) {
  if (p == nullptr) return VSA_ERR_NULL;
  if (p->B < 1 || p->heads < 1) return VSA_ERR_SHAPE;
  const int ct = p->cube_t ? p->cube_t : 4, ch = p->cube_h ? p->cube_h : 4, cw = p->cube_w ? p->cube_w : 4;
  const bool kown = p->kcube_t || p->kcube_h || p->kcube_w;   // key blocks of their own shape
  const int kt = kown ? p->kcube_t : ct, kh = kown ? p->kcube_h : ch, kw = kown ? p->kcube_w : cw;
  for (int side : {ct, ch, cw, kt, kh, kw})
    if (!pow2_side(side)) return VSA_ERR_SHAPE;
  if (cw < 4 || kw < 4) return VSA_ERR_SHAPE;
  if (p->T < ct || p->H < ch || p->W < cw || p->T % ct || p->H % ch || p->W % cw) return VSA_ERR_SHAPE;
  if (p->T % kt || p->H % kh || p->W % kw) return VSA_ERR_SHAPE;
  const long Bt = (long)ct * ch * cw, Bk = (long)kt * kh * kw;
  if (Bt != 32 && Bt != 64 && Bt != 128 && Bt != 256) return VSA_ERR_UNSUPPORTED;
  if (Bk != 16 && Bk != 32 && Bk != 64 && Bk != 128 && Bk != 256) return VSA_ERR_UNSUPPORTED;
  const bool same = kt == ct && kh == ch && kw == cw;
  const long N = (long)p->T * p->H * p->W;
  const long BH = (long)p->B * p->heads;
  if (N > (1L << 30) || BH > (1L << 24)) return VSA_ERR_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return VSA_ERR_HEAD_DIM;
  if (p->dtype != VSA_F32 && p->dtype != VSA_BF16) return VSA_ERR_DTYPE;
  const long Nc = N / Bt, Nk = N / Bk;
  if (BH * (Nc > Nk ? Nc : Nk) > 0x7fffffffL) return VSA_ERR_SHAPE;
  if (BH * N * p->head_dim > (1L << 40)) return VSA_ERR_SHAPE;
  if (!std::isfinite(p->scale) || p->scale < 0.f) return VSA_ERR_SCALE;
  if (p->topk < 0 || p->topk > Nk) return VSA_ERR_TOPK;
  const long stride = p->list_stride == 0 ? p->topk : p->list_stride;
  if (p->topk > 0 && stride < p->topk) return VSA_ERR_TOPK;
  if (stride < 1 || stride > Nk) return VSA_ERR_TOPK;
  if (Nc > coarse_max_cubes() || Nk > coarse_max_cubes()) return VSA_ERR_UNSUPPORTED;
  if (p->pool_mode != VSA_POOL_MEAN && p->pool_mode != VSA_POOL_MAX) return VSA_ERR_UNSUPPORTED;
  if (p->layout != VSA_LAYOUT_RASTER && p->layout != VSA_LAYOUT_TILED) return VSA_ERR_UNSUPPORTED;
  if (p->layout == VSA_LAYOUT_TILED && !same) return VSA_ERR_UNSUPPORTED;   // one cube-major order
  if (L != nullptr) {
    L->g = make_grid(p->T, p->H, p->W, p->layout == VSA_LAYOUT_TILED ? 1 : 0, ct, ch, cw);
    L->gk = make_grid(p->T, p->H, p->W, p->layout == VSA_LAYOUT_TILED ? 1 : 0, kt, kh, kw);
    L->BH = (int)BH;
    L->D = p->head_dim;
    L->bf16 = p->dtype == VSA_BF16;
    L->scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->head_dim);
    L->topk = p->topk;
    L->stride = (int)stride;
    L->pool_max = p->pool_mode == VSA_POOL_MAX;
    L->stream = nullptr;
  }
  if (d != nullptr) {
    d->BH = BH; d->N = N; d->Nq = Nc; d->Nk = Nk; d->Bk = Bk; d->D = p->head_dim; d->stride = stride;
    d->elem = p->dtype == VSA_BF16 ? 2 : 4;
    d->qsplit = Bt == 256;
    d->ksplit = Bk == 256;
    d->Nq2 = d->qsplit ? 2 * Nc : Nc;
    d->Nk2 = d->ksplit ? 2 * Nk : Nk;
    d->stride2 = d->ksplit ? 2 * stride : stride;
  }
  return VSA_OK;
}

// The launch context of the fine kernels: 256-token query cubes and key
// blocks become their 128-token halves (half_grid), lists double with split
// key blocks.
Launch fine_view(const Launch& L) {
  Launch S = L;
  if (L.g.B == 256) S.g = half_grid(L.g);
  if (L.gk.B == 256) {
    S.gk = half_grid(L.gk);
    S.stride = 2 * L.stride;
  }
  return S;
}

inline bool misaligned(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0; }

// Checks a list of (pointer, required) pairs: NULL and alignment.
vsa_status check_ptrs(std::initializer_list<std::pair<const void*, bool>> ptrs) {
  for (const auto& pr : ptrs) {
    if (pr.first == nullptr) {
      if (pr.second) return VSA_ERR_NULL;
      continue;
    }
    if (misaligned(pr.first)) return VSA_ERR_ALIGN;
  }
  return VSA_OK;
}

// ---- buffer layouts (every region 256-byte aligned) -----------------------
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T> T* take(size_t count) {
    T* r = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return r;
  }
};

// Saved for backward: pooled means, O_c, LSE_c, LSE_f, O_f.
struct Saved {
  float *qc, *kc, *vc, *oc, *lse_c, *lse_f;
  void* of;
  size_t bytes;
};
Saved carve_saved(const Dims& d, void* base) {
  Carver c(base);
  Saved s;
  const size_t pq = d.BH * d.Nq * d.D, pk = d.BH * d.Nk * d.D;
  s.qc = c.take<float>(pq);
  s.kc = c.take<float>(pk);
  s.vc = c.take<float>(pk);
  s.oc = c.take<float>(pq);
  s.lse_c = c.take<float>(d.BH * d.Nq);
  s.lse_f = c.take<float>(d.BH * d.N);
  s.of = c.take<char>(d.BH * d.N * d.D * d.elem);
  s.bytes = c.off;
  return s;
}

// Forward workspace: the query-cube order, the coarse logits and, for
// inference, the pooled tensors.
struct FwdWs {
  int32_t* order;
  float *s, *qc, *kc, *vc, *oc, *lse_c;
  int32_t *idx2, *len2;   // lists of the query halves (256-token tiles only)
  float* oc2;             // O_c per query half (256-token query cubes only)
  size_t bytes;
};
FwdWs carve_fwd_ws(const Dims& d, void* base) {
  Carver c(base);
  FwdWs w;
  w.order = c.take<int32_t>(d.BH * d.Nq2);
  const bool split = d.qsplit || d.ksplit;
  w.idx2 = split ? c.take<int32_t>(d.BH * d.Nq2 * d.stride2) : nullptr;
  w.len2 = split ? c.take<int32_t>(d.BH * d.Nq2) : nullptr;
  w.oc2 = d.qsplit ? c.take<float>(d.BH * d.Nq2 * d.D) : nullptr;
  w.s = c.take<float>(d.BH * d.Nq * (size_t)coarse_ld((int)d.Nk));
  const size_t pq = d.BH * d.Nq * d.D, pk = d.BH * d.Nk * d.D;
  w.qc = c.take<float>(pq);
  w.kc = c.take<float>(pk);
  w.vc = c.take<float>(pk);
  w.oc = c.take<float>(pq);
  w.lse_c = c.take<float>(d.BH * d.Nq);
  w.bytes = c.off;
  return w;
}

// Backward workspace.
struct BwdWs {
  void* dof;   // d_o_f, in the problem's dtype
  float *delta, *doc, *dqc, *dkc, *dvc, *p_scr, *ds_scr, *dc_scr;
  int32_t *k2q_off, *k2q, *qorder, *korder;
  int32_t* pairs;   // 16-token key blocks: union lists of block pairs and their lengths
  uint32_t* k2q_bits;
  uint8_t* args;   // max pooling: argmax positions of q, k, v
  // 256-token tiles: lists of the query halves, pooled gradients and argmax
  // positions per half (null where a side is not split)
  int32_t *idx2, *len2;
  float *dqc2, *dkc2, *dvc2;
  uint8_t* args2;
  size_t bytes;
};
BwdWs carve_bwd_ws(const Dims& d, void* base) {
  Carver c(base);
  BwdWs w;
  const size_t rast = d.BH * d.N * d.D;
  w.dof = c.take<char>(rast * d.elem);
  w.delta = c.take<float>(d.BH * d.N);
  const size_t pq = d.BH * d.Nq * d.D, pk = d.BH * d.Nk * d.D;
  w.doc = c.take<float>(pq);
  w.dqc = c.take<float>(pq);
  w.dkc = c.take<float>(pk);
  w.dvc = c.take<float>(pk);
  const size_t ldc = (size_t)coarse_ld((int)d.Nk);
  w.p_scr = c.take<float>(d.BH * d.Nq * ldc);
  w.ds_scr = c.take<float>(d.BH * d.Nq * ldc);
  w.dc_scr = c.take<float>(d.BH * d.Nq);
  // Transposed lists, orders and pairs are sized for the fine kernels' view
  // (at least the cubes' own sizes, which vsa_index_transpose uses).
  w.k2q_off = c.take<int32_t>(d.BH * (d.Nk2 + 1));
  w.k2q = c.take<int32_t>(d.BH * d.Nq2 * d.stride2);
  w.k2q_bits = c.take<uint32_t>(d.BH * d.Nk2 * (size_t)k2q_bits_words((int)d.Nq2));
  w.qorder = c.take<int32_t>(d.BH * d.Nq2);
  w.korder = c.take<int32_t>(d.BH * d.Nk2);
  w.args = c.take<uint8_t>(d.BH * (d.Nq + 2 * d.Nk) * d.D);
  w.pairs = d.Bk == 16 ? c.take<int32_t>(d.BH * d.Nq2 * d.stride2 + d.BH * ((d.Nk + 1) / 2)) : nullptr;
  const bool split = d.qsplit || d.ksplit;
  w.idx2 = split ? c.take<int32_t>(d.BH * d.Nq2 * d.stride2) : nullptr;
  w.len2 = split ? c.take<int32_t>(d.BH * d.Nq2) : nullptr;
  w.dqc2 = d.qsplit ? c.take<float>(d.BH * d.Nq2 * d.D) : nullptr;
  w.dkc2 = d.ksplit ? c.take<float>(d.BH * d.Nk2 * d.D) : nullptr;
  w.dvc2 = d.ksplit ? c.take<float>(d.BH * d.Nk2 * d.D) : nullptr;
  w.args2 = split ? c.take<uint8_t>(d.BH * (d.Nq2 + 2 * d.Nk2) * d.D) : nullptr;
  w.bytes = c.off;
  return w;
}

inline vsa_status hip_status(hipError_t e) { return e == hipSuccess ? VSA_OK : VSA_ERR_HIP; }

// The fine forward (with the fused combine when oc is not null) on the
// cubes' lists. With 256-token tiles the kernels run on the 128-token halves:
// the lists (and O_c) are expanded first.
hipError_t run_fine_forward(const Launch& L, const Dims& d, const FwdWs& ws, const void* q, const void* k,
                            const void* v, const int32_t* idx, const int32_t* len, void* of, float* lse_f,
                            const float* oc, const void* g_c, const void* g_f, void* o) {
  const Launch S = fine_view(L);
  const int32_t *fi = idx, *fl = len;
  const float* foc = oc;
  hipError_t e = hipSuccess;
  if (d.qsplit || d.ksplit) {
    e = launch_split_lists(L, S, idx, len, ws.idx2, ws.len2);
    fi = ws.idx2;
    fl = ws.len2;
    if (e == hipSuccess && d.qsplit && oc != nullptr) {
      e = launch_split_rows(L, L.g, S.g, oc, ws.oc2, nullptr, nullptr, 1.0f);
      foc = ws.oc2;
    }
  }
  int32_t* order = L.bf16 ? ws.order : nullptr;
  if (e == hipSuccess && order != nullptr) e = launch_order(S, fi, fl, order);
  if (e == hipSuccess) e = launch_fine_fwd(S, q, k, v, fi, fl, order, of, lse_f, foc, g_c, g_f, o);
  return e;
}

// The fine backward with the pool backward. k2q_off / k2q: the transposed
// lists when the caller has them for the kernels' view (null: built here into
// the workspace). With 256-token tiles the kernels run on the 128-token
// halves: lists, pooled gradients (mean pooling: halved, since a half's
// kernel divides by its 128 tokens) and max-pool argmax positions are
// expanded first, and the transposed lists are always built here.
hipError_t run_fine_backward(const Launch& L, const Dims& d, const BwdWs& ws, const void* q, const void* k,
                             const void* v, const int32_t* idx, const int32_t* len, const int32_t* k2q_off,
                             const int32_t* k2q, const float* lse_f, const void* dof, const float* delta,
                             const float* dqc, const float* dkc, const float* dvc, void* dq, void* dk, void* dv) {
  const Launch S = fine_view(L);
  const bool split = d.qsplit || d.ksplit;
  const int32_t *fi = idx, *fl = len;
  const float *fq = dqc, *fk = dkc, *fv = dvc;
  const float mul = L.pool_max ? 1.0f : 0.5f;
  hipError_t e = hipSuccess;
  if (split) {
    e = launch_split_lists(L, S, idx, len, ws.idx2, ws.len2);
    fi = ws.idx2;
    fl = ws.len2;
    if (e == hipSuccess && d.qsplit) {
      e = launch_split_rows(L, L.g, S.g, dqc, ws.dqc2, nullptr, nullptr, mul);
      fq = ws.dqc2;
    }
    if (e == hipSuccess && d.ksplit) e = launch_split_rows(L, L.gk, S.gk, dkc, ws.dkc2, nullptr, nullptr, mul);
    if (e == hipSuccess && d.ksplit) e = launch_split_rows(L, L.gk, S.gk, dvc, ws.dvc2, nullptr, nullptr, mul);
    if (d.ksplit) {
      fk = ws.dkc2;
      fv = ws.dvc2;
    }
  }
  if (split || k2q_off == nullptr) {
    if (e == hipSuccess) e = launch_index_transpose(S, fi, fl, ws.k2q_off, ws.k2q, ws.k2q_bits);
    k2q_off = ws.k2q_off;
    k2q = ws.k2q;
  }
  if (e == hipSuccess && L.bf16) e = launch_order(S, fi, fl, ws.qorder);
  if (e == hipSuccess && L.bf16) e = launch_order_by_count(S, k2q_off, ws.korder);
  const uint8_t* args = nullptr;
  if (e == hipSuccess && L.pool_max) {
    e = launch_pool(L, q, k, v, nullptr, nullptr, nullptr, ws.args);
    args = ws.args;
    if (e == hipSuccess && split) {
      // planes q (query cubes), k and v (key blocks) of the halves' view
      const size_t D = (size_t)L.D, pq = (size_t)d.BH * d.Nq * D, pk = (size_t)d.BH * d.Nk * D;
      const size_t pq2 = (size_t)d.BH * d.Nq2 * D, pk2 = (size_t)d.BH * d.Nk2 * D;
      const uint8_t* a = ws.args;
      uint8_t* a2 = ws.args2;
      e = d.qsplit ? launch_split_rows(L, L.g, S.g, nullptr, nullptr, a, a2, 1.0f)
                   : hipMemcpyAsync(a2, a, pq, hipMemcpyDeviceToDevice, L.stream);
      for (int w = 0; w < 2 && e == hipSuccess; ++w) {
        const uint8_t* src = a + pq + w * pk;
        uint8_t* dst = a2 + pq2 + w * pk2;
        e = d.ksplit ? launch_split_rows(L, L.gk, S.gk, nullptr, nullptr, src, dst, 1.0f)
                     : hipMemcpyAsync(dst, src, pk, hipMemcpyDeviceToDevice, L.stream);
      }
      args = ws.args2;
    }
  }
  if (e == hipSuccess)
    e = launch_fine_bwd(S, q, k, v, fi, fl, ws.qorder, k2q_off, k2q, ws.korder, lse_f, dof, delta, fq, fk, fv, dq,
                        dk, dv, args, ws.pairs);
  return e;
}

// ---- static scratch of vsa_fine_combine_noalloc ---------------------------
// The query-cube processing order (one int32 per query cube of every
// (b, h)), the only scratch of the fine + combine kernels, kept in a
// file-scope device array so that the call allocates nothing. Each GPU holds
// its own copy for the life of the process. Host code never uses the array's
// name as an address: its device address is looked up per device.
constexpr size_t kNoAllocScratchBytes = size_t(4) << 20;
constexpr long kNoAllocMaxCubes = long(kNoAllocScratchBytes / sizeof(int32_t));
constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

namespace {
// Device address of `scratch` on the current device, looked up on the first
// call there (with that device current) and kept; nullptr on failure.
int32_t* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  int32_t* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
  ptr = static_cast<int32_t*>(addr);
  g_scratch[dev].store(ptr, std::memory_order_release);
  return ptr;
}
}  // namespace

extern "C" {

const char* vsa_status_string(vsa_status s) {
  switch (s) {
    case VSA_OK: return "ok";
    case VSA_ERR_NULL: return "a required pointer is NULL";
    case VSA_ERR_SHAPE: return "invalid shape (B, heads >= 1; T, H, W positive multiples of the cube and key-block sides; sizes in range)";
    case VSA_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case VSA_ERR_DTYPE: return "unknown dtype";
    case VSA_ERR_TOPK: return "topk outside [0, Nk] or invalid list_stride";
    case VSA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case VSA_ERR_WORKSPACE: return "workspace or saved buffer too small";
    case VSA_ERR_INDEX: return "an index list is invalid";
    case VSA_ERR_UNSUPPORTED: return "not supported by this build";
    case VSA_ERR_HIP: return "a HIP call or kernel launch failed";
    case VSA_ERR_SCALE: return "scale must be finite and >= 0";
  }
  return "unknown status";
}

int32_t vsa_version(void) { return 100; }

int32_t vsa_max_cubes(void) { return coarse_max_cubes(); }

size_t vsa_workspace_bytes(const vsa_problem* p, int32_t training) {
  Dims d;
  if (check_problem(p, nullptr, &d) != VSA_OK) return 0;
  const size_t f = carve_fwd_ws(d, nullptr).bytes;
  if (!training) return f;
  const size_t b = carve_bwd_ws(d, nullptr).bytes;
  return f > b ? f : b;
}

size_t vsa_saved_bytes(const vsa_problem* p) {
  Dims d;
  if (check_problem(p, nullptr, &d) != VSA_OK) return 0;
  return carve_saved(d, nullptr).bytes;
}

vsa_status vsa_forward(const vsa_problem* p, const void* q, const void* k, const void* v, const void* g_c,
                       const void* g_f, int32_t* idx, int32_t* len, void* o, void* saved, void* workspace,
                       size_t ws_bytes, void* stream) {
  Launch L;
  Dims d;
  vsa_status st = check_problem(p, &L, &d);
  if (st != VSA_OK) return st;
  st = check_ptrs({{q, true}, {k, true}, {v, true}, {g_c, false}, {g_f, false}, {idx, true}, {len, true},
                   {o, true}, {saved, false}, {workspace, true}});
  if (st != VSA_OK) return st;
  const FwdWs ws = carve_fwd_ws(d, workspace);
  if (ws_bytes < ws.bytes) return VSA_ERR_WORKSPACE;
  L.stream = static_cast<hipStream_t>(stream);
  float *qc = ws.qc, *kc = ws.kc, *vc = ws.vc, *oc = ws.oc, *lse_c = ws.lse_c, *lse_f = nullptr;
  void* of = nullptr;
  if (saved != nullptr) {
    const Saved s = carve_saved(d, saved);
    qc = s.qc; kc = s.kc; vc = s.vc; oc = s.oc; lse_c = s.lse_c; lse_f = s.lse_f; of = s.of;
  }
  hipError_t e = launch_pool(L, q, k, v, qc, kc, vc);
  if (e == hipSuccess)
    e = launch_coarse(L, qc, kc, vc, oc, lse_c, L.topk > 0 ? idx : nullptr, L.topk > 0 ? len : nullptr, ws.s);
  if (e == hipSuccess) e = run_fine_forward(L, d, ws, q, k, v, idx, len, of, lse_f, oc, g_c, g_f, o);
  return hip_status(e);
}

vsa_status vsa_backward(const vsa_problem* p, const void* q, const void* k, const void* v, const void* g_c,
                        const void* g_f, const int32_t* idx, const int32_t* len, const void* saved,
                        const void* d_o, void* dq, void* dk, void* dv, void* dg_c, void* dg_f, void* workspace,
                        size_t ws_bytes, void* stream) {
  Launch L;
  Dims d;
  vsa_status st = check_problem(p, &L, &d);
  if (st != VSA_OK) return st;
  st = check_ptrs({{q, true}, {k, true}, {v, true}, {g_c, false}, {g_f, false}, {idx, true}, {len, true},
                   {saved, true}, {d_o, true}, {dq, true}, {dk, true}, {dv, true}, {dg_c, false},
                   {dg_f, false}, {workspace, true}});
  if (st != VSA_OK) return st;
  const BwdWs ws = carve_bwd_ws(d, workspace);
  if (ws_bytes < ws.bytes) return VSA_ERR_WORKSPACE;
  const Saved s = carve_saved(d, const_cast<void*>(saved));
  L.stream = static_cast<hipStream_t>(stream);
  hipError_t e = launch_combine_bwd(L, d_o, s.oc, s.of, g_c, g_f, g_c ? dg_c : nullptr, g_f ? dg_f : nullptr,
                                    ws.dof, ws.delta, ws.doc);
  if (e == hipSuccess)
    e = launch_coarse_bwd(L, s.qc, s.kc, s.vc, s.oc, s.lse_c, ws.doc, ws.dqc, ws.dkc, ws.dvc, ws.ds_scr, ws.p_scr, ws.dc_scr);
  if (e == hipSuccess)
    e = run_fine_backward(L, d, ws, q, k, v, idx, len, nullptr, nullptr, s.lse_f, ws.dof, ws.delta, ws.dqc, ws.dkc,
                          ws.dvc, dq, dk, dv);
  return hip_status(e);
}

vsa_status vsa_pool(const vsa_problem* p, const void* q, const void* k, const void* v, float* q_c, float* k_c,
                    float* v_c, void* stream) {
  Launch L;
  vsa_status st = check_problem(p, &L, nullptr);
  if (st != VSA_OK) return st;
  st = check_ptrs({{q, true}, {k, true}, {v, true}, {q_c, true}, {k_c, true}, {v_c, true}});
  if (st != VSA_OK) return st;
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_pool(L, q, k, v, q_c, k_c, v_c));
}

vsa_status vsa_coarse(const vsa_problem* p, const float* q_c, const float* k_c, const float* v_c, float* o_c,
                      float* lse_c, int32_t* idx, int32_t* len, void* workspace, size_t ws_bytes, void* stream) {
  Launch L;
  Dims d;
  vsa_status st = check_problem(p, &L, &d);
  if (st != VSA_OK) return st;
  const bool sel = L.topk > 0;
  st = check_ptrs({{q_c, true}, {k_c, true}, {v_c, true}, {o_c, true}, {lse_c, true}, {idx, sel}, {len, sel},
                   {workspace, true}});
  if (st != VSA_OK) return st;
  const FwdWs ws = carve_fwd_ws(d, workspace);
  if (ws_bytes < ws.bytes) return VSA_ERR_WORKSPACE;
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_coarse(L, q_c, k_c, v_c, o_c, lse_c, sel ? idx : nullptr, sel ? len : nullptr, ws.s));
}

vsa_status vsa_fine_forward(const vsa_problem* p, const void* q, const void* k, const void* v, const int32_t* idx,
                            const int32_t* len, void* o_f, float* lse_f, const void* workspace, size_t ws_bytes,
                            void* stream) {
  Launch L;
  Dims d;
  vsa_status st = check_problem(p, &L, &d);
  if (st != VSA_OK) return st;
  const bool need_ws = L.bf16 || d.qsplit || d.ksplit;
  st = check_ptrs({{q, true}, {k, true}, {v, true}, {idx, true}, {len, true}, {o_f, true}, {lse_f, true},
                   {workspace, need_ws}});
  if (st != VSA_OK) return st;
  FwdWs ws{};
  if (need_ws) {
    ws = carve_fwd_ws(d, const_cast<void*>(workspace));
    if (ws_bytes < ws.bytes) return VSA_ERR_WORKSPACE;
  }
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(run_fine_forward(L, d, ws, q, k, v, idx, len, o_f, lse_f, nullptr, nullptr, nullptr, nullptr));
}

vsa_status vsa_fine_combine(const vsa_problem* p, const void* q, const void* k, const void* v, const int32_t* idx,
                            const int32_t* len, const float* o_c, const void* g_c, const void* g_f, void* o, void* o_f,
                            float* lse_f, const void* workspace, size_t ws_bytes, void* stream) {
  Launch L;
  Dims d;
  vsa_status st = check_problem(p, &L, &d);
  if (st != VSA_OK) return st;
  const bool need_ws = L.bf16 || d.qsplit || d.ksplit;
  st = check_ptrs({{q, true}, {k, true}, {v, true}, {idx, true}, {len, true}, {o_c, true}, {g_c, false},
                   {g_f, false}, {o, true}, {o_f, false}, {lse_f, false}, {workspace, need_ws}});
  if (st != VSA_OK) return st;
  FwdWs ws{};
  if (need_ws) {
    ws = carve_fwd_ws(d, const_cast<void*>(workspace));
    if (ws_bytes < ws.bytes) return VSA_ERR_WORKSPACE;
  }
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(run_fine_forward(L, d, ws, q, k, v, idx, len, o_f, lse_f, o_c, g_c, g_f, o));
}

vsa_status vsa_fine_combine_noalloc(const vsa_problem* p, const void* q, const void* k, const void* v,
                                    const int32_t* idx, const int32_t* len, const float* o_c, const void* g_c,
                                    const void* g_f, void* o, void* o_f, float* lse_f, void* stream) {
  Launch L;
  Dims d;
  vsa_status st = check_problem(p, &L, &d);
  if (st != VSA_OK) return st;
  st = check_ptrs({{q, true}, {k, true}, {v, true}, {idx, true}, {len, true}, {o_c, true}, {g_c, false},
                   {g_f, false}, {o, true}, {o_f, false}, {lse_f, false}});
  if (st != VSA_OK) return st;
  if (d.BH * d.Nq > kNoAllocMaxCubes) return VSA_ERR_WORKSPACE;
  if (d.qsplit || d.ksplit) return VSA_ERR_UNSUPPORTED;   // 256-token tiles need expanded lists (a workspace)
  int32_t* order = nullptr;
  if (L.bf16) {
    order = scratch_ptr();
    if (order == nullptr) return VSA_ERR_HIP;
  }
  L.stream = static_cast<hipStream_t>(stream);
  // launch_order writes all B*heads*Nq entries before the fine kernel reads
  // any, so nothing left by an earlier call is ever read.
  hipError_t e = order != nullptr ? launch_order(L, idx, len, order) : hipSuccess;
  if (e == hipSuccess) e = launch_fine_fwd(L, q, k, v, idx, len, order, o_f, lse_f, o_c, g_c, g_f, o);
  return hip_status(e);
}

vsa_status vsa_combine(const vsa_problem* p, const float* o_c, const void* o_f, const void* g_c, const void* g_f,
                       void* o, void* stream) {
  Launch L;
  vsa_status st = check_problem(p, &L, nullptr);
  if (st != VSA_OK) return st;
  st = check_ptrs({{o_c, true}, {o_f, true}, {g_c, false}, {g_f, false}, {o, true}});
  if (st != VSA_OK) return st;
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_combine(L, o_c, o_f, g_c, g_f, o));
}

vsa_status vsa_combine_backward(const vsa_problem* p, const void* d_o, const float* o_c, const void* o_f,
                                const void* g_c, const void* g_f, void* dg_c, void* dg_f, void* d_o_f, float* delta,
                                float* d_o_c, void* stream) {
  Launch L;
  vsa_status st = check_problem(p, &L, nullptr);
  if (st != VSA_OK) return st;
  st = check_ptrs({{d_o, true}, {o_c, true}, {o_f, true}, {g_c, false}, {g_f, false}, {dg_c, false},
                   {dg_f, false}, {d_o_f, true}, {delta, true}, {d_o_c, true}});
  if (st != VSA_OK) return st;
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_combine_bwd(L, d_o, o_c, o_f, g_c, g_f, dg_c, dg_f, d_o_f, delta, d_o_c));
}

vsa_status vsa_index_transpose(const vsa_problem* p, const int32_t* idx, const int32_t* len, int32_t* k2q_off,
                               int32_t* k2q, void* workspace, size_t ws_bytes, void* stream) {
  Launch L;
  Dims d;
  vsa_status st = check_problem(p, &L, &d);
  if (st != VSA_OK) return st;
  st = check_ptrs({{idx, true}, {len, true}, {k2q_off, true}, {k2q, true}, {workspace, true}});
  if (st != VSA_OK) return st;
  const BwdWs ws = carve_bwd_ws(d, workspace);
  if (ws_bytes < ws.bytes) return VSA_ERR_WORKSPACE;
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_index_transpose(L, idx, len, k2q_off, k2q, ws.k2q_bits));
}

vsa_status vsa_fine_backward(const vsa_problem* p, const void* q, const void* k, const void* v, const int32_t* idx,
                             const int32_t* len, const int32_t* k2q_off, const int32_t* k2q, const float* lse_f,
                             const void* d_o_f, const float* delta, const float* dq_c, const float* dk_c,
                             const float* dv_c, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                             void* stream) {
  Launch L;
  Dims d;
  vsa_status st = check_problem(p, &L, &d);
  if (st != VSA_OK) return st;
  st = check_ptrs({{q, true}, {k, true}, {v, true}, {idx, true}, {len, true}, {k2q_off, true}, {k2q, true},
                   {lse_f, true}, {d_o_f, true}, {delta, true}, {dq_c, true}, {dk_c, true}, {dv_c, true},
                   {dq, true}, {dk, true}, {dv, true}, {workspace, true}});
  if (st != VSA_OK) return st;
  const BwdWs ws = carve_bwd_ws(d, workspace);
  if (ws_bytes < ws.bytes) return VSA_ERR_WORKSPACE;
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(run_fine_backward(L, d, ws, q, k, v, idx, len, k2q_off, k2q, lse_f, d_o_f, delta, dq_c, dk_c,
                                      dv_c, dq, dk, dv));
}

vsa_status vsa_coarse_backward(const vsa_problem* p, const float* q_c, const float* k_c, const float* v_c,
                               const float* o_c, const float* lse_c, const float* d_o_c, float* dq_c, float* dk_c,
                               float* dv_c, void* workspace, size_t ws_bytes, void* stream) {
  Launch L;
  Dims d;
  vsa_status st = check_problem(p, &L, &d);
  if (st != VSA_OK) return st;
  st = check_ptrs({{q_c, true}, {k_c, true}, {v_c, true}, {o_c, true}, {lse_c, true}, {d_o_c, true},
                   {dq_c, true}, {dk_c, true}, {dv_c, true}, {workspace, true}});
  if (st != VSA_OK) return st;
  const BwdWs ws = carve_bwd_ws(d, workspace);
  if (ws_bytes < ws.bytes) return VSA_ERR_WORKSPACE;
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_coarse_bwd(L, q_c, k_c, v_c, o_c, lse_c, d_o_c, dq_c, dk_c, dv_c, ws.ds_scr, ws.p_scr, ws.dc_scr));
}

static vsa_status relayout(const vsa_problem* p, const void* src, void* dst, bool to_tiled, void* stream) {
  Launch L;
  vsa_status st = check_problem(p, &L, nullptr);
  if (st != VSA_OK) return st;
  st = check_ptrs({{src, true}, {dst, true}});
  if (st != VSA_OK) return st;
  if (src == dst) return VSA_ERR_UNSUPPORTED;
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_relayout(L, src, dst, to_tiled));
}

vsa_status vsa_tile(const vsa_problem* p, const void* x, void* xt, void* stream) {
  return relayout(p, x, xt, true, stream);
}

vsa_status vsa_untile(const vsa_problem* p, const void* xt, void* x, void* stream) {
  return relayout(p, xt, x, false, stream);
}

vsa_status vsa_compatible_latent(int32_t T, int32_t H, int32_t W, int32_t ct, int32_t ch, int32_t cw, int32_t* Tc,
                                 int32_t* Hc, int32_t* Wc) {
  if (Tc == nullptr || Hc == nullptr || Wc == nullptr) return VSA_ERR_NULL;
  const int32_t side[3] = {ct ? ct : 4, ch ? ch : 4, cw ? cw : 4}, n[3] = {T, H, W};
  int32_t out[3];
  for (int a = 0; a < 3; ++a) {
    if (!pow2_side(side[a]) || n[a] <= 0) return VSA_ERR_SHAPE;
    const long r = ((long)n[a] + side[a] - 1) / side[a] * side[a];
    if (r > 0x7fffffffL) return VSA_ERR_SHAPE;
    out[a] = (int32_t)r;
  }
  *Tc = out[0];
  *Hc = out[1];
  *Wc = out[2];
  return VSA_OK;
}

static vsa_status crop_pad(const vsa_problem* p, const void* src, int32_t T, int32_t H, int32_t W, void* dst,
                           bool to_small, void* stream) {
  Launch L;
  vsa_status st = check_problem(p, &L, nullptr);
  if (st != VSA_OK) return st;
  if (T <= 0 || H <= 0 || W <= 0 || T > p->T || H > p->H || W > p->W) return VSA_ERR_SHAPE;
  st = check_ptrs({{src, true}, {dst, true}});
  if (st != VSA_OK) return st;
  if (src == dst) return VSA_ERR_UNSUPPORTED;
  L.stream = static_cast<hipStream_t>(stream);
  return hip_status(launch_crop_pad(L, src, dst, T, H, W, to_small));
}

vsa_status vsa_crop(const vsa_problem* p, const void* x, int32_t T, int32_t H, int32_t W, void* out, void* stream) {
  return crop_pad(p, x, T, H, W, out, true, stream);
}

vsa_status vsa_pad(const vsa_problem* p, const void* x, int32_t T, int32_t H, int32_t W, void* out, void* stream) {
  return crop_pad(p, x, T, H, W, out, false, stream);
}

vsa_status vsa_check_lists_host(const vsa_problem* p, const int32_t* idx, const int32_t* len) {
  Dims d;
  vsa_status st = check_problem(p, nullptr, &d);
  if (st != VSA_OK) return st;
  if (idx == nullptr || len == nullptr) return VSA_ERR_NULL;
  const long rows = d.BH * d.Nq;
  for (long r = 0; r < rows; ++r) {
    const int n = len[r];
    if (n < 0 || n > d.stride) return VSA_ERR_INDEX;
    int prev = -1;
    for (int t = 0; t < n; ++t) {
      const int v = idx[r * d.stride + t];
      if (v <= prev || v >= d.Nk) return VSA_ERR_INDEX;
      prev = v;
    }
  }
  return VSA_OK;
}

vsa_status vsa_validate_lists(const vsa_problem* p, const int32_t* idx, const int32_t* len, int32_t* flag,
                              void* stream) {
  Launch L;
  vsa_status st = check_problem(p, &L, nullptr);
  if (st != VSA_OK) return st;
  st = check_ptrs({{idx, true}, {len, true}});
  if (st != VSA_OK) return st;
  if (flag == nullptr) return VSA_ERR_NULL;
  L.stream = static_cast<hipStream_t>(stream);
  if (hipMemsetAsync(flag, 0, sizeof(int32_t), L.stream) != hipSuccess) return VSA_ERR_HIP;
  if (launch_validate_lists(L, idx, len, flag) != hipSuccess) return VSA_ERR_HIP;
  int32_t h = 0;
  if (hipMemcpyAsync(&h, flag, sizeof(int32_t), hipMemcpyDeviceToHost, L.stream) != hipSuccess) return VSA_ERR_HIP;
  if (hipStreamSynchronize(L.stream) != hipSuccess) return VSA_ERR_HIP;
  return h ? VSA_ERR_INDEX : VSA_OK;
}

}  // extern "C"
