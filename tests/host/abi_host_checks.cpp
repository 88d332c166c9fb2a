// Host-only driver for the C ABI's host logic (validation, buffer carving,
// the host list checker), built together with vsa_api.cpp under
// AddressSanitizer and UndefinedBehaviorSanitizer (host code only). Every
// kernel launcher is replaced by a stub that reports a failed launch, so the
// driver needs no GPU: calls that pass validation end in VSA_ERR_HIP.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "vsa.h"
#include "../../block_sparse_video_cube_amd/csrc/vsa_kernels.h"

namespace vsa {
static int g_launches = 0;
static hipError_t stub() { ++g_launches; return hipErrorInvalidValue; }
hipError_t launch_pool(const Launch&, const void*, const void*, const void*, float*, float*, float*, uint8_t*) { return stub(); }
hipError_t launch_relayout(const Launch&, const void*, void*, bool) { return stub(); }
hipError_t launch_crop_pad(const Launch&, const void*, void*, int, int, int, bool) { return stub(); }
int coarse_max_cubes() { return 8192; }
int coarse_ld(int Nc) { return (Nc + 3) & ~3; }
hipError_t launch_coarse(const Launch&, const float*, const float*, const float*, float*, float*, int32_t*, int32_t*, float*) { return stub(); }
hipError_t launch_order(const Launch&, const int32_t*, const int32_t*, int32_t*) { return stub(); }
hipError_t launch_fine_fwd(const Launch&, const void*, const void*, const void*, const int32_t*, const int32_t*,
                           const int32_t*, void*, float*, const float*, const void*, const void*, void*) { return stub(); }
hipError_t launch_combine(const Launch&, const float*, const void*, const void*, const void*, void*) { return stub(); }
hipError_t launch_combine_bwd(const Launch&, const void*, const float*, const void*, const void*, const void*, void*,
                              void*, void*, float*, float*) { return stub(); }
int k2q_bits_words(int Nc) { return (Nc + 31) / 32; }
hipError_t launch_index_transpose(const Launch&, const int32_t*, const int32_t*, int32_t*, int32_t*, uint32_t*) { return stub(); }
hipError_t launch_coarse_bwd(const Launch&, const float*, const float*, const float*, const float*, const float*,
                             const float*, float*, float*, float*, float*, float*, float*) { return stub(); }
hipError_t launch_order_by_count(const Launch&, const int32_t*, int32_t*) { return stub(); }
hipError_t launch_fine_bwd(const Launch&, const void*, const void*, const void*, const int32_t*, const int32_t*,
                           const int32_t*, const int32_t*, const int32_t*, const int32_t*, const float*, const void*,
                           const float*, const float*, const float*, const float*, void*, void*, void*,
                           const uint8_t*, int32_t*) { return stub(); }
hipError_t launch_key_pairs(const Launch&, const int32_t*, const int32_t*, int32_t*, int32_t*) { return stub(); }
hipError_t launch_validate_lists(const Launch&, const int32_t*, const int32_t*, int32_t*) { return stub(); }
hipError_t launch_split_lists(const Launch&, const Launch&, const int32_t*, const int32_t*, int32_t*, int32_t*) { return stub(); }
hipError_t launch_split_rows(const Launch&, const Grid&, const Grid&, const float*, float*, const uint8_t*, uint8_t*, float) { return stub(); }
}  // namespace vsa

static int failures = 0;
#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) { std::fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, #cond); ++failures; } \
  } while (0)

static vsa_problem base() {
  vsa_problem p;
  std::memset(&p, 0, sizeof(p));
  p.B = 1; p.heads = 2; p.T = 8; p.H = 16; p.W = 16; p.head_dim = 64; p.dtype = VSA_BF16; p.topk = 4;
  return p;
}

int main() {
  // Validation: every status forcible from the host.
  vsa_problem p = base();
  CHECK(vsa_workspace_bytes(&p, 0) > 0 && vsa_workspace_bytes(&p, 1) >= vsa_workspace_bytes(&p, 0));
  CHECK(vsa_saved_bytes(&p) > 0);
  CHECK(vsa_workspace_bytes(nullptr, 0) == 0);
  { vsa_problem b = base(); b.T = 6; CHECK(vsa_workspace_bytes(&b, 0) == 0); }
  { vsa_problem b = base(); b.head_dim = 96; CHECK(vsa_workspace_bytes(&b, 0) == 0); }
  { vsa_problem b = base(); b.topk = 100000; CHECK(vsa_workspace_bytes(&b, 0) == 0); }
  { vsa_problem b = base(); b.cube_t = 3; CHECK(vsa_workspace_bytes(&b, 0) == 0); }
  { vsa_problem b = base(); b.cube_t = 2; CHECK(vsa_workspace_bytes(&b, 0) > 0); }
  { vsa_problem b = base(); b.B = 0x7fffffff; b.heads = 0x7fffffff; CHECK(vsa_workspace_bytes(&b, 0) == 0); }
  { vsa_problem b = base(); b.T = 1 << 20; b.H = 1 << 12; CHECK(vsa_workspace_bytes(&b, 0) == 0); }

  // Buffers large enough for the problem; the stubbed launches fail, so the
  // entry points return VSA_ERR_HIP after validating and carving them.
  const size_t n = (size_t)p.B * p.heads * p.T * p.H * p.W * p.head_dim;
  std::vector<uint16_t> q(n), o(n);
  const int nc = p.T * p.H * p.W / 64;
  std::vector<int32_t> idx((size_t)p.B * p.heads * nc * p.topk), len((size_t)p.B * p.heads * nc);
  std::vector<unsigned char> ws(vsa_workspace_bytes(&p, 1) + 256), saved(vsa_saved_bytes(&p) + 256);
  void* wsp = ws.data() + (256 - ((uintptr_t)ws.data() & 255)) % 256;
  void* svp = saved.data() + (256 - ((uintptr_t)saved.data() & 255)) % 256;
  CHECK(vsa_forward(&p, q.data(), q.data(), q.data(), nullptr, nullptr, idx.data(), len.data(), o.data(), svp, wsp,
                    vsa_workspace_bytes(&p, 0), nullptr) == VSA_ERR_HIP);
  CHECK(vsa_forward(&p, q.data(), q.data(), q.data(), nullptr, nullptr, idx.data(), len.data(), o.data(), svp, wsp,
                    vsa_workspace_bytes(&p, 0) - 1, nullptr) == VSA_ERR_WORKSPACE);
  CHECK(vsa_forward(&p, nullptr, q.data(), q.data(), nullptr, nullptr, idx.data(), len.data(), o.data(), svp, wsp,
                    vsa_workspace_bytes(&p, 0), nullptr) == VSA_ERR_NULL);
  CHECK(vsa_forward(&p, (char*)q.data() + 2, q.data(), q.data(), nullptr, nullptr, idx.data(), len.data(), o.data(),
                    svp, wsp, vsa_workspace_bytes(&p, 0), nullptr) == VSA_ERR_ALIGN);
  CHECK(vsa_backward(&p, q.data(), q.data(), q.data(), nullptr, nullptr, idx.data(), len.data(), svp, q.data(),
                     o.data(), o.data(), o.data(), nullptr, nullptr, wsp, vsa_workspace_bytes(&p, 1),
                     nullptr) == VSA_ERR_HIP);
  { vsa_problem f = base(); f.dtype = VSA_F32;   // fp32 backward: validated, then launched like bf16
    std::vector<unsigned char> wf(vsa_workspace_bytes(&f, 1) + 256);
    void* wfp = wf.data() + (256 - ((uintptr_t)wf.data() & 255)) % 256;
    CHECK(vsa_backward(&f, q.data(), q.data(), q.data(), nullptr, nullptr, idx.data(), len.data(), svp, q.data(),
                       o.data(), o.data(), o.data(), nullptr, nullptr, wfp, vsa_workspace_bytes(&f, 1), nullptr) ==
          VSA_ERR_HIP);
    CHECK(vsa_backward(&f, q.data(), q.data(), q.data(), nullptr, nullptr, idx.data(), len.data(), svp, q.data(),
                       o.data(), o.data(), o.data(), nullptr, nullptr, wfp, vsa_workspace_bytes(&f, 1) - 1,
                       nullptr) == VSA_ERR_WORKSPACE); }
  CHECK(vsa_tile(&p, q.data(), o.data(), nullptr) == VSA_ERR_HIP);
  CHECK(vsa_crop(&p, q.data(), 5, 7, 9, o.data(), nullptr) == VSA_ERR_HIP);

  // Host list checker: valid lists, then each kind of invalid entry.
  vsa_problem l = base(); l.topk = 0; l.list_stride = 4;
  for (int r = 0; r < p.B * p.heads * nc; ++r) {
    len[r] = r % 5;
    for (int t = 0; t < 4; ++t) idx[(size_t)r * 4 + t] = t < len[r] ? 3 * t + r % 3 : -1;
  }
  CHECK(vsa_check_lists_host(&l, idx.data(), len.data()) == VSA_OK);
  idx[9] = idx[8];                        // row 2: duplicate
  CHECK(vsa_check_lists_host(&l, idx.data(), len.data()) == VSA_ERR_INDEX);
  idx[9] = nc;                            // out of range
  CHECK(vsa_check_lists_host(&l, idx.data(), len.data()) == VSA_ERR_INDEX);
  idx[9] = 5; len[3] = 5;                 // length beyond the stride
  CHECK(vsa_check_lists_host(&l, idx.data(), len.data()) == VSA_ERR_INDEX);
  CHECK(vsa_check_lists_host(&l, nullptr, len.data()) == VSA_ERR_NULL);

  int32_t tc, hc, wc;
  CHECK(vsa_compatible_latent(9, 13, 30, 0, 0, 0, &tc, &hc, &wc) == VSA_OK && tc == 12 && hc == 16 && wc == 32);
  CHECK(vsa_compatible_latent(0x7fffffff, 4, 4, 0, 0, 0, &tc, &hc, &wc) == VSA_ERR_SHAPE);
  for (int s = 0; s <= 12; ++s) CHECK(vsa_status_string((vsa_status)s) != nullptr);

  CHECK(vsa::g_launches > 0);
  if (failures == 0) std::printf("host checks passed (%d stubbed launches)\n", vsa::g_launches);
  return failures == 0 ? 0 : 1;
}
