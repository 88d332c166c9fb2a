// Measurement aids behind two bounds quoted with the VSA kernels on the
// MI355X (declared in include/vsa_probe.h; not steps of the operator):
//  * how much independent vector-ALU work hides under 32x32x16 bf16 MFMAs,
//    at one or two waves per SIMD (the budget of the fine kernels' softmax);
//  * the rate of a plain streaming read of HBM (the ceiling of the pool and
//    combine-backward stages, which read every input element once);
//  * the rate at which L2-resident data reaches LDS, by direct-to-LDS loads
//    (the fine kernels' chunk path) or by loads into registers and LDS
//    writes.
// The kernels stay inside their buffers and run a fixed number of
// iterations; their outputs only keep the work from being removed.
#include <stdint.h>

#include "../../include/vsa.h"
#include "../../include/vsa_probe.h"
#include "fine_common.h"
#include "vsa_common.h"

namespace vsa {

// Four waves per workgroup, one per SIMD of a CU; LDSK KB of static LDS caps
// the workgroups per CU (96 KB: one, 64 KB: two), i.e. the waves per SIMD.
// Each round: four independent MFMA chains, each MFMA followed by NV
// independent VALU instructions (OP 0: fp32 FMA, 1: exp2), kept in program
// order by scheduling barriers.
template <int NV, int OP, int LDSK>
__global__ __launch_bounds__(256) void probe_mfma_valu_kernel(float* __restrict__ out, int iters) {
  __shared__ float pad[LDSK * 256];
  pad[threadIdx.x] = 1.0f;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)(0.001f * (lane + i));
    b[i] = (bf16)(0.002f * (lane - i));
  }
  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[m][e] = 0.f;
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = -0.001f * (lane + j) - 1.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[m] = mfma32_bf16(a, b, acc[m]);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        if (OP == 0) x[j & 15] = __builtin_fmaf(x[j & 15], 0.999f, 0.0001f);
        else x[j & 15] = __builtin_amdgcn_exp2f(x[j & 15]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = pad[(threadIdx.x + 1) & 255];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[m][e];
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Grid-stride 16-byte loads of n16 units, U loads in flight per thread
// (issued before any is used), summed into one float per thread; NT: the
// loads carry the non-temporal hint.
template <int U, bool NT>
__global__ __launch_bounds__(256) void probe_stream_read_kernel(const f32x4* __restrict__ src, long n16,
                                                                float* __restrict__ out) {
  const long stride = (long)gridDim.x * 256;
  float s = 0.f;
  for (long base = (long)blockIdx.x * 256 + threadIdx.x; base < n16; base += stride * U) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long i = base + u * stride;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      v[u] = i < n16 ? (NT ? __builtin_nontemporal_load(src + i) : src[i]) : z;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) s += v[u][0] + v[u][1] + v[u][2] + v[u][3];
  }
  out[(long)blockIdx.x * 256 + threadIdx.x] = s;
}

template <bool NT>
static hipError_t launch_stream_read(const f32x4* s4, long n16, int blocks, int inflight, float* out,
                                     hipStream_t st) {
  const dim3 grid(blocks), block(256);
  switch (inflight) {
    case 1: hipLaunchKernelGGL((probe_stream_read_kernel<1, NT>), grid, block, 0, st, s4, n16, out); break;
    case 2: hipLaunchKernelGGL((probe_stream_read_kernel<2, NT>), grid, block, 0, st, s4, n16, out); break;
    case 4: hipLaunchKernelGGL((probe_stream_read_kernel<4, NT>), grid, block, 0, st, s4, n16, out); break;
    case 8: hipLaunchKernelGGL((probe_stream_read_kernel<8, NT>), grid, block, 0, st, s4, n16, out); break;
    default: hipLaunchKernelGGL((probe_stream_read_kernel<16, NT>), grid, block, 0, st, s4, n16, out); break;
  }
  return hipGetLastError();
}

// L2 to LDS: workgroups of two waves with 40 KB of LDS (four per CU, as in
// the fine forward). Iteration c moves the 16 KB chunk at byte
// ((blockIdx * 7 + c) * 16 KB) mod src_bytes of src into stage c % 2, each
// wave 8 KB in 1 KB loads, the next chunk's loads in flight while the
// current one completes, a barrier per iteration. MODE 0: direct-to-LDS
// loads; 1: 16-byte loads into registers, then LDS writes.
constexpr int kL2Stage = 16384;
template <int MODE>
__global__ __launch_bounds__(128) void probe_l2_lds_kernel(const char* __restrict__ src, uint32_t src_mask,
                                                           int iters, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char buf[2 * kL2Stage + 8192];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto chunk_src = [&](int c) {
    const uint32_t off = ((uint32_t)(blockIdx.x * 7 + c) * (uint32_t)kL2Stage) & src_mask;
    return reinterpret_cast<const char*>(uniform_ptr(src + off));
  };
  if constexpr (MODE == 0) {
    const uint32_t base = lds_addr(buf);
    auto issue = [&](int c) {
      const char* s = chunk_src(c);
      const uint32_t dst = base + (c & 1) * kL2Stage;
#pragma unroll
      for (int t = 0; t < 8; ++t) dma16(s, (uint32_t)((wv * 8 + t) * 1024 + lane * 16), dst + (wv * 8 + t) * 1024);
    };
    issue(0);
    for (int c = 0; c < iters; ++c) {
      if (c + 1 < iters) {
        issue(c + 1);
        wait_vmcnt<8>();
      } else {
        wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();
    }
    vm_settled();
  } else {
    f32x4 cur[8], nxt[8];
    auto load = [&](int c, f32x4 (&r)[8]) {
      const char* s = chunk_src(c);
#pragma unroll
      for (int t = 0; t < 8; ++t) r[t] = *reinterpret_cast<const f32x4*>(s + (wv * 8 + t) * 1024 + lane * 16);
    };
    load(0, cur);
    for (int c = 0; c < iters; ++c) {
      if (c + 1 < iters) load(c + 1, nxt);
      char* d = buf + (c & 1) * kL2Stage;
#pragma unroll
      for (int t = 0; t < 8; ++t) *reinterpret_cast<f32x4*>(d + (wv * 8 + t) * 1024 + lane * 16) = cur[t];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int t = 0; t < 8; ++t) cur[t] = nxt[t];
    }
  }
  __syncthreads();
  out[blockIdx.x * 128 + threadIdx.x] = reinterpret_cast<const float*>(buf)[(threadIdx.x * 37) & (2 * kL2Stage / 4 - 1)];
}

template <int NV, int OP>
static hipError_t launch_probe_mfma(int waves, int iters, float* out, hipStream_t st) {
  const dim3 grid(256 * waves), block(256);
  if (waves == 1)
    hipLaunchKernelGGL((probe_mfma_valu_kernel<NV, OP, 96>), grid, block, 0, st, out, iters);
  else
    hipLaunchKernelGGL((probe_mfma_valu_kernel<NV, OP, 64>), grid, block, 0, st, out, iters);
  return hipGetLastError();
}

template <int OP>
static hipError_t probe_mfma_op(int valu, int waves, int iters, float* out, hipStream_t st) {
  switch (valu) {
    case 0: return launch_probe_mfma<0, OP>(waves, iters, out, st);
    case 1: return launch_probe_mfma<1, OP>(waves, iters, out, st);
    case 2: return launch_probe_mfma<2, OP>(waves, iters, out, st);
    case 4: return launch_probe_mfma<4, OP>(waves, iters, out, st);
    case 8: return launch_probe_mfma<8, OP>(waves, iters, out, st);
    default: return launch_probe_mfma<16, OP>(waves, iters, out, st);
  }
}

}  // namespace vsa

extern "C" {

int32_t vsa_probe_mfma_valu(int32_t valu, int32_t op, int32_t waves_per_simd, int32_t iters, float* out,
                            void* stream) {
  if (out == nullptr) return VSA_ERR_NULL;
  if (valu != 0 && valu != 1 && valu != 2 && valu != 4 && valu != 8 && valu != 16) return VSA_ERR_UNSUPPORTED;
  if (op != 0 && op != 1) return VSA_ERR_UNSUPPORTED;
  if (waves_per_simd != 1 && waves_per_simd != 2) return VSA_ERR_UNSUPPORTED;
  if (iters < 1) return VSA_ERR_SHAPE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = op == 0 ? vsa::probe_mfma_op<0>(valu, waves_per_simd, iters, out, st)
                               : vsa::probe_mfma_op<1>(valu, waves_per_simd, iters, out, st);
  return e == hipSuccess ? VSA_OK : VSA_ERR_HIP;
}

int32_t vsa_probe_stream_read(const void* src, size_t bytes, int32_t blocks, int32_t inflight, int32_t nontemporal,
                              float* out, void* stream) {
  if (src == nullptr || out == nullptr) return VSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (bytes & 15u) != 0) return VSA_ERR_ALIGN;
  if (blocks < 1 || blocks > (1 << 20) || bytes == 0) return VSA_ERR_SHAPE;
  if (inflight != 1 && inflight != 2 && inflight != 4 && inflight != 8 && inflight != 16) return VSA_ERR_UNSUPPORTED;
  if (nontemporal != 0 && nontemporal != 1) return VSA_ERR_UNSUPPORTED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const vsa::f32x4* s4 = static_cast<const vsa::f32x4*>(src);
  const long n16 = (long)(bytes / 16);
  const hipError_t e = nontemporal ? vsa::launch_stream_read<true>(s4, n16, blocks, inflight, out, st)
                                   : vsa::launch_stream_read<false>(s4, n16, blocks, inflight, out, st);
  return e == hipSuccess ? VSA_OK : VSA_ERR_HIP;
}

int32_t vsa_probe_l2_to_lds(int32_t mode, const void* src, size_t src_bytes, int32_t blocks, int32_t iters,
                            float* out, void* stream) {
  if (src == nullptr || out == nullptr) return VSA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0) return VSA_ERR_ALIGN;
  if (src_bytes < (size_t)vsa::kL2Stage || src_bytes > ((size_t)1 << 30) || (src_bytes & (src_bytes - 1)) != 0)
    return VSA_ERR_SHAPE;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1) return VSA_ERR_SHAPE;
  if (mode != 0 && mode != 1) return VSA_ERR_UNSUPPORTED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const char* s = static_cast<const char*>(src);
  const uint32_t mask = (uint32_t)(src_bytes - 1);
  if (mode == 0)
    hipLaunchKernelGGL(vsa::probe_l2_lds_kernel<0>, dim3(blocks), dim3(128), 0, st, s, mask, iters, out);
  else
    hipLaunchKernelGGL(vsa::probe_l2_lds_kernel<1>, dim3(blocks), dim3(128), 0, st, s, mask, iters, out);
  return hipGetLastError() == hipSuccess ? VSA_OK : VSA_ERR_HIP;
}

}  // extern "C"
