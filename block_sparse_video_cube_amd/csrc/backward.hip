// List utilities of the backward: the index transpose (for each key block,
// the query cubes whose lists hold it) and the list validator.
// The transposed lists are what the dK / dV walk of the fine backward
// (fine_bwd.hip) consumes; the validator checks caller-supplied lists.
#include "vsa_kernels.h"

namespace vsa {

// ------------------------------------------------------------ list helpers
// Index transpose through a key-major bitmask: bit i of row j of `bits`
// (Nk rows of W = ceil(Nq / 32) words) is set when query cube i lists key
// block j. Counting a row's bits gives the length of j's list, and walking them
// writes it in ascending order, so the result is deterministic.
__global__ __launch_bounds__(256) void k2q_zero_kernel(uint32_t* __restrict__ bits, long n) {
  for (long e = (long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long)gridDim.x * 256) bits[e] = 0u;
}

__global__ __launch_bounds__(256) void k2q_bits_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ len, uint32_t* __restrict__ bits,
                                                       int Nq, int Nk, int stride, int W) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;   // entry of this head's lists
  const long bh = blockIdx.y;
  if (e >= (long)Nq * stride) return;
  const int i = (int)(e / stride), t = (int)(e - (long)i * stride);
  const long row = bh * Nq + i;
  if (t >= min(max(len[row], 0), stride)) return;
  const int j = idx[row * stride + t];
  if (j < 0 || j >= Nk) return;
  atomicOr(&bits[(bh * Nk + j) * W + (i >> 5)], 1u << (i & 31));
}

// cnt[bh][j + 1] = number of query cubes listing j (cnt[bh][0] is set by the scan).
__global__ __launch_bounds__(256) void k2q_count_kernel(const uint32_t* __restrict__ bits, int32_t* __restrict__ cnt,
                                                        int Nk, int W) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const long bh = blockIdx.y;
  if (j >= Nk) return;
  const uint32_t* r = bits + (bh * Nk + j) * W;
  int c = 0;
  for (int w = 0; w < W; ++w) c += __popc(r[w]);
  cnt[bh * (Nk + 1) + j + 1] = c;
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
                                                       int Nq, int Nk, int stride, int W) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const long bh = blockIdx.y;
  if (j >= Nk) return;
  const uint32_t* r = bits + (bh * Nk + j) * W;
  int32_t* out = k2q + bh * (long)Nq * stride;
  int pos = off[bh * (Nk + 1) + j];
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
  const int Nq = L.g.Nc, Nk = L.gk.Nc, W = k2q_bits_words(Nq);
  const long nbits = (long)L.BH * Nk * W;
  hipLaunchKernelGGL(k2q_zero_kernel, dim3((unsigned)min((nbits + 255) / 256, 65536L)), dim3(256), 0, L.stream,
                     bits, nbits);
  const long entries = (long)Nq * L.stride;
  hipLaunchKernelGGL(k2q_bits_kernel, dim3((unsigned)((entries + 255) / 256), L.BH), dim3(256), 0, L.stream, idx,
                     len, bits, Nq, Nk, L.stride, W);
  const dim3 grid((Nk + 255) / 256, L.BH);
  hipLaunchKernelGGL(k2q_count_kernel, grid, dim3(256), 0, L.stream, bits, k2q_off, Nk, W);
  hipLaunchKernelGGL(k2q_scan_kernel, dim3(L.BH), dim3(256), 0, L.stream, k2q_off, Nk);
  hipLaunchKernelGGL(k2q_fill_kernel, grid, dim3(256), 0, L.stream, bits, k2q_off, k2q, Nq, Nk, L.stride, W);
  return hipGetLastError();
}

// Union of the transposed lists of key blocks 2P and 2P + 1 (16-token
// blocks, which the dK / dV kernels take two at a time): a merge of two
// ascending lists, one thread per pair, written where block 2P's list starts
// (the union is no longer than the two lists together). Offsets are clamped
// to the k2q array, so malformed offsets cannot move a write outside it.
__global__ __launch_bounds__(256) void k2q_pair_kernel(const int32_t* __restrict__ off,
                                                       const int32_t* __restrict__ k2q, int32_t* __restrict__ k2u,
                                                       int32_t* __restrict__ plen, int Nq, int Nk, int stride) {
  const int P = blockIdx.x * 256 + threadIdx.x;
  const long bh = blockIdx.y;
  const int npairs = (Nk + 1) >> 1;
  if (P >= npairs) return;
  const int cap = Nq * stride;
  const int32_t* o = off + bh * (Nk + 1);
  const int32_t* src = k2q + bh * (long)cap;
  int32_t* dst = k2u + bh * (long)cap;
  int a = min(max(o[2 * P], 0), cap);
  const int a1 = min(max(o[2 * P + 1], a), cap);
  int b = a1;
  const int b1 = 2 * P + 1 < Nk ? min(max(o[2 * P + 2], a1), cap) : a1;
  const int w0 = a;
  int w = w0;
  while (a < a1 || b < b1) {
    const int va = a < a1 ? src[a] : 0x7fffffff, vb = b < b1 ? src[b] : 0x7fffffff;
    if (va == vb) { dst[w++] = va | (3 << 24); ++a; ++b; }
    else if (va < vb) { dst[w++] = va | (1 << 24); ++a; }
    else { dst[w++] = vb | (2 << 24); ++b; }
  }
  plen[bh * npairs + P] = w - w0;
}

hipError_t launch_key_pairs(const Launch& L, const int32_t* k2q_off, const int32_t* k2q, int32_t* k2u,
                            int32_t* plen) {
  const int Nk = L.gk.Nc, npairs = (Nk + 1) / 2;
  hipLaunchKernelGGL(k2q_pair_kernel, dim3((npairs + 255) / 256, L.BH), dim3(256), 0, L.stream, k2q_off, k2q, k2u,
                     plen, L.g.Nc, Nk, L.stride);
  return hipGetLastError();
}

// Lists valid? len in [0, stride], ids in [0, Nk), strictly increasing.
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
                     flag, rows, L.gk.Nc, L.stride);
  return hipGetLastError();
}

}  // namespace vsa
