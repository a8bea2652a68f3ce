// Packing of the selected KV blocks for sequence-sharded context parallelism.
//
// Method: the DSV pages ("DSV: Exploiting Dynamic Sparsity to Accelerate Large-Scale Video
// DiT Training", gist.science/de and /es, technical summary §2.C) shard long sequences over
// GPUs and exploit the sparsity so that only the KV that the selection needs moves between
// them.  The one-GPU share of that exchange: for a receiver's range of query blocks, the union
// of the KV blocks its lists select (per head, ascending), copied contiguously into a send
// buffer, and the lists rewritten to positions in that buffer -- so the receiver runs the
// unchanged sparse forward on (its Q, packed K, packed V, rewritten lists).
//
// Kernels: mark the union (a flag per KV block: every writer stores the same 1, after a fill),
// a per-head exclusive scan of the flags (one workgroup per head, deterministic), the copy of
// K and V rows block by block (16-byte lanes, HBM-bound), and the rewrite of the lists.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <mutex>

namespace dsv {

__global__ void pack_fill_kernel(int32_t* __restrict__ p, size_t n, int32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// one thread per list entry (bh, qb in [qb0, qb1), j)
__global__ void pack_mark_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnts,
                                 int32_t* __restrict__ flags, int nqb, int nkb, int topk, int qb0, int nsh,
                                 size_t total) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int j = (int)(t % topk);
  const size_t r = t / topk;  // bh * nsh + (qb - qb0)
  const size_t bh = r / nsh;
  const size_t row = bh * nqb + qb0 + (r % nsh);
  if (j >= list_len(cnts, row, topk)) return;
  const int kb = idx[row * topk + j];
  if ((unsigned)kb < (unsigned)nkb) flags[bh * nkb + kb] = 1;
}

// one workgroup per head: pos[kb] = rank of kb among the flagged blocks (-1 if unflagged),
// blocks[u] = the u-th flagged block (then -1), count = number flagged
__global__ __launch_bounds__(1024) void pack_scan_kernel(const int32_t* __restrict__ flags, int32_t* __restrict__ pos,
                                                         int32_t* __restrict__ blocks, int32_t* __restrict__ count,
                                                         int nkb) {
  __shared__ int wave_tot[16];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* f = flags + (size_t)bh * nkb;
  int base = 0;
  for (int c0 = 0; c0 < nkb; c0 += 1024) {
    const int kb = c0 + tid;
    const int v = kb < nkb ? f[kb] : 0;
    int incl = v;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    int chunk = 0;
    for (int w = 0; w < 16; ++w) chunk += wave_tot[w];
    const int p = base + before + incl - v;
    if (kb < nkb) {
      pos[(size_t)bh * nkb + kb] = v ? p : -1;
      if (v) blocks[(size_t)bh * nkb + p] = kb;
    }
    base += chunk;
    __syncthreads();
  }
  for (int u = base + tid; u < nkb; u += 1024) blocks[(size_t)bh * nkb + u] = -1;
  if (tid == 0) count[bh] = base;
}

// grid (nkb, bh): workgroup u copies block blocks[u] of K and V (if u < count) to rows u*64..;
// a block is 64 rows of row_bytes bytes at a 16-byte-aligned offset
__global__ __launch_bounds__(256) void pack_copy_kernel(const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                                                        uint8_t* __restrict__ kp, uint8_t* __restrict__ vp,
                                                        const int32_t* __restrict__ blocks,
                                                        const int32_t* __restrict__ count, int n, int nkb,
                                                        int row_bytes) {
  const int u = blockIdx.x, bh = blockIdx.y;
  if (u >= count[bh]) return;
  const int kb = blocks[(size_t)bh * nkb + u];
  const int block_bytes = 64 * row_bytes;
  const size_t src = ((size_t)bh * n + (size_t)kb * 64) * row_bytes;
  const size_t dst = ((size_t)bh * n + (size_t)u * 64) * row_bytes;
  for (int o = threadIdx.x * 16; o < block_bytes; o += 256 * 16) {
    st16(kp + dst + o, ld16(k + src + o));
    st16(vp + dst + o, ld16(v + src + o));
  }
}

// one thread per list entry of the shard: its position in the packed buffer (-1 past the count)
__global__ void pack_remap_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnts,
                                  const int32_t* __restrict__ pos, int32_t* __restrict__ out, int nqb, int nkb,
                                  int topk, int qb0, int nsh, size_t total) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int j = (int)(t % topk);
  const size_t r = t / topk;
  const size_t bh = r / nsh;
  const size_t row = bh * nqb + qb0 + (r % nsh);
  int val = -1;
  if (j < list_len(cnts, row, topk)) {
    const int kb = idx[row * topk + j];
    if ((unsigned)kb < (unsigned)nkb) val = pos[bh * nkb + kb];
  }
  out[t] = val;
}

hipError_t launch_pack_kv(const void* k, const void* v, const int32_t* idx, const int32_t* cnts, void* kp, void* vp,
                          int32_t* blocks, int32_t* count, int32_t* packed_idx, int32_t* flags, int32_t* pos, int bh,
                          int n, int row_bytes, int nqb, int nkb, int topk, int qb0, int qb1, hipStream_t st) {
  const size_t nflags = (size_t)bh * nkb;
  hipLaunchKernelGGL(pack_fill_kernel, dim3((unsigned)std::min<size_t>((nflags + 255) / 256, 65535)), dim3(256), 0, st,
                     flags, nflags, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nsh = qb1 - qb0;
  const size_t total = (size_t)bh * nsh * topk;
  if (total) {
    hipLaunchKernelGGL(pack_mark_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, idx, cnts, flags, nqb,
                       nkb, topk, qb0, nsh, total);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(pack_scan_kernel, dim3(bh), dim3(1024), 0, st, flags, pos, blocks, count, nkb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const uint8_t* k8 = static_cast<const uint8_t*>(k);
  const uint8_t* v8 = static_cast<const uint8_t*>(v);
  uint8_t* kp8 = static_cast<uint8_t*>(kp);
  uint8_t* vp8 = static_cast<uint8_t*>(vp);
  hipLaunchKernelGGL(pack_copy_kernel, dim3(nkb, bh), dim3(256), 0, st, k8, v8, kp8, vp8, blocks, count, n, nkb,
                     row_bytes);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (total) {
    hipLaunchKernelGGL(pack_remap_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, idx, cnts, pos,
                       packed_idx, nqb, nkb, topk, qb0, nsh, total);
    e = hipGetLastError();
  }
  return e;
}

// ---------------------------------------------------------------- allocation-free variant
//
// For callers that cannot allocate device memory (graph capture, tight serving loops): the
// flags and positions live in this file-scope device array instead of a caller workspace.
// Every GPU the library runs on holds its own copy until the process ends.  In host code the
// array's name is only a stand-in for the symbol: its device address, which differs per
// device, comes from hipGetSymbolAddress and is cached per device ordinal below; only that
// address is ever handed to a kernel.
static __device__ __align__(256) int32_t scratch[2 * kPackScratchEntries];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t pack_scratch(int32_t** flags, int32_t** pos) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy (the device is current)
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *flags = g_scratch_ptr[dev];
  *pos = g_scratch_ptr[dev] + kPackScratchEntries;
  return hipSuccess;
}

}  // namespace dsv
