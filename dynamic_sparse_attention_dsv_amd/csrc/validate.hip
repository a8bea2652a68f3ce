// Optional device-side check of block lists (DSV_DEBUG_VALIDATE=1): the attention calls are
// defined only for lists whose used entries are distinct indices in [0, N/Bk).  One wave per
// query block marks its entries in a bitmap in LDS; an entry out of range, or one whose bit is
// already set, makes the query block bad.  The number of bad query blocks is counted in a device
// word of the library (one per GPU) that the host reads after the check.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace dsv {

static __device__ __align__(256) uint32_t bad_lists[1];  // the count of bad query blocks (each GPU has its own copy)

__global__ void clear_count_kernel(uint32_t* __restrict__ c) {
  if (threadIdx.x == 0) c[0] = 0u;
}

__global__ __launch_bounds__(256) void check_lists_kernel(const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ cnts,
                                                          uint32_t* __restrict__ bad, int rows, int nkb, int k) {
  __shared__ uint32_t seen_s[4][4096 / 32];  // N/Bk <= 4096 blocks: one bit each, per wave
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + w;
  if (row >= rows) return;  // whole wave; no workgroup barrier below
  uint32_t* seen = seen_s[w];
  for (int i = lane; i < 4096 / 32; i += 64) seen[i] = 0u;
  __builtin_amdgcn_wave_barrier();  // one wave's LDS operations complete in order
  const int used = list_len(cnts, (size_t)row, k);
  const int32_t* list = idx + (size_t)row * k;
  bool wrong = false;
  for (int j = lane; j < used; j += 64) {
    const int kb = list[j];
    if ((unsigned)kb >= (unsigned)nkb) {
      wrong = true;
      continue;
    }
    const uint32_t bit = 1u << (kb & 31);
    if (atomicOr(&seen[kb >> 5], bit) & bit) wrong = true;  // seen before: a repeated entry
  }
  if (__any(wrong) && lane == 0) atomicAdd(bad, 1u);
}

namespace {
std::mutex g_mu;
uint32_t* g_count[64] = {};
}  // namespace

hipError_t check_block_lists(const int32_t* idx, const int32_t* cnts, int rows, int nkb, int k, hipStream_t st,
                             uint32_t* bad_rows) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  uint32_t* count = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_count[dev]) {
      void* p = nullptr;
      if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(bad_lists))) != hipSuccess) return e;  // this device's copy
      if (!p) return hipErrorInvalidSymbol;
      g_count[dev] = static_cast<uint32_t*>(p);
    }
    count = g_count[dev];
  }
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(64), 0, st, count);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(check_lists_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, idx, cnts, count, rows, nkb, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
  return hipMemcpy(bad_rows, count, sizeof(uint32_t), hipMemcpyDeviceToHost);
}

}  // namespace dsv
