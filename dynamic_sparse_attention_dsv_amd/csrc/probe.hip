// Peak-rate probes: the sustained rates of this device that the hot path's kernels are held
// against (MFMA for the attention products, the transcendental unit for the predictor's one
// exponential per logit, HBM for the copies and the selection).  Each probe is a kernel that does
// nothing but the operation it measures, over enough waves to fill every SIMD:
//  * MFMA: eight independent 32x32x16 accumulator chains per wave (bf16 or fp16 operands held in
//    registers), two waves per SIMD;
//  * exp: eight independent chains x <- 2^-x per lane (one v_exp_f32 each, values stay in
//    [0.5, 1]), eight waves per SIMD;
//  * copy: a grid-stride 16-byte copy of a buffer larger than the last-level cache, four loads
//    in flight per thread;
//  * read: the same grid-stride walk over a buffer, loads only (folded into one value per thread).
// The MFMA and exp probes store one float per thread so that no work is dead.
#include "common.hpp"
#include "kernels.hpp"

namespace dsv {

constexpr int kProbeChains = 8;

template <bool F16>
__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(float* __restrict__ out, int iters, float seed) {
  const float x = seed * (float)(threadIdx.x + 1), y = seed * 0.5f;
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x16{};
  if constexpr (F16) {
    const f16x8 a = cvt8h(x, x, x, x, x, x, x, x), b = cvt8h(y, y, y, y, y, y, y, y);
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma32h(a, b, acc[c]);
  } else {
    const bf16x8 a = cvt8(x, x, x, x, x, x, x, x), b = cvt8(y, y, y, y, y, y, y, y);
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void exp_probe_kernel(float* __restrict__ out, int iters, float seed) {
  float x[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) x[c] = seed + 0.01f * (float)c + 1e-4f * (float)threadIdx.x;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) x[c] = fast_exp2(-x[c]);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) s += x[c];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// four loads in flight per thread (a strided group of four 16-byte elements per trip)
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * stride < n) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * stride < n) dst[i + u * stride] = v[u];
  }
}

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, size_t n,
                                                         uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += 4 * stride) {
    u32x4 v[4] = {};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * stride < n) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

static int probe_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
  }
  return cus < kProbeMaxCus ? cus : kProbeMaxCus;
}

hipError_t launch_peak_probe(int kind, void* ws, size_t ws_bytes, hipStream_t st, double* work) {
  const int cus = probe_cus();
  switch (kind) {
    case 0:
    case 1: {  // two 4-wave workgroups per compute unit: two waves per SIMD
      const int grid = cus * 2, iters = 4096;
      if (kind == 0)
        hipLaunchKernelGGL((mfma_probe_kernel<false>), dim3(grid), dim3(256), 0, st, static_cast<float*>(ws), iters,
                           1e-3f);
      else
        hipLaunchKernelGGL((mfma_probe_kernel<true>), dim3(grid), dim3(256), 0, st, static_cast<float*>(ws), iters,
                           1e-3f);
      *work = (double)grid * 4 * iters * kProbeChains * (2.0 * 32 * 32 * 16);
      return hipGetLastError();
    }
    case 2: {  // eight 4-wave workgroups per compute unit: eight waves per SIMD
      const int grid = cus * 8, iters = 2048;
      hipLaunchKernelGGL(exp_probe_kernel, dim3(grid), dim3(256), 0, st, static_cast<float*>(ws), iters, 0.5f);
      *work = (double)grid * 256 * iters * kProbeChains;
      return hipGetLastError();
    }
    case 3: {  // read the first half of the workspace, write the second
      const size_t n = ws_bytes / 2 / sizeof(u32x4);
      const u32x4* src = static_cast<const u32x4*>(ws);
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(ws) + n * sizeof(u32x4));
      hipLaunchKernelGGL(copy_probe_kernel, dim3(cus * 8), dim3(256), 0, st, src, dst, n);
      *work = 2.0 * (double)n * sizeof(u32x4);
      return hipGetLastError();
    }
    case 4: {  // read the first kProbeCopyBytes of the workspace; one word per thread after them
      const size_t n = kProbeCopyBytes / sizeof(u32x4);
      uint32_t* out = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kProbeCopyBytes);
      hipLaunchKernelGGL(read_probe_kernel, dim3(cus * 8), dim3(256), 0, st, static_cast<const u32x4*>(ws), n, out);
      *work = (double)n * sizeof(u32x4);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace dsv
