// Copies of bf16 tensors in fp16 with a power-of-two per-head scale.
//
// The attention kernels take a few products in fp16 (P V in the training forward, S and dQ in
// the dQ kernel): fp16 keeps 11 significant bits against bf16's 8, so a value rounded to fp16
// carries 8x less error, and a bf16 input converts exactly.  fp16's range is narrow (largest
// finite 65504, normal down to 2^-14), so each head's tensor is scaled by 2^s with s chosen from
// the head's largest magnitude (f16_shift): the maximum lands in [2^14, 2^15) and every element
// down to 2^-28 of it stays exact.  The consumers undo the scale exactly (ldexp).
//
// Kernels: partial maxima of |x| per head (kAbsmaxParts workgroups per head, deterministic, no
// atomics), their reduction to one value per head, and the scaled copy (16-byte lanes).
#include "common.hpp"
#include "kernels.hpp"

namespace dsv {

// |x| of a bf16 value orders like its bit pattern with the sign cleared; maxima are kept as the
// float bits of the largest |x|
__global__ __launch_bounds__(256) void absmax_part_kernel(const uint16_t* __restrict__ x, uint32_t* __restrict__ part,
                                                          size_t per_head /* elements, multiple of 8 */) {
  __shared__ uint32_t red[4];
  const int bh = blockIdx.y, ch = blockIdx.x;
  const size_t units = per_head / 8;  // 16-byte units
  const size_t chunk = (units + kAbsmaxParts - 1) / kAbsmaxParts;
  const size_t u0 = ch * chunk, u1 = min(units, u0 + chunk);
  const uint16_t* src = x + (size_t)bh * per_head;
  uint32_t m = 0;
  for (size_t u = u0 + threadIdx.x; u < u1; u += 256) {
    const u32x4 w = ld16(src + u * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) m = max(m, max((w[e] & 0x7fffu) << 16, w[e] & 0x7fff0000u));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[bh * kAbsmaxParts + ch] = max(max(red[0], red[1]), max(red[2], red[3]));
}

// one wave per head
__global__ __launch_bounds__(256) void absmax_final_kernel(const uint32_t* __restrict__ part,
                                                           uint32_t* __restrict__ maxbits, int bh_total) {
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (bh >= bh_total) return;  // whole wave exits together
  uint32_t m = lane < kAbsmaxParts ? part[bh * kAbsmaxParts + lane] : 0u;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if (lane == 0) maxbits[bh] = m;
}

// grid (ceil(per_head / 2048), BH): 8 elements per thread
__global__ __launch_bounds__(256) void to_f16_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ maxbits,
                                                     uint16_t* __restrict__ y, size_t per_head, int wide) {
  const int bh = blockIdx.y;
  const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= per_head / 8) return;
  const int s = wide ? f16_shift_wide(maxbits[bh]) : f16_shift(maxbits[bh]);
  const u32x4 w = ld16(x + (size_t)bh * per_head + u * 8);
  float f[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = ldexpf(__uint_as_float(w[e] << 16), s);
    f[2 * e + 1] = ldexpf(__uint_as_float(w[e] & 0xffff0000u), s);
  }
  st16(y + (size_t)bh * per_head + u * 8, __builtin_bit_cast(u32x4, cvt8h(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7])));
}

size_t head_absmax_ws_bytes(int bh) { return align_ws((size_t)bh * kAbsmaxParts * 4); }

hipError_t launch_head_absmax(const uint16_t* x, uint32_t* part, uint32_t* maxbits, int bh, size_t per_head,
                              hipStream_t st) {
  hipLaunchKernelGGL(absmax_part_kernel, dim3(kAbsmaxParts, bh), dim3(256), 0, st, x, part, per_head);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(absmax_final_kernel, dim3((bh + 3) / 4), dim3(256), 0, st, part, maxbits, bh);
  return hipGetLastError();
}

hipError_t launch_to_f16(const uint16_t* x, const uint32_t* maxbits, uint16_t* y, int bh, size_t per_head,
                         hipStream_t st, bool wide) {
  hipLaunchKernelGGL(to_f16_kernel, dim3((unsigned)((per_head / 8 + 255) / 256), bh), dim3(256), 0, st, x, maxbits, y,
                     per_head, wide ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dsv
