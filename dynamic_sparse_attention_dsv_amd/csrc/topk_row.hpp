// Wave-level top-k of one row of float scores, shared by the selection kernel and the fused
// representative-row predictor.  The k largest values, ties toward the smaller index, written
// in ascending index order.
#pragma once

#include "common.hpp"

namespace dsv {

// Order-preserving 32-bit key of a float (a NaN sorts above +inf).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// One wave: lane l holds the keys of indices e*64 + l (e < NPL) in key[e]: valid keys are >= 1,
// padding past the row's length is 0.  At least k valid keys exist.  An MSB-first search over
// ballots finds the k-th largest key T; ties at T are kept in ascending index order through a
// running prefix count, so the output positions fall out of the same ballots.
template <int NPL>
__device__ __forceinline__ void topk_row(const uint32_t (&key)[NPL], int k, int32_t* dst, int lane) {
  uint32_t prefix = 0;  // T = the largest value with count(key >= T) >= k
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e) cnt += popc64(__ballot(key[e] >= cand));
    if (cnt >= k) prefix = cand;
  }
  const uint32_t T = prefix;
  int gt = 0;
#pragma unroll
  for (int e = 0; e < NPL; ++e) gt += popc64(__ballot(key[e] > T));
  const int need = k - gt;  // ties at T to keep, smallest index first
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int taken = 0, ties_seen = 0;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const bool tie = key[e] == T && key[e] != 0u;
    const uint64_t tie_m = __ballot(tie);
    const int tie_rank = ties_seen + popc64(tie_m & lt_mask);
    const bool sel = key[e] > T || (tie && tie_rank < need);
    const uint64_t sel_m = __ballot(sel);
    if (sel) dst[taken + popc64(sel_m & lt_mask)] = e * 64 + lane;
    taken += popc64(sel_m);
    ties_seen += popc64(tie_m);
  }
}

}  // namespace dsv
