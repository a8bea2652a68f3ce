// Critical-KV selection: top-k KV blocks per query block.
//
// Method: the DSV pages ("DSV: Exploiting Dynamic Sparsity to Accelerate
// Large-Scale Video DiT Training", gist.science/de and /es, technical summary
// §2.B) select the top-k critical KV pairs from the low-rank estimate; tokens of
// one query group share the selection.  Here the unit is the KV block: for each
// (b, h, query block) the k blocks with the largest predicted mass are kept,
// ties toward the smaller block index, and written in ascending block order.
//
// gfx950 design: one wave64 per query block.  Lane l holds blocks e*64 + l
// (e = 0 .. NPL-1), loaded coalesced, as order-preserving 32-bit keys; the
// wave-level search of topk_row.hpp picks the k largest.  The kernel is bound by
// the HBM read of the score rows.
#include "common.hpp"
#include "kernels.hpp"
#include "topk_row.hpp"

namespace dsv {

template <int NPL>
__global__ __launch_bounds__(256) void select_topk_kernel(const float* __restrict__ scores,
                                                          int32_t* __restrict__ idx, int rows, int nkb,
                                                          int k) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave exits together
  const float* src = scores + (size_t)row * nkb;
  uint32_t key[NPL];
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const int kb = e * 64 + lane;
    key[e] = kb < nkb ? max(order_key(src[kb]), 1u) : 0u;  // padding = 0, valid keys >= 1
  }
  topk_row<NPL>(key, k, idx + (size_t)row * k, lane);
}

// ---------------------------------------------------------------- mass-threshold selection
//
// The pages keep the critical KV blocks that carry most (~90%) of the attention score ([de]
// §2.A, [es] §2.A).  Per query block: the smallest set of KV blocks, taken by descending score
// with ties to the smaller index, whose scores sum to at least tau times the row's total;
// at most kmax blocks, never empty.  Output: ascending indices padded with -1 to kmax, and
// the count.
//
// One wave64 per query block, lane l holding blocks e*64 + l.  Each block gets a unique key
// (score key << 12 | (4095 - kb)), so descending key order is descending score with ties to
// the smaller index, and the chosen set is {key >= T} for one threshold T.  T is the largest
// key whose suffix mass S(T) = sum_{key >= T} score reaches the target, found by an MSB-first
// bisection; every S is a per-lane sum in block order followed by a fixed butterfly, so the
// result is deterministic.  A set larger than kmax is cut to its kmax largest keys by a second
// bisection on counts.

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <int NPL>
__global__ __launch_bounds__(256) void select_mass_kernel(const float* __restrict__ scores,
                                                          int32_t* __restrict__ idx, int32_t* __restrict__ cnts,
                                                          int rows, int nkb, int kmax, float tau) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave exits together
  const float* src = scores + (size_t)row * nkb;
  float val[NPL];
  uint64_t key[NPL];
  uint64_t kmaxkey = 0;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const int kb = e * 64 + lane;
    val[e] = kb < nkb ? src[kb] : 0.f;
    // padding keys are 0; valid keys are >= 1
    key[e] = kb < nkb ? ((uint64_t)max(order_key(val[e]), 1u) << 12) | (uint64_t)(4095 - kb) : 0ull;
    kmaxkey = key[e] > kmaxkey ? key[e] : kmaxkey;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(kmaxkey, off);
    kmaxkey = o > kmaxkey ? o : kmaxkey;
  }
  auto suffix_mass = [&](uint64_t t) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < NPL; ++e) acc += key[e] >= t ? val[e] : 0.f;
    return wave_sum(acc);
  };
  auto count_ge = [&](uint64_t t) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e) c += popc64(__ballot(key[e] >= t));
    return c;
  };
  const float target = tau * suffix_mass(1ull);
  uint64_t T = 0;
  for (int bit = 43; bit >= 0; --bit) {
    const uint64_t cand = T | (1ull << bit);
    if (cand <= kmaxkey && suffix_mass(cand) >= target) T = cand;
  }
  int m = count_ge(T);
  if (m > kmax) {  // keep the kmax largest keys
    T = 0;
    for (int bit = 43; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      if (count_ge(cand) >= kmax) T = cand;
    }
    m = kmax;
  }
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* dst = idx + (size_t)row * kmax;
  int taken = 0;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const bool sel = key[e] >= T && key[e] != 0ull;
    const uint64_t sel_m = __ballot(sel);
    if (sel) dst[taken + popc64(sel_m & lt_mask)] = e * 64 + lane;
    taken += popc64(sel_m);
  }
  for (int p = m + lane; p < kmax; p += 64) dst[p] = -1;
  if (lane == 0) cnts[row] = m;
}

hipError_t launch_select_mass(const float* scores, int32_t* idx, int32_t* cnts, int rows, int nkb, int kmax,
                              float tau, hipStream_t st) {
  const dim3 grid((rows + 3) / 4), block(256);
  const int npl = (nkb + 63) / 64;
#define SEL(N_)                                                                                          \
  if (npl <= N_) {                                                                                       \
    hipLaunchKernelGGL((select_mass_kernel<N_>), grid, block, 0, st, scores, idx, cnts, rows, nkb, kmax, tau); \
    return hipGetLastError();                                                                            \
  }
  SEL(1) SEL(2) SEL(4) SEL(8) SEL(16) SEL(32) SEL(64)
#undef SEL
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- recall of a selection
//
// The profiler's question ([de] §2.A: the critical KV carry most of the score): how much of a
// row's true attention mass do its selected blocks capture?  With LSE_J the log-sum-exp of the
// row's scaled logits over its selected keys (the sparse forward's lse) and LSE_all over all
// keys (the forward with every block selected), the captured mass is exp(LSE_J - LSE_all).
// One wave per query block averages it over the block's rows.
__global__ __launch_bounds__(256) void block_recall_kernel(const float* __restrict__ lse_sel,
                                                           const float* __restrict__ lse_all,
                                                           float* __restrict__ recall, int rows, int bq) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // bh * nqb + qb
  if (row >= rows) return;  // whole wave exits together
  const size_t base = (size_t)row * bq;
  float acc = 0.f;
  for (int i = lane; i < bq; i += 64) acc += expf(lse_sel[base + i] - lse_all[base + i]);
  acc = wave_sum(acc);
  if (lane == 0) recall[row] = acc / (float)bq;
}

hipError_t launch_block_recall(const float* lse_sel, const float* lse_all, float* recall, int rows, int bq,
                               hipStream_t st) {
  hipLaunchKernelGGL(block_recall_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, lse_sel, lse_all, recall, rows, bq);
  return hipGetLastError();
}

// ---------------------------------------------------------------- per-head density (activation)
//
// The pages switch a block of the model to sparse attention once it is sparse enough ([de] §2.A,
// stage 2).  The measure here: a head's selected density, its selected KV blocks summed over its
// query blocks (exact integers) over query blocks x KV blocks, and a dense flag, set when that sum
// exceeds `limit` = floor(dense_above * cells) (computed by the host).  One wave per head.
__global__ __launch_bounds__(256) void head_density_kernel(const int32_t* __restrict__ cnts, float* __restrict__ density,
                                                           int32_t* __restrict__ dense, int nqb, int k, int nkb,
                                                           long long limit, int bh_total) {
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= bh_total) return;  // whole wave exits together
  long long tot = 0;
  if (cnts) {
    for (int qb = lane; qb < nqb; qb += 64) tot += list_len(cnts, (size_t)bh * nqb + qb, k);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  } else {
    tot = (long long)k * nqb;
  }
  if (lane == 0) {
    density[bh] = (float)((double)tot / ((double)nqb * (double)nkb));
    if (dense) dense[bh] = tot > limit ? 1 : 0;
  }
}

hipError_t launch_head_density(const int32_t* cnts, float* density, int32_t* dense, int nqb, int k, int nkb,
                               long long limit, int bh, hipStream_t st) {
  hipLaunchKernelGGL(head_density_kernel, dim3((bh + 3) / 4), dim3(256), 0, st, cnts, density, dense, nqb, k, nkb,
                     limit, bh);
  return hipGetLastError();
}

hipError_t launch_select_topk(const float* scores, int32_t* idx, int rows, int nkb, int k, hipStream_t st) {
  const dim3 grid((rows + 3) / 4), block(256);
  const int npl = (nkb + 63) / 64;
#define SEL(N_)                                                                                   \
  if (npl <= N_) {                                                                                \
    hipLaunchKernelGGL((select_topk_kernel<N_>), grid, block, 0, st, scores, idx, rows, nkb, k); \
    return hipGetLastError();                                                                     \
  }
  SEL(1) SEL(2) SEL(4) SEL(8) SEL(16) SEL(32) SEL(64)
#undef SEL
  return hipErrorInvalidValue;
}

}  // namespace dsv
