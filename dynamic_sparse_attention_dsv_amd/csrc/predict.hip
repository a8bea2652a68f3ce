// Low-rank sparsity predictor: projection and predicted block mass.
//
// Method: the DSV pages ("DSV: Exploiting Dynamic Sparsity to Accelerate
// Large-Scale Video DiT Training", gist.science/es and /de, technical summary
// §2.A) train per-head low-rank matrices W^Q_lr, W^K_lr whose product
// approximates Q K^T, and use them to find the critical KV pairs -- those that
// carry most of the attention score -- without materialising the full matrix
// (§2.B, the fused matmul and top-k: no O(S^2) intermediate in HBM).  The quantity
// computed here is the predicted softmax mass of each query block on each KV
// block, summed over the block's rows:
//   score[qb, kb] = sum_{i in qb} sum_{j in kb} exp(l_ij - LSE_i),
//   l_ij = pred_scale <Q_lr_i, K_lr_j>,  LSE_i = log sum_j exp(l_ij).
//
// gfx950 design (bf16):
//  * projection: one MFMA 16x16x32 GEMM per 16-row tile, W^T held in registers;
//  * scores: persistent workgroups of 4 waves; each work item is 128 query rows
//    of one head.  Each wave sweeps every KV block once: a 32x32x16 MFMA
//    produces 32 rows x 64 keys of logits, the lane-local block max, exp2 and
//    sum give the block's log-mass t_i,kb (log2 domain), and an online
//    log-sum-exp over blocks gives LSE_i.  t_i,kb goes to a per-workgroup
//    scratch of nkb x 128 floats (never N x N); after the sweep the same
//    workgroup turns it into block scores.  The sweep is bound by the vector
//    ALU (one exp2 per logit), not by MFMA or memory.
#include "common.hpp"
#include "kernels.hpp"

namespace dsv {

// ---------------------------------------------------------------- projection (bf16)

template <int D, int R>
__global__ __launch_bounds__(256) void proj_bf16_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w,
                                                        uint16_t* __restrict__ out, int n, int heads) {
  // grid: (ceil(n/256), B*H). x, out: [BH, n, D] / [BH, n, R]; w: [H, D, R].
  const int bh = blockIdx.y;
  const int h = bh % heads;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const uint16_t* wh = w + (size_t)h * D * R;
  // A operand = W^T [R x D]: lane holds row r = rt*16 + c16, k = kc*32 + g*8 + e
  bf16x8 wa[R / 16][D / 32];
#pragma unroll
  for (int rt = 0; rt < R / 16; ++rt)
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = bf16_to_f32(wh[(size_t)(kc * 32 + g * 8 + e) * R + rt * 16 + c16]);
      wa[rt][kc] = cvt8(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
    }
  const uint16_t* xb = x + (size_t)bh * n * D;
  uint16_t* ob = out + (size_t)bh * n * R;
  const int tiles = n / 16;
  for (int t = blockIdx.x * 16 + wave; t < min(tiles, (int)(blockIdx.x + 1) * 16); t += 4) {
    const int row = t * 16 + c16;
    bf16x8 xb8[D / 32];
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) xb8[kc] = as_bf16x8(ld16(xb + (size_t)row * D + kc * 32 + g * 8));
#pragma unroll
    for (int rt = 0; rt < R / 16; ++rt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < D / 32; ++kc) acc = mfma16(wa[rt][kc], xb8[kc], acc);
      // D layout: lane holds col (row index) c16, registers rows r = rt*16 + g*4 + v
      u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(ob + (size_t)row * R + rt * 16 + g * 4) = pk;
    }
  }
}

// ---------------------------------------------------------------- projection (f32)

__global__ void proj_f32_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                float* __restrict__ out, int n, int d, int r, int heads) {
  // grid: (ceil(n*r/256), B*H)
  const int bh = blockIdx.y;
  const int h = bh % heads;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)n * r) return;
  const int row = (int)(i / r), col = (int)(i % r);
  const float* xr = x + ((size_t)bh * n + row) * d;
  const float* wc = w + (size_t)h * d * r + col;
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wc[(size_t)c * r], acc);
  out[((size_t)bh * n + row) * r + col] = acc;
}

// ---------------------------------------------------------------- scores (bf16, MFMA)

constexpr int kScoreRows = 256;  // query rows per work item (4 waves x 64)

template <int R, int BQ>
__global__ __launch_bounds__(256) void scores_bf16_kernel(const uint16_t* __restrict__ qlr,
                                                          const uint16_t* __restrict__ klr,
                                                          float* __restrict__ scratch,
                                                          float* __restrict__ scores, int n, int nkb,
                                                          int items, float pc) {
  // qlr, klr: [BH, n, R] bf16.  scratch: gridDim.x slots of [nkb][256] float.
  // scores: [BH, n/BQ, nkb].  pc = pred_scale * log2(e).
  // Each wave owns 64 query rows (two 32-row halves): every K_lr fragment it loads feeds
  // two MFMA tiles, halving the K_lr traffic per logit.
  static_assert(kScoreRows % BQ == 0 && BQ % 64 == 0, "BQ must be 64 or 128");
  constexpr int NC = R / 16;
  __shared__ float lse2_s[kScoreRows];
  __shared__ float part_s[4][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  float* slot = scratch + (size_t)blockIdx.x * nkb * kScoreRows;
  const int items_per_head = n / kScoreRows;

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int bh = item / items_per_head;
    const int row0 = (item % items_per_head) * kScoreRows;
    const uint16_t* kh = klr + (size_t)bh * n * R;
    // B operands = Q_lr^T for the wave's two 32-row halves: lane holds its query row, 8 consecutive r
    bf16x8 qf[2][NC];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t* qrow = qlr + ((size_t)bh * n + row0 + wave * 64 + h * 32 + c32) * R;
#pragma unroll
      for (int c = 0; c < NC; ++c) qf[h][c] = as_bf16x8(ld16(qrow + c * 16 + g * 8));
    }
    // A operands (K_lr rows, 8 consecutive r) of one KV block: 2 tiles x NC chunks
    auto load_k = [&](int kb, u32x4 (&ka)[2][NC]) {
      const uint16_t* kp = kh + (size_t)kb * 64 * R;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) ka[t][c] = ld16(kp + (size_t)(t * 32 + c32) * R + c * 16 + g * 8);
    };
    auto logits = [&](const u32x4 (&ka)[2][NC], f32x16 (&acc)[2][2]) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc[h][t] = f32x16{};
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[h][t] = mfma32(as_bf16x8(ka[t][c]), qf[h][c], acc[h][t]);
        }
    };
    float run_m[2], run_s[2];
    auto fold = [&](int h, float t2) {  // online log-sum-exp over blocks
      const float nm = fmaxf(run_m[h], t2);
      run_s[h] = run_s[h] * fast_exp2(run_m[h] - nm) + fast_exp2(t2 - nm);
      run_m[h] = nm;
    };
    // block mass of half h with shift sh (log2 units): t = sh + log2 sum_j 2^(pc a_ij - sh)
    auto block_t2 = [&](const f32x16 (&acc)[2], float sh) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s0 += fast_exp2(fmaf(acc[0][v], pc, -sh));
        s1 += fast_exp2(fmaf(acc[1][v], pc, -sh));
      }
      return sh + fast_log2(sum_xor32(s0 + s1));
    };
    auto own_max = [&](const f32x16 (&acc)[2]) {  // the block's largest logit, log2 units
      float m0 = acc[0][0], m1 = acc[1][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) {
        m0 = fmaxf(m0, acc[0][v]);
        m1 = fmaxf(m1, acc[1][v]);
      }
      return max_xor32(fmaxf(m0, m1)) * pc;
    };
    auto store = [&](int kb, int h, float t2) {
      if (g == 0) slot[(size_t)kb * kScoreRows + wave * 64 + h * 32 + c32] = t2;
    };
    // Fast sweep.  Block 0 is shifted by its own max; every later block by the row's running
    // log-mass bound one block back (>= each earlier logit, up to +6), so no per-block max is
    // needed and consecutive blocks stay independent.  A logit more than 127 above that bound
    // would overflow; this is detected once per item below and the item is redone exactly.
    u32x4 ka[2][NC], kn[2][NC];
    f32x16 cur[2][2], nxt[2][2];
    float lag[2];
    load_k(0, ka);
    if (nkb > 1) load_k(1, kn);
    logits(ka, cur);
    if (nkb > 1) logits(kn, nxt);
    if (nkb > 2) load_k(2, kn);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float t0 = block_t2(cur[h], own_max(cur[h]));
      store(0, h, t0);
      run_m[h] = t0;
      run_s[h] = 1.f;
      lag[h] = t0;
    }
    // steady state without branches: issue block kb+1, prefetch kb+2 (clamped), finish kb
    for (int kb = 1; kb + 1 < nkb; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        cur[h][0] = nxt[h][0];
        cur[h][1] = nxt[h][1];
      }
      logits(kn, nxt);
      load_k(min(kb + 2, nkb - 1), kn);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float t2 = block_t2(cur[h], lag[h]);
        store(kb, h, t2);
        lag[h] = run_m[h];
        fold(h, t2);
      }
    }
    if (nkb > 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float t2 = block_t2(nxt[h], lag[h]);
        store(nkb - 1, h, t2);
        fold(h, t2);
      }
    }
    // an overflowed row redoes the item with a per-block max (the exact path)
    if (__syncthreads_or(!(run_m[0] + fast_log2(run_s[0]) < INFINITY) ||
                         !(run_m[1] + fast_log2(run_s[1]) < INFINITY))) {
      for (int kb = 0; kb < nkb; ++kb) {
        load_k(kb, ka);
        logits(ka, cur);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float t2 = block_t2(cur[h], own_max(cur[h]));
          store(kb, h, t2);
          if (kb == 0) {
            run_m[h] = t2;
            run_s[h] = 1.f;
          } else {
            fold(h, t2);
          }
        }
      }
    }
    if (g == 0) {
      lse2_s[wave * 64 + c32] = run_m[0] + fast_log2(run_s[0]);
      lse2_s[wave * 64 + 32 + c32] = run_m[1] + fast_log2(run_s[1]);
    }
    __threadfence_block();
    __syncthreads();

    // finalize: score[qb, kb] = sum_{i in qb} 2^(t2[kb][i] - lse2[i]).
    // chunks of 64 KV blocks: lane <-> kb, wave w sums its rows [64w, 64w+64).
    float* sc_head = scores + (size_t)bh * (n / BQ) * nkb;
    const int qb0 = row0 / BQ;
    for (int kb0 = 0; kb0 < nkb; kb0 += 64) {
      const int kb = kb0 + lane;
      float acc0 = 0.f, acc1 = 0.f;
      if (kb < nkb) {
        const float* src = slot + (size_t)kb * kScoreRows + wave * 64;
        const float* ls = lse2_s + wave * 64;
#pragma unroll
        for (int i = 0; i < 64; i += 4) {
          const f32x4 tv = *reinterpret_cast<const f32x4*>(src + i);
          acc0 += fast_exp2(tv[0] - ls[i]) + fast_exp2(tv[1] - ls[i + 1]);
          acc1 += fast_exp2(tv[2] - ls[i + 2]) + fast_exp2(tv[3] - ls[i + 3]);
        }
      }
      part_s[wave][lane] = acc0 + acc1;
      __syncthreads();
      constexpr int QBS = kScoreRows / BQ;    // query blocks per item
      constexpr int WPQ = BQ / 64;            // waves per query block
      if (threadIdx.x < 64 * QBS) {
        const int qq = threadIdx.x / 64, kk = kb0 + (threadIdx.x & 63);
        if (kk < nkb) {
          float tot = 0.f;
#pragma unroll
          for (int w = 0; w < WPQ; ++w) tot += part_s[qq * WPQ + w][threadIdx.x & 63];
          sc_head[(size_t)(qb0 + qq) * nkb + kk] = tot;
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- scores (f32, plain VALU)

__global__ void row_lse_f32_kernel(const float* __restrict__ qlr, const float* __restrict__ klr,
                                   float* __restrict__ lse, int n, int r, float ps, int bhn) {
  // one thread per query row; two passes over all keys (max, then sum)
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= bhn) return;
  const int bh = i / n;
  const float* q = qlr + (size_t)i * r;
  const float* kh = klr + (size_t)bh * n * r;
  float m = -INFINITY;
  for (int j = 0; j < n; ++j) {
    float a = 0.f;
    for (int c = 0; c < r; ++c) a = fmaf(q[c], kh[(size_t)j * r + c], a);
    m = fmaxf(m, a * ps);
  }
  float s = 0.f;
  for (int j = 0; j < n; ++j) {
    float a = 0.f;
    for (int c = 0; c < r; ++c) a = fmaf(q[c], kh[(size_t)j * r + c], a);
    s += expf(a * ps - m);
  }
  lse[i] = m + logf(s);
}

__global__ void scores_f32_kernel(const float* __restrict__ qlr, const float* __restrict__ klr,
                                  const float* __restrict__ lse, float* __restrict__ scores, int n, int r,
                                  int bq, int bk, float ps, int total) {
  // one thread per (bh, qb, kb)
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int nkb = n / bk, nqb = n / bq;
  const int kb = t % nkb, qb = (t / nkb) % nqb, bh = t / (nkb * nqb);
  const float* qh = qlr + (size_t)bh * n * r;
  const float* kh = klr + (size_t)bh * n * r;
  float acc = 0.f;
  for (int i = qb * bq; i < (qb + 1) * bq; ++i) {
    const float li = lse[(size_t)bh * n + i];
    for (int j = kb * bk; j < (kb + 1) * bk; ++j) {
      float a = 0.f;
      for (int c = 0; c < r; ++c) a = fmaf(qh[(size_t)i * r + c], kh[(size_t)j * r + c], a);
      acc += expf(a * ps - li);
    }
  }
  scores[t] = acc;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_proj_bf16(const uint16_t* x, const uint16_t* w, uint16_t* out, int bh, int n, int heads,
                            int d, int r, hipStream_t st) {
  dim3 grid((n + 255) / 256, bh);
#define PROJ(D_, R_)                                                                                  \
  if (d == D_ && r == R_) {                                                                           \
    hipLaunchKernelGGL((proj_bf16_kernel<D_, R_>), grid, dim3(256), 0, st, x, w, out, n, heads);      \
    return hipGetLastError();                                                                         \
  }
  PROJ(64, 16) PROJ(64, 32) PROJ(128, 16) PROJ(128, 32)
#undef PROJ
  return hipErrorInvalidValue;
}

hipError_t launch_proj_f32(const float* x, const float* w, float* out, int bh, int n, int heads, int d,
                           int r, hipStream_t st) {
  dim3 grid((unsigned)(((size_t)n * r + 255) / 256), bh);
  hipLaunchKernelGGL(proj_f32_kernel, grid, dim3(256), 0, st, x, w, out, n, d, r, heads);
  return hipGetLastError();
}

int score_slots(int items) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
  }
  const int slots = cus * 4;  // 4 resident workgroups (16 waves) per compute unit
  return items < slots ? items : slots;
}

size_t score_scratch_bytes(int items, int nkb) {
  return (size_t)score_slots(items) * nkb * kScoreRows * sizeof(float);
}

hipError_t launch_scores_bf16(const uint16_t* qlr, const uint16_t* klr, float* scratch, float* scores,
                              int bh, int n, int nkb, int r, int bq, float pred_scale, hipStream_t st) {
  const int items = bh * (n / kScoreRows);
  const int slots = score_slots(items);
  const float pc = pred_scale * kLog2e;
#define SC(R_, BQ_)                                                                                    \
  if (r == R_ && bq == BQ_) {                                                                          \
    hipLaunchKernelGGL((scores_bf16_kernel<R_, BQ_>), dim3(slots), dim3(256), 0, st, qlr, klr, scratch, \
                       scores, n, nkb, items, pc);                                                     \
    return hipGetLastError();                                                                          \
  }
  SC(16, 64) SC(16, 128) SC(32, 64) SC(32, 128)
#undef SC
  return hipErrorInvalidValue;
}

hipError_t launch_scores_f32(const float* qlr, const float* klr, float* lse, float* scores, int bh, int n,
                             int r, int bq, int bk, float pred_scale, hipStream_t st) {
  const int bhn = bh * n;
  hipLaunchKernelGGL(row_lse_f32_kernel, dim3((bhn + 255) / 256), dim3(256), 0, st, qlr, klr, lse, n, r,
                     pred_scale, bhn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = bh * (n / bq) * (n / bk);
  hipLaunchKernelGGL(scores_f32_kernel, dim3((total + 255) / 256), dim3(256), 0, st, qlr, klr, lse, scores,
                     n, r, bq, bk, pred_scale, total);
  return hipGetLastError();
}

}  // namespace dsv
