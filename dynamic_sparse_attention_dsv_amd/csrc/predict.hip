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
//    the query side is scaled by pred_scale * log2(e) before its one rounding to
//    bf16, so that the query operand Q~ = bf16(pred_scale log2(e) Q W^Q_lr)
//    against K_lr = bf16(K W^K_lr) gives each logit in log2 units;
//  * scores: persistent workgroups of 4 waves; each work item is 256 query rows
//    of one head, 64 per wave.  Each wave sweeps every KV block once: one bf16
//    32x32x16 MFMA product of Q~ and K_lr gives the logits in log2 units, and 2^l
//    summed over the block's 64 keys gives the row's block mass.  Block masses go to
//    a per-workgroup scratch of nkb x 256 floats (never N x N); the row totals are
//    their sums, and the same workgroup divides and sums them into block scores
//    while it sweeps its next item (two scratch halves per workgroup).  The sweep is
//    bound by the vector ALU (one exp2 and one add per logit), not by MFMA or memory.
#include "common.hpp"
#include "kernels.hpp"
#include "topk_row.hpp"

namespace dsv {

// ---------------------------------------------------------------- projection (bf16)

template <int D, int R>
__global__ __launch_bounds__(256) void proj_bf16_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ w,
                                                        uint16_t* __restrict__ out, int n, int heads, float scale) {
  // grid: (ceil(n/256), B*H). x, out: [BH, n, D] / [BH, n, R]; w: [H, D, R].
  // out = bf16(scale * x w): the fp32 product is scaled, then rounded once (scale = 1: exact no-op).
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
      u32x2 pk = {pack_bf16x2(acc[0] * scale, acc[1] * scale), pack_bf16x2(acc[2] * scale, acc[3] * scale)};
      *reinterpret_cast<u32x2*>(ob + (size_t)row * R + rt * 16 + g * 4) = pk;
    }
  }
}

// ---------------------------------------------------------------- projection (f32)

__global__ void proj_f32_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                float* __restrict__ out, int n, int d, int r, int heads, float scale) {
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
  out[((size_t)bh * n + row) * r + col] = acc * scale;
}

// ---------------------------------------------------------------- scores (bf16, MFMA)

constexpr int kScoreRows = 256;  // query rows per work item (4 waves x 64)

// REP = false: work-item rows are 256 consecutive query rows; a score sums its query block's rows.
// REP = true (representative rows, [de] §2.B query grouping): work-item rows are the rows
// qb * BQ + rep of 256 consecutive query blocks, and a score is that one row's mass.
template <int R, int BQ, bool REP>
__global__ __launch_bounds__(256) void scores_bf16_kernel(const uint16_t* __restrict__ qlr,
                                                          const uint16_t* __restrict__ klr,
                                                          float* __restrict__ scratch,
                                                          float* __restrict__ scores, int n, int nkb,
                                                          int items, int rep) {
  // qlr, klr: [BH, n, R] bf16, qlr the scaled query projection Q~ (logits <Q~_i, K_lr_j> in log2
  // units).  scratch: gridDim.x slots of two [nkb][256] float halves (REP: one).  scores:
  // [BH, n/BQ, nkb].
  // Each wave owns 64 query rows (two 32-row halves): every K_lr fragment it loads feeds
  // two MFMA tiles, halving the K_lr traffic per logit.
  //
  // Each MFMA result is already a logit in log2 units (the projection carries the scale), so the
  // fast sweep takes 2^logit with no shift and sums block masses linearly: one exp and one add per
  // logit.  That is exact (up to rounding) for
  // rows whose total mass T = sum_j 2^l_ij lies in [2^-100, fp32 max]; an item holding any
  // other row is redone with a per-block maximum in the log domain.
  static_assert(kScoreRows % BQ == 0 && BQ % 64 == 0, "BQ must be 64 or 128");
  constexpr int NC = R / 16;
  constexpr float kTinyMass = 7.888609052210118e-31f;  // 2^-100
  __shared__ float row_s[2][kScoreRows];  // per slot half: 1/T (fast path) or log2 T (exact path) per row
  __shared__ float part_s[4][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const size_t slot_elems = (size_t)nkb * kScoreRows;
  float* const slots = scratch + (size_t)blockIdx.x * (REP ? 1 : 2) * slot_elems;
  const int nqb = n / BQ;
  const int items_per_head = REP ? (nqb + kScoreRows - 1) / kScoreRows : n / kScoreRows;

  // Exact-path finalisation, at once after the item's sweep: score[qb, kb] = sum_{i in qb}
  // 2^(t[kb][i] - log2 T_i) over the log-domain block masses t.  Chunks of 64 KV blocks: lane <-> kb,
  // wave w sums its rows [64w, 64w+64).
  auto finalize_exact = [&](const float* sl, const float* rs_all, float* sc_head, int qb0) {
    for (int kb0 = 0; kb0 < nkb; kb0 += 64) {
      const int kb = kb0 + lane;
      float acc0 = 0.f, acc1 = 0.f;
      if (kb < nkb) {
        const float* src = sl + (size_t)kb * kScoreRows + wave * 64;
        const float* rs = rs_all + wave * 64;
#pragma unroll
        for (int i = 0; i < 64; i += 4) {
          const f32x4 tv = *reinterpret_cast<const f32x4*>(src + i);
          acc0 += fast_exp2(tv[0] - rs[i]) + fast_exp2(tv[1] - rs[i + 1]);
          acc1 += fast_exp2(tv[2] - rs[i + 2]) + fast_exp2(tv[3] - rs[i + 3]);
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
  };

  // Deferred finalisation (fast path, REP = false).  A fast item's masses stay in one half of the
  // slot while the next item's sweep fills the other half; that sweep finalises them in passing,
  // one 16-row step per trip, so the HBM-bound reads overlap the VALU-bound sweeps of the whole
  // grid instead of running in step across all slots.  Wave w owns the chunks of 64 KV blocks
  // w, w + 4, ...; each step of a wave reads 16 rows of one chunk for the lane's KV block and adds
  // them, weighted by 1/T, into the running score of their query block.
  bool pend = false;  // the other half holds a fast item still to be finalised
  int pbh = 0, pqb0 = 0, buf = 0;
  const int nch = (nkb + 63) / 64;
  const int nchw = wave < nch ? (nch - 1 - wave) / 4 + 1 : 0;

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int bh = item / items_per_head;
    const int row0 = (item % items_per_head) * kScoreRows;  // first row, or first query block (REP)
    float* const slot = slots + (size_t)buf * slot_elems;
    // query row of the item's local row i (REP: past the last query block the row is clamped
    // to a valid one and its scores are never written)
    auto qrow_of = [&](int i) { return REP ? min(row0 + i, nqb - 1) * BQ + rep : row0 + i; };
    const uint16_t* kh = klr + (size_t)bh * n * R;
    // B operands = Q~^T for the wave's two 32-row halves: lane holds its query row, 8 consecutive
    // r per chunk
    bf16x8 qh[2][NC];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint16_t* qrow = qlr + ((size_t)bh * n + qrow_of(wave * 64 + h * 32 + c32)) * R;
#pragma unroll
      for (int c = 0; c < NC; ++c) qh[h][c] = as_bf16x8(ld16(qrow + c * 16 + g * 8));
    }
    // A operands (K_lr rows, 8 consecutive r) of one KV block: 2 tiles x NC chunks
    auto load_k = [&](int kb, u32x4 (&ka)[2][NC]) {
      const uint16_t* kp = kh + (size_t)kb * 64 * R;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) ka[t][c] = ld16(kp + (size_t)(t * 32 + c32) * R + c * 16 + g * 8);
    };
    // logits in log2 units: lane holds query c32 of half h, registers hold 16 of each tile's keys
    auto logits = [&](const u32x4 (&ka)[2][NC], f32x16 (&acc)[2][2]) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc[h][t] = f32x16{};
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[h][t] = mfma32(as_bf16x8(ka[t][c]), qh[h][c], acc[h][t]);
        }
    };
    // the block's mass for this lane's query of half h: 2^l summed over its 64 keys (two lanes)
    auto block_mass = [&](const f32x16 (&acc)[2]) {
      // seeded with the first exponentials rather than 0: 0 + x is not folded away (it would
      // turn -0 into +0), and these four adds per half are a tenth of the sweep's adds
      float s0 = fast_exp2(acc[0][0]), s1 = fast_exp2(acc[0][1]), s2 = fast_exp2(acc[1][0]),
            s3 = fast_exp2(acc[1][1]);
#pragma unroll
      for (int v = 2; v < 16; v += 2) {
        s0 += fast_exp2(acc[0][v]);
        s1 += fast_exp2(acc[0][v + 1]);
        s2 += fast_exp2(acc[1][v]);
        s3 += fast_exp2(acc[1][v + 1]);
      }
      return sum_xor32((s0 + s1) + (s2 + s3));
    };
    // lanes g = 0 store half 0's rows, lanes g = 1 half 1's: one 256-byte row of the slot per wave
    auto store = [&](int kb, float v) { slot[(size_t)kb * kScoreRows + wave * 64 + g * 32 + c32] = v; };

    // Fast sweep, software-pipelined and branch-free: two blocks per trip in alternating
    // accumulators (nkb is even), the next block's K_lr loads and MFMAs issued before the current
    // block's exponentials.  The prefetch index is clamped, so the last trip recomputes block
    // nkb - 1 into an accumulator nobody reads.
    u32x4 ka[2][NC];
    f32x16 A[2][2], B[2][2], cur[2][2];
    float tot0 = 0.f, tot1 = 0.f;
    auto finish = [&](int kb, const f32x16 (&acc)[2][2]) {
      const float b0 = block_mass(acc[0]), b1 = block_mass(acc[1]);
      store(kb, g ? b1 : b0);
      tot0 += b0;
      tot1 += b1;
    };
    // the pending item's finalisation: P steps for this wave, one in each of the first E1 trips
    // (spreading them thinner over the sweep, with an unrolled group of trips per step, measured
    // slower: the larger loop body costs more than the lighter bursts of reads save).
    // Step p covers chunk p / 16 and its rows 16 (p mod 16) .. +15 (four 16-byte loads per lane).
    const float* const pslot = slots + (size_t)(buf ^ 1) * slot_elems;
    const float* const prs = row_s[buf ^ 1];
    float* const psc = scores + (size_t)pbh * nqb * nkb;
    const int P = (!REP && pend) ? nchw * (kScoreRows / 16) : 0;
    const int E1 = min(nkb / 2, P);
    f32x4 fv[4];
    float fa = 0.f;
    auto issue = [&](int p) {
      const uint32_t voff = (uint32_t)min((wave + 4 * (p >> 4)) * 64 + lane, nkb - 1) * (kScoreRows * 4);
      const char* b = reinterpret_cast<const char*>(pslot + (p & 15) * 16);
#pragma unroll
      for (int u = 0; u < 4; ++u) fv[u] = *reinterpret_cast<const f32x4*>(b + voff + u * 16);
    };
    auto consume = [&](int p) {
      const int r0 = (p & 15) * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(prs + r0 + 4 * u);
        fa = fmaf(fv[u][3], w[3], fmaf(fv[u][2], w[2], fmaf(fv[u][1], w[1], fmaf(fv[u][0], w[0], fa))));
      }
      if (((p + 1) & (BQ / 16 - 1)) == 0) {  // the query block's last sixteen rows
        const int kbs = (wave + 4 * (p >> 4)) * 64 + lane;
        if (kbs < nkb) psc[(size_t)(pqb0 + r0 / BQ) * nkb + kbs] = fa;
        fa = 0.f;
      }
    };
    // one trip: blocks kb and kb + 1.  The finalisation loads are issued after the trip's last
    // K_lr loads, so the K_lr waits that follow leave them in flight; the first trip with loads is
    // peeled so that the loop is entered with the same loads outstanding as at its back edge.
    auto trip = [&](int kb, bool ev, bool cons) {
      logits(ka, B);  // block kb + 1
      load_k(min(kb + 2, nkb - 1), ka);
      finish(kb, A);
      logits(ka, A);  // block kb + 2
      load_k(min(kb + 3, nkb - 1), ka);
      if (ev) {
        if (cons) consume(kb / 2 - 1);
        issue(kb / 2);
      }
      finish(kb + 1, B);
    };
    load_k(0, ka);
    logits(ka, A);
    load_k(1, ka);
    int kb = 0;
    if (E1 > 0) {
      trip(0, true, false);
      for (kb = 2; kb < 2 * E1; kb += 2) trip(kb, true, true);
    }
    for (; kb < nkb; kb += 2) trip(kb, false, false);
    if (P > 0) {  // the last step, and any beyond the sweep's trips (nkb / 2 < P)
      consume(E1 - 1);
      for (int p = E1; p < P; ++p) {
        issue(p);
        consume(p);
      }
    }
    const bool exact = __syncthreads_or(!(tot0 < INFINITY) || !(tot0 >= kTinyMass) || !(tot1 < INFINITY) ||
                                        !(tot1 >= kTinyMass));
    if (!exact) {
      if (g == 0) {
        row_s[buf][wave * 64 + c32] = 1.f / tot0;
        row_s[buf][wave * 64 + 32 + c32] = 1.f / tot1;
      }
    } else {
      // exact path: block log-masses t = m + log2 sum_j 2^(l_ij - m) with m the block's own
      // maximum, and an online log-sum-exp over blocks for log2 T
      float run_m[2], run_s[2];
      for (int kb = 0; kb < nkb; ++kb) {
        load_k(kb, ka);
        logits(ka, cur);
        float t2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float m = cur[h][0][0];
#pragma unroll
          for (int v = 0; v < 16; ++v) m = fmaxf(m, fmaxf(cur[h][0][v], cur[h][1][v]));
          m = max_xor32(m);
          float sm = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) sm += fast_exp2(cur[h][0][v] - m) + fast_exp2(cur[h][1][v] - m);
          t2[h] = m + fast_log2(sum_xor32(sm));
          if (kb == 0) {
            run_m[h] = t2[h];
            run_s[h] = 1.f;
          } else {
            const float nm = fmaxf(run_m[h], t2[h]);
            run_s[h] = run_s[h] * fast_exp2(run_m[h] - nm) + fast_exp2(t2[h] - nm);
            run_m[h] = nm;
          }
        }
        store(kb, g ? t2[1] : t2[0]);
      }
      if (g == 0) {
        row_s[buf][wave * 64 + c32] = run_m[0] + fast_log2(run_s[0]);
        row_s[buf][wave * 64 + 32 + c32] = run_m[1] + fast_log2(run_s[1]);
      }
    }
    __threadfence_block();
    __syncthreads();

    if constexpr (REP) {
      // finalize: score[qb0 + i, kb] = mass[kb][i] / T_i (log domain on the exact path); each
      // wave writes its 64 rows, lane <-> kb
      float* sc_head = scores + (size_t)bh * nqb * nkb;
      for (int kb0 = 0; kb0 < nkb; kb0 += 64) {
        const int kb = kb0 + lane;
        if (kb >= nkb) continue;
        const float* src = slot + (size_t)kb * kScoreRows;
        for (int i = wave * 64; i < wave * 64 + 64; ++i) {
          if (row0 + i >= nqb) break;
          sc_head[(size_t)(row0 + i) * nkb + kb] =
              exact ? fast_exp2(src[i] - row_s[0][i]) : src[i] * row_s[0][i];
        }
      }
      __syncthreads();  // the slot and row_s are reused by the next item
      continue;
    }
    if (exact) {  // finalised at once (its masses are log-domain); nothing stays pending
      finalize_exact(slot, row_s[buf], scores + (size_t)bh * nqb * nkb, row0 / BQ);
      pend = false;
    } else {
      pend = true;
      pbh = bh;
      pqb0 = row0 / BQ;
      buf ^= 1;
    }
  }
  if (!REP && pend) {
    // The slot's last fast item: the same steps as the deferred finalisation, in the same order, so
    // that no score depends on which item of a slot came last (nor on the grid, the head count of
    // the call or the device's compute units).
    const float* const pslot = slots + (size_t)(buf ^ 1) * slot_elems;
    const float* const prs = row_s[buf ^ 1];
    float* const psc = scores + (size_t)pbh * nqb * nkb;
    const int P = nchw * (kScoreRows / 16);
    float fa = 0.f;
#pragma unroll 4
    for (int p = 0; p < P; ++p) {  // P is a multiple of 16: four steps' loads are issued together
      const int kbs = (wave + 4 * (p >> 4)) * 64 + lane, r0 = (p & 15) * 16;
      const float* src = pslot + (size_t)min(kbs, nkb - 1) * kScoreRows + r0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * u);
        const f32x4 w = *reinterpret_cast<const f32x4*>(prs + r0 + 4 * u);
        fa = fmaf(v[3], w[3], fmaf(v[2], w[2], fmaf(v[1], w[1], fmaf(v[0], w[0], fa))));
      }
      if (((p + 1) & (BQ / 16 - 1)) == 0) {  // the query block's last sixteen rows
        if (kbs < nkb) psc[(size_t)(pqb0 + r0 / BQ) * nkb + kbs] = fa;
        fa = 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------- fused representative predict + top-k (bf16)
//
// The pages' fused matmul and top-k kernel with query grouping by one representative row per
// group ([de] §2.B): the critical KV blocks of a query block are chosen from the logits of its
// row qb * Bq + rep, and no score matrix is written.  For one row, ranking KV blocks by predicted
// softmax mass equals ranking them by the in-block log-sum-exp of the row's logits (the row's
// normaliser is common to all its blocks), so selection needs no other statistic.
//
// One workgroup per (head, 64 consecutive query blocks).  Its waves take the chunks of 32 KV blocks
// round-robin (wave w: chunks w, w + 4, ...) and sweep them for all 64 representative rows: one
// bf16 32x32x16 MFMA product of Q~ and K_lr gives log2-unit logits, and each (row, block) key is
// the block's mass sum_j 2^l_j (one exp and one add per logit).  An item holding a row whose
// largest block mass leaves [2^-100, fp32 max] is swept again with keys m + log2 sum_j 2^(l_j - m),
// m the block's maximum, exact at any logit range.
// A chunk's keys are transposed through LDS so that each row's 32 keys leave as one 128-byte line
// into the workgroup's row-major scratch (64 x nkb floats); after one barrier each wave picks the
// top k of 16 rows with topk_row and writes their ascending index lists.
template <int R, int NPL>
__global__ __launch_bounds__(256) void rep_select_bf16_kernel(const uint16_t* __restrict__ qlr,
                                                              const uint16_t* __restrict__ klr,
                                                              float* __restrict__ scratch,
                                                              int32_t* __restrict__ idx, int n, int nkb, int bq,
                                                              int rep, int k, int items) {
  constexpr int NC = R / 16;
  constexpr int CH = 32;           // KV blocks per chunk
  constexpr int TP = 65;           // padded row pitch of the transpose tile (conflict-free writes)
  constexpr float kTinyMass = 7.888609052210118e-31f;  // 2^-100
  __shared__ float tile_s[4][CH * TP];
  __shared__ float rmax_s[4][64];  // per wave: the largest fast-sweep block mass of each row
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const int nqb = n / bq;
  const int groups = (nqb + 63) / 64;  // work items per head
  float* const keys = scratch + (size_t)blockIdx.x * 64 * nkb;
  float* const tile = tile_s[wave];
  const int nchunks = (nkb + CH - 1) / CH;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int bh = item / groups;
    const int qb0 = (item % groups) * 64;
    const uint16_t* kh = klr + (size_t)bh * n * R;
    // B operands = Q~^T of the two 32-row halves: lane holds the representative row of query block
    // qb0 + h*32 + c32 (clamped past the last query block: computed, never selected)
    bf16x8 qh[2][NC];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int qb = min(qb0 + h * 32 + c32, nqb - 1);
      const uint16_t* qrow = qlr + ((size_t)bh * n + (size_t)qb * bq + rep) * R;
#pragma unroll
      for (int c = 0; c < NC; ++c) qh[h][c] = as_bf16x8(ld16(qrow + c * 16 + g * 8));
    }
    // A operands (K_lr rows, 8 consecutive r) of one KV block: 2 tiles x NC chunks
    auto load_k = [&](int kb, u32x4 (&ka)[2][NC]) {
      const uint16_t* kp = kh + (size_t)kb * 64 * R;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) ka[t][c] = ld16(kp + (size_t)(t * 32 + c32) * R + c * 16 + g * 8);
    };
    // One sweep over the item's KV blocks.  Fast (exact = false): the key of (row, block) is the
    // block's mass sum_j 2^l_j, one exp and one add per logit, as in the score sweep; returned is
    // the largest mass of this lane's row (row = lane) over the wave's chunks.  Exact: the key is
    // the in-block log-sum-exp m + log2 sum_j 2^(l_j - m), m the block's maximum, valid at any
    // logit range.  Either key orders a row's blocks as their predicted softmax mass does.
    auto sweep = [&](bool exact) {
      float rmax = 0.f;
      for (int ch = wave; ch < nchunks; ch += 4) {
        const int cb0 = ch * CH, cnt = min(CH, nkb - cb0);  // cnt is a multiple of 4 (nkb is)
        u32x4 ka[2][NC];
        f32x16 acc[2][2];
        load_k(cb0, ka);
        for (int j = 0; j < cnt; ++j) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              acc[h][t] = f32x16{};
#pragma unroll
              for (int c = 0; c < NC; ++c) acc[h][t] = mfma32(as_bf16x8(ka[t][c]), qh[h][c], acc[h][t]);
            }
          if (j + 1 < cnt) load_k(cb0 + j + 1, ka);
          // lane holds 32 of the block's 64 logits for its row of half h; lane ^ 32 the other 32
          float key2[2];
          if (!exact) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float sp[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) sp[e] = fast_exp2(acc[h][e >> 1][e & 1]);
#pragma unroll
              for (int v = 2; v < 16; v += 2)
#pragma unroll
                for (int e = 0; e < 4; ++e) sp[e] += fast_exp2(acc[h][e >> 1][v + (e & 1)]);
              key2[h] = sum_xor32((sp[0] + sp[1]) + (sp[2] + sp[3]));
            }
          } else {
            // a tree maximum and four partial sums: short dependency chains, since few waves share
            // a SIMD
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float mx[16];
#pragma unroll
              for (int v = 0; v < 16; ++v) mx[v] = fmaxf(acc[h][0][v], acc[h][1][v]);
#pragma unroll
              for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                for (int v = 0; v < w; ++v) mx[v] = fmaxf(mx[v], mx[v + w]);
              const float m = max_xor32(mx[0]);
              float sp[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) sp[e] = fast_exp2(acc[h][e >> 1][e & 1] - m);
#pragma unroll
              for (int v = 2; v < 16; v += 2)
#pragma unroll
                for (int e = 0; e < 4; ++e) sp[e] += fast_exp2(acc[h][e >> 1][v + (e & 1)] - m);
              key2[h] = m + fast_log2(sum_xor32((sp[0] + sp[1]) + (sp[2] + sp[3])));
            }
          }
          // lanes g = 0 hold half 0's rows, lanes g = 1 half 1's: tile[block][row], row = lane
          const float mine = g ? key2[1] : key2[0];
          rmax = fmaxf(rmax, mine);
          tile[j * TP + g * 32 + c32] = mine;
        }
        // the chunk's keys, row by row: lane L writes 4 keys (one 16-byte segment) of row
        // (u * 64 + L) / 8, so that eight lanes fill one row's 128-byte line
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int f = u * 64 + lane, row = f >> 3, seg = (f & 7) * 4;
          if (seg < cnt) {
            const f32x4 v4 = {tile[(seg + 0) * TP + row], tile[(seg + 1) * TP + row], tile[(seg + 2) * TP + row],
                              tile[(seg + 3) * TP + row]};
            *reinterpret_cast<f32x4*>(keys + (size_t)row * nkb + cb0 + seg) = v4;
          }
        }
      }
      return rmax;
    };
    // The fast keys hold (up to rounding) for rows whose largest block mass is finite and at least
    // 2^-100 (the top blocks then keep full precision); an item with any other valid row is swept
    // again in the log domain.
    rmax_s[wave][lane] = sweep(false);
    __syncthreads();
    bool off_range = false;
    if (threadIdx.x < 64 && qb0 + (int)threadIdx.x < nqb) {
      const float m = fmaxf(fmaxf(rmax_s[0][threadIdx.x], rmax_s[1][threadIdx.x]),
                            fmaxf(rmax_s[2][threadIdx.x], rmax_s[3][threadIdx.x]));
      off_range = !(m >= kTinyMass && m < INFINITY);
    }
    if (__syncthreads_or(off_range)) sweep(true);
    __threadfence_block();
    __syncthreads();
    // selection: wave w takes the item's rows [16w, 16w + 16)
    for (int i = wave * 16; i < wave * 16 + 16; ++i) {
      const int qb = qb0 + i;
      if (qb >= nqb) break;
      const float* row = keys + (size_t)i * nkb;
      uint32_t key[NPL];
#pragma unroll
      for (int e = 0; e < NPL; ++e) {
        const int kb = e * 64 + lane;
        key[e] = kb < nkb ? max(order_key(row[kb]), 1u) : 0u;  // padding = 0, valid keys >= 1
      }
      topk_row<NPL>(key, k, idx + ((size_t)bh * nqb + qb) * k, lane);
    }
    __syncthreads();  // the next item's sweep refills the scratch
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

// representative rows (f32): the log-sum-exp of row qb * bq + rep over all keys, then that
// row's mass on each KV block
__global__ void rep_lse_f32_kernel(const float* __restrict__ qlr, const float* __restrict__ klr,
                                   float* __restrict__ lse, int n, int r, int bq, int rep, float ps, int rows) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;  // bh * nqb + qb
  if (t >= rows) return;
  const int nqb = n / bq, bh = t / nqb, qb = t % nqb;
  const float* q = qlr + ((size_t)bh * n + (size_t)qb * bq + rep) * r;
  const float* kh = klr + (size_t)bh * n * r;
  float m = -INFINITY;
  for (int j = 0; j < n; ++j) {
    float a = 0.f;
    for (int c = 0; c < r; ++c) a = fmaf(q[c], kh[(size_t)j * r + c], a);
    m = fmaxf(m, a * ps);
  }
  float sum = 0.f;
  for (int j = 0; j < n; ++j) {
    float a = 0.f;
    for (int c = 0; c < r; ++c) a = fmaf(q[c], kh[(size_t)j * r + c], a);
    sum += expf(a * ps - m);
  }
  lse[t] = m + logf(sum);
}

__global__ void rep_scores_f32_kernel(const float* __restrict__ qlr, const float* __restrict__ klr,
                                      const float* __restrict__ lse, float* __restrict__ scores, int n, int r,
                                      int bq, int bk, int rep, float ps, int total) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;  // (bh * nqb + qb) * nkb + kb
  if (t >= total) return;
  const int nkb = n / bk, nqb = n / bq;
  const int kb = t % nkb, row = t / nkb, bh = row / nqb, qb = row % nqb;
  const float* q = qlr + ((size_t)bh * n + (size_t)qb * bq + rep) * r;
  const float* kh = klr + (size_t)bh * n * r;
  float acc = 0.f;
  for (int j = kb * bk; j < (kb + 1) * bk; ++j) {
    float a = 0.f;
    for (int c = 0; c < r; ++c) a = fmaf(q[c], kh[(size_t)j * r + c], a);
    acc += expf(a * ps - lse[row]);
  }
  scores[t] = acc;
}

hipError_t launch_rep_scores_f32(const float* qlr, const float* klr, float* lse, float* scores, int bh, int n,
                                 int r, int bq, int bk, float pred_scale, int rep, hipStream_t st) {
  const int rows = bh * (n / bq);
  hipLaunchKernelGGL(rep_lse_f32_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, qlr, klr, lse, n, r, bq, rep,
                     pred_scale, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int total = rows * (n / bk);
  hipLaunchKernelGGL(rep_scores_f32_kernel, dim3((total + 255) / 256), dim3(256), 0, st, qlr, klr, lse, scores, n, r,
                     bq, bk, rep, pred_scale, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers

hipError_t launch_proj_bf16(const uint16_t* x, const uint16_t* w, uint16_t* out, int bh, int n, int heads,
                            int d, int r, float scale, hipStream_t st) {
  dim3 grid((n + 255) / 256, bh);
#define PROJ(D_, R_)                                                                                  \
  if (d == D_ && r == R_) {                                                                           \
    hipLaunchKernelGGL((proj_bf16_kernel<D_, R_>), grid, dim3(256), 0, st, x, w, out, n, heads, scale); \
    return hipGetLastError();                                                                         \
  }
  PROJ(64, 16) PROJ(64, 32) PROJ(128, 16) PROJ(128, 32)
#undef PROJ
  return hipErrorInvalidValue;
}

hipError_t launch_proj_f32(const float* x, const float* w, float* out, int bh, int n, int heads, int d,
                           int r, float scale, hipStream_t st) {
  dim3 grid((unsigned)(((size_t)n * r + 255) / 256), bh);
  hipLaunchKernelGGL(proj_f32_kernel, grid, dim3(256), 0, st, x, w, out, n, d, r, heads, scale);
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

size_t score_scratch_bytes(int items, int nkb) {  // two halves per slot (deferred finalisation)
  return (size_t)score_slots(items) * 2 * nkb * kScoreRows * sizeof(float);
}

int score_items(int bh, int n, int bq, bool representative) {
  return representative ? bh * ((n / bq + kScoreRows - 1) / kScoreRows) : bh * (n / kScoreRows);
}

hipError_t launch_scores_bf16(const uint16_t* qlr, const uint16_t* klr, float* scratch, float* scores,
                              int bh, int n, int nkb, int r, int bq, int rep, hipStream_t st) {
  const bool representative = rep >= 0;
  const int items = score_items(bh, n, bq, representative);
  const int slots = score_slots(items);
#define SC(R_, BQ_)                                                                                           \
  if (r == R_ && bq == BQ_) {                                                                                 \
    if (representative)                                                                                       \
      hipLaunchKernelGGL((scores_bf16_kernel<R_, BQ_, true>), dim3(slots), dim3(256), 0, st, qlr, klr, scratch, \
                         scores, n, nkb, items, rep);                                                         \
    else                                                                                                      \
      hipLaunchKernelGGL((scores_bf16_kernel<R_, BQ_, false>), dim3(slots), dim3(256), 0, st, qlr, klr,         \
                         scratch, scores, n, nkb, items, 0);                                                  \
    return hipGetLastError();                                                                                 \
  }
  SC(16, 64) SC(16, 128) SC(32, 64) SC(32, 128)
#undef SC
  return hipErrorInvalidValue;
}

int rep_select_items(int bh, int n, int bq) { return bh * ((n / bq + 63) / 64); }

// Grid of the fused kernel: its per-workgroup scratch (64 x nkb floats) is 1/8 of a score slot's
// (two halves of 256 x nkb), so eight of its workgroups fit in each slot of dsv_predict's workspace.
int rep_select_slots(int bh, int n, int bq) {
  const int items = rep_select_items(bh, n, bq);
  const int cap = 8 * score_slots(score_items(bh, n, bq, false));
  return items < cap ? items : cap;
}

hipError_t launch_rep_select_bf16(const uint16_t* qlr, const uint16_t* klr, float* scratch, int32_t* idx, int bh,
                                  int n, int nkb, int r, int bq, int rep, int k, hipStream_t st) {
  const int items = rep_select_items(bh, n, bq);
  const int grid = rep_select_slots(bh, n, bq);
  const int npl = (nkb + 63) / 64;
#define RS(R_, N_)                                                                                             \
  if (r == R_ && npl <= N_) {                                                                                  \
    hipLaunchKernelGGL((rep_select_bf16_kernel<R_, N_>), dim3(grid), dim3(256), 0, st, qlr, klr, scratch, idx, n, \
                       nkb, bq, rep, k, items);                                                                \
    return hipGetLastError();                                                                                  \
  }
  RS(16, 1) RS(16, 2) RS(16, 4) RS(16, 8) RS(16, 16) RS(16, 32) RS(16, 64)
  RS(32, 1) RS(32, 2) RS(32, 4) RS(32, 8) RS(32, 16) RS(32, 32) RS(32, 64)
#undef RS
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
