// Block-sparse attention forward.
//
// Method: the DSV pages ("DSV: Exploiting Dynamic Sparsity to Accelerate
// Large-Scale Video DiT Training", gist.science/es technical summary §3 and
// gist.science/de §2.A stage 2) run exact attention over the selected critical
// KV only.  For query block qb with selected blocks J:
//   O_i = softmax_J(sm_scale q_i K_J^T) V_J,  lse_i = log sum_{j in J} exp(sm_scale q_i.k_j).
//
// gfx950 design (bf16, d in {64,128}, Bq in {64,128}, Bk = 64):
//  * one workgroup per (b, h, qb), Bq/32 waves, each wave owns 32 query rows;
//    registers are capped so that two waves share each SIMD (one's softmax
//    VALU work overlaps the other's MFMAs);
//    workgroups run in plain dispatch order, so that the eight XCDs work on one head
//    at a time (its gathered K/V tiles then stay within the Infinity Cache);
//  * Q stays in registers as the B operand of S^T = K Q^T (v_mfma 32x32x16);
//  * each selected KV block is gathered into swizzled LDS tiles (K and V both
//    row-major, as stored) by direct global->LDS loads, double-buffered: the
//    next block's copies are in flight while the current block is computed,
//    without staging registers; the V^T operand of
//    O^T += V^T P^T comes from transposing LDS reads (ds_read_b64_tr_b16);
//  * S^T's D layout puts one query per lane, so the online-softmax row max and
//    row sum are lane-local plus one exchange with lane ^ 32; K rows are loaded
//    in the sigma order so that P^T feeds O^T += V^T P^T directly from registers;
//  * the training forward (when the caller asks for O's rounding residual) takes
//    P V in fp16: V is first copied to fp16 with a power-of-two per-head scale
//    (exact for bf16 values), P is rounded to fp16 (2^-11 relative instead of
//    bf16's 2^-8) -- one product, O accurate enough for the backward's D.
#include "common.hpp"
#include "kernels.hpp"

namespace dsv {

// PV16: the training forward.  v is then the fp16 copy of V scaled by 2^f16_shift(vmax[bh]);
// P enters O += P V rounded to fp16, and the kernel also writes O's rounding residual o_lo.
template <int D, int BQ, bool PV16>
__global__ __launch_bounds__(BQ * 2, (kMinWavesPerSimd<D, BQ>)) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnts, uint16_t* __restrict__ o,
    float* __restrict__ lse, uint16_t* __restrict__ o_lo /* rounding residual of O (PV16) */,
    const uint32_t* __restrict__ vmax /* PV16: per-head max |V| (float bits) */, int n, int topk,
    float c /* sm_scale * log2(e) */) {
  constexpr int WAVES = BQ / 32;
  constexpr int NI = 2 * 64 * D / 512;  // global->LDS instructions per KV block (K and V tiles)
  // separate arrays per buffer: with one array the compiler cannot tell that the
  // asynchronous copy into one buffer never aliases reads of the other, and would
  // wait for the copy before every transposing read
  __shared__ __attribute__((aligned(16))) uint16_t K0[64 * D], K1[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[64 * D], V1[64 * D];

  const int nqb = n / BQ;
  const int id = blockIdx.x;  // measured faster here than the per-XCD remap of dK/dV
  const int bh = id / nqb, qb = id % nqb;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const size_t head = (size_t)bh * n * D;
  const int32_t* blocks = idx + ((size_t)bh * nqb + qb) * topk;
  const int kq = list_len(cnts, (size_t)bh * nqb + qb, topk);  // blocks in this query block's list
  const int nkb = n / 64;
  // out-of-range block indices are clamped: wrong results, but no access outside the tensors
  auto blk_at = [&](int j) { return min(max(blocks[j], 0), nkb - 1); };
  // gather the K (or V) tile of KV block `blk` into an LDS buffer (asynchronous; visible after
  // the next barrier)
  static_assert((NI / 2) % WAVES == 0, "each wave issues the same number of copies");
  auto issue = [&](const uint16_t* src, int blk, uint16_t* dst) {
    const int ln = opaque(lane);  // the copies' lane offset is computed here, once per batch
#pragma unroll
    for (int m = 0; m < NI / 2 / WAVES; ++m)
      lds_load_rows<D>(src + head + (size_t)blk * 64 * D, dst, wave + m * WAVES, ln);
  };

  // Q^T as the B operand of S^T = K Q^T: lane holds its query row, 8 consecutive d per 16-wide chunk
  const int qrow = qb * BQ + wave * 32 + c32;
  if (kq == 0) {  // an empty block list: O = 0, lse = -inf (uniform over the workgroup)
    uint16_t* orow = o + head + (size_t)qrow * D;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) st16(orow + dc * 16 + g * 8, u32x4{0, 0, 0, 0});
    if constexpr (PV16) {
      uint16_t* lrow = o_lo + head + (size_t)qrow * D;
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) st16(lrow + dc * 16 + g * 8, u32x4{0, 0, 0, 0});
    }
    if (g == 0) lse[(size_t)bh * n + qrow] = -INFINITY;
    return;
  }
  bf16x8 qf[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) qf[dc] = as_bf16x8(ld16(q + head + (size_t)qrow * D + dc * 16 + g * 8));


  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int arow = sigma(c32);
  // loop-invariant fragment offsets (row_offsets / tr_offsets): the 32-key tile t adds t*64*D
  // bytes to a K read, the 16-key chunk cc adds cc*32*D to a transposed V read
  int rbs[D / 16], vb0s[D / 32], vb1s[D / 32];
  row_offsets<D>(rbs, arow, lane);
  tr_offsets<D>(vb0s, vb1s, 0, lane);

  // S^T = K Q^T for one KV block (two 32-key tiles, K rows in sigma order: byte base + t*64*D), each
  // k-step's K operand read one step ahead; fragment offsets from one base, recomputed per block
  auto scores = [&](const uint16_t* Kc, f32x16 (&s)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x16{};
      bf16x8 ka = row_frag_off(Kc, rbs[0], t * 64 * D);
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        bf16x8 kn = ka;
        if (dc + 1 < D / 16) kn = row_frag_off(Kc, rbs[dc + 1], t * 64 * D);
        s[t] = mfma32(ka, qf[dc], s[t]);
        ka = kn;
      }
    }
  };
  // Row maximum of a block's raw scores: a tree over the lane's 32 values, then lane ^ 32.
  auto raw_max = [&](const f32x16 (&s)[2]) {
    float mx8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      mx8[e] = fmaxf(fmaxf(s[0][e], s[0][e + 8]), fmaxf(s[1][e], s[1][e + 8]));
#pragma unroll
    for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
      for (int e = 0; e < w; ++e) mx8[e] = fmaxf(mx8[e], mx8[e + w]);
    return max_xor32(mx8[0]);
  };
  // online softmax of one block's scores, part 1: the exponents t = s c - m_run (in place), their
  // row maximum and the (rare) rescaling.
  // Lazy rescaling: the running shift m_run only moves when an exponent exceeds 8 (log2 units),
  // so exponentials stay below 2^8 and the accumulator and row sum are rescaled rarely.  Any
  // shift gives the same O = acc / l; the choice only moves rounding.  Taking the maximum over
  // the exponents rather than the raw MFMA results saves work: they are needed anyway, and as
  // fma results they take three-input maxima with no canonicalisation.
  auto rescale = [&](f32x16 (&s)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) s[t][vv] = fmaf(s[t][vv], c, -m_run);
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
    for (int e = 3; e < 31; e += 2) {
      const float a = e < 16 ? s[0][e] : s[1][e - 16], b = e + 1 < 16 ? s[0][e + 1] : s[1][e + 1 - 16];
      mx = fmaxf(fmaxf(mx, a), b);
    }
    mx = fmaxf(mx, s[1][15]);
    mx = max_xor32(mx);
    if (__builtin_amdgcn_ballot_w64(mx > 8.f) != 0) {
      const float shift = fmaxf(mx, 0.f);
      const float alpha = fast_exp2(-shift);
      m_run += shift;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) s[t][vv] -= shift;
    }
  };
  // part 2: exponentials, row sum and O^T += V^T P^T from Vc
  auto exp_pv = [&](f32x16 (&s)[2], const uint16_t* Vc) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) s[t][vv] = fast_exp2(s[t][vv]);
    float psum = s[0][0];  // seeded with the first term: 0 + x would cost an add
#pragma unroll
    for (int e = 1; e < 32; ++e) psum += e < 16 ? s[0][e] : s[1][e - 16];
    l_run += psum;
    // O^T += V^T P^T: V^T operands by transposed reads of the row-major V tile (rows cc*16..:
    // byte bases + cc*32*D); P^T chunk cc = registers (cc%2)*8.. of tile cc/2.  P <= 2^8 (lazy
    // rescaling), so fp16 holds it; a bf16 rounding of P (2^-8 relative) would be fine for O
    // itself but too coarse for the backward's D = rowsum(dO * O), which the dQ product
    // multiplies by K -- the training forward therefore rounds P to fp16 against fp16 V.
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const f32x16& st = s[cc >> 1];
      const int b0 = (cc & 1) * 8;
      bf16x8 va = tr_frag_off(Vc, vb0s[0], vb1s[0], cc * 32 * D);
      if constexpr (PV16) {
        const f16x8 ph = cvt8h(st[b0], st[b0 + 1], st[b0 + 2], st[b0 + 3], st[b0 + 4], st[b0 + 5], st[b0 + 6],
                               st[b0 + 7]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          bf16x8 vn = va;
          if (dt + 1 < D / 32) vn = tr_frag_off(Vc, vb0s[dt + 1], vb1s[dt + 1], cc * 32 * D);
          oacc[dt] = mfma32h(as_f16x8(va), ph, oacc[dt]);
          va = vn;
        }
      } else {
        const bf16x8 ph = cvt8(st[b0], st[b0 + 1], st[b0 + 2], st[b0 + 3], st[b0 + 4], st[b0 + 5], st[b0 + 6],
                               st[b0 + 7]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          bf16x8 vn = va;
          if (dt + 1 < D / 32) vn = tr_frag_off(Vc, vb0s[dt + 1], vb1s[dt + 1], cc * 32 * D);
          oacc[dt] = mfma32(va, ph, oacc[dt]);
          va = vn;
        }
      }
    }
  };

  // Pipelined over blocks: the scores of block j+1 are issued between the row maximum and the
  // exponentials of block j, in one straight-line region with block j's PV product, so the matrix
  // pipe works while the vector ALU runs the softmax.  K runs one block ahead of V: in step j
  // (after the barrier that ends step j-1) K_{j+2} goes into the buffer of K_j, whose scores were
  // computed in step j-1, and V_{j+1} into the buffer of V_{j-1}.  Prefetch indices are clamped
  // (a redundant copy lands in a free buffer) and the scores computed past the last block are
  // never used.  Two steps per trip so that each buffer is a distinct array.
  f32x16 sa[2], sb[2];
  const int last = kq - 1;
  issue(k, blk_at(0), K0);
  issue(k, blk_at(min(1, last)), K1);
  issue(v, blk_at(0), V0);
  __syncthreads();
  scores(K0, sa);
  m_run = raw_max(sa) * c;  // the first block sets the shift
  __syncthreads();  // every wave has read K0 before step 0 refills it
  int j = 0;
  for (; j + 1 < kq; j += 2) {
    // step j: sa = S_j, K1 = K_{j+1}, V0 = V_j
    issue(k, blk_at(min(j + 2, last)), K0);
    issue(v, blk_at(j + 1), V1);
    rescale(sa);
    scores(K1, sb);
    exp_pv(sa, V0);
    __syncthreads();
    // step j+1: sb = S_{j+1}, K0 = K_{j+2}, V1 = V_{j+1}
    issue(k, blk_at(min(j + 3, last)), K1);
    issue(v, blk_at(min(j + 2, last)), V0);
    rescale(sb);
    scores(K0, sa);
    exp_pv(sb, V1);
    __syncthreads();
  }
  if (j < kq) {  // odd length: the last block (sa = S_last, V0 = V_last)
    rescale(sa);
    exp_pv(sa, V0);
  }

  const float l = l_run + xor32(l_run);
  const float inv = 1.f / l;
  const int unscale = PV16 ? -f16_shift(vmax[bh]) : 0;  // O was accumulated against the scaled V
  uint16_t* orow = o + head + (size_t)qrow * D;
  uint16_t* lrow = PV16 ? o_lo + head + (size_t)qrow * D : nullptr;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      const int d0 = dt * 32 + vq * 8 + g * 4;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = PV16 ? ldexpf(oacc[dt][vq * 4 + e] * inv, unscale) : oacc[dt][vq * 4 + e] * inv;
      const u32x2 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      *reinterpret_cast<u32x2*>(orow + d0) = pk;
      if constexpr (PV16) {  // residual x - bf16(x), itself rounded to bf16
        const u32x2 rk = {pack_bf16x2(x[0] - __uint_as_float(pk[0] << 16), x[1] - __uint_as_float(pk[0] & 0xffff0000u)),
                          pack_bf16x2(x[2] - __uint_as_float(pk[1] << 16), x[3] - __uint_as_float(pk[1] & 0xffff0000u))};
        *reinterpret_cast<u32x2*>(lrow + d0) = rk;
      }
    }
  if (g == 0) lse[(size_t)bh * n + qrow] = (m_run + fast_log2(l)) * kLn2;
}

// ---------------------------------------------------------------- f32 path (plain VALU)

template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ cnts, float* __restrict__ o,
                                                          float* __restrict__ lse, int n, int d, int bq, int bk,
                                                          int topk, float scale) {
  // one thread per query row; grid (ceil(n/64), BH)
  const int bh = blockIdx.y;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= n) return;
  const size_t head = (size_t)bh * n * d;
  const float* qi = q + head + (size_t)i * d;
  float qv[D], acc[D];
  for (int c = 0; c < d; ++c) { qv[c] = qi[c]; acc[c] = 0.f; }
  const size_t qrow = (size_t)bh * (n / bq) + i / bq;
  const int32_t* blocks = idx + qrow * topk;
  const int kq = list_len(cnts, qrow, topk);
  float m = -INFINITY, l = 0.f;
  for (int jb = 0; jb < kq; ++jb) {
    const int kb = min(max(blocks[jb], 0), n / bk - 1);  // clamp out-of-range indices
    for (int j = kb * bk; j < (kb + 1) * bk; ++j) {
      const float* kj = k + head + (size_t)j * d;
      float s = 0.f;
      for (int c = 0; c < d; ++c) s = fmaf(qv[c], kj[c], s);
      s *= scale;
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn), p = expf(s - mn);
      l = l * a + p;
      const float* vj = v + head + (size_t)j * d;
      for (int c = 0; c < d; ++c) acc[c] = fmaf(p, vj[c], acc[c] * a);
      m = mn;
    }
  }
  float* oi = o + head + (size_t)i * d;
  const float inv = l > 0.f ? 1.f / l : 0.f;  // an empty block list gives O = 0, lse = -inf
  for (int c = 0; c < d; ++c) oi[c] = acc[c] * inv;
  lse[(size_t)bh * n + i] = l > 0.f ? m + logf(l) : -INFINITY;
}

// ---------------------------------------------------------------- launchers

size_t attn_fwd_bf16_ws_bytes(int bh, int n, int d) {
  return align_ws((size_t)bh * n * d * 2) + head_absmax_ws_bytes(bh) + align_ws((size_t)bh * 4);
}

hipError_t launch_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                                const int32_t* cnts, uint16_t* o, float* lse, uint16_t* o_lo, void* ws, int bh, int n,
                                int d, int bq, int topk, float sm_scale, hipStream_t st) {
  const int nwg = bh * (n / bq);
  const float c = sm_scale * kLog2e;
  uint16_t* v16 = nullptr;
  uint32_t* vmax = nullptr;
  if (o_lo) {  // training forward: V to fp16 first
    const size_t per_head = (size_t)n * d;
    char* w = static_cast<char*>(ws);
    v16 = reinterpret_cast<uint16_t*>(w);
    uint32_t* part = reinterpret_cast<uint32_t*>(w + align_ws((size_t)bh * per_head * 2));
    vmax = reinterpret_cast<uint32_t*>(w + align_ws((size_t)bh * per_head * 2) + head_absmax_ws_bytes(bh));
    hipError_t e = launch_head_absmax(v, part, vmax, bh, per_head, st);
    if (e != hipSuccess) return e;
    if ((e = launch_to_f16(v, vmax, v16, bh, per_head, st)) != hipSuccess) return e;
  }
#define FWD(D_, BQ_)                                                                                      \
  if (d == D_ && bq == BQ_) {                                                                             \
    if (o_lo)                                                                                             \
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<D_, BQ_, true>), dim3(nwg), dim3(BQ_ * 2), 0, st, q, k, v16, idx, \
                         cnts, o, lse, o_lo, vmax, n, topk, c);                                           \
    else                                                                                                  \
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<D_, BQ_, false>), dim3(nwg), dim3(BQ_ * 2), 0, st, q, k, v, \
                         idx, cnts, o, lse, o_lo, vmax, n, topk, c);                                      \
    return hipGetLastError();                                                                             \
  }
  FWD(64, 64) FWD(64, 128) FWD(128, 64) FWD(128, 128)
#undef FWD
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, const int32_t* idx,
                               const int32_t* cnts, float* o, float* lse, int bh, int n, int d, int bq, int bk, int topk,
                               float sm_scale, hipStream_t st) {
  dim3 grid((n + 63) / 64, bh);
#define FF(D_)                                                                                            \
  if (d <= D_) {                                                                                          \
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D_>), grid, dim3(64), 0, st, q, k, v, idx, cnts, o, lse, n, d, bq, \
                       bk, topk, sm_scale);                                                               \
    return hipGetLastError();                                                                             \
  }
  FF(32) FF(64) FF(128)
#undef FF
  return hipErrorInvalidValue;
}

}  // namespace dsv
