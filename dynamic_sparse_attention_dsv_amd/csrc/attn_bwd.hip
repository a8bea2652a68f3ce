// Block-sparse attention backward, plus its small helper kernels (the
// D = rowsum(dO o O) preprocess, and the transpose of the block lists from
// "query block -> KV blocks" to "KV block -> query blocks").
//
// Method: the DSV pages ("DSV: Exploiting Dynamic Sparsity to Accelerate
// Large-Scale Video DiT Training", gist.science/de technical summary §2.A,
// stage 2, and gist.science/es §2.A, fase 2) train the video DiT with the
// sparse attention, so its gradients are needed.  For every selected (qb, kb)
// pair, with P = exp(S - lse) the forward's probabilities:
//   dV_kb += P^T dO_qb,  dP = dO_qb V_kb^T,  dS = P o (dP - D),  D = rowsum(dO o O),
//   dK_kb += sm_scale dS^T Q_qb,  dQ_qb += sm_scale dS K_kb.
//
// gfx950 design (bf16 inputs and outputs):
//  * dK/dV: one workgroup per KV block walks the list of query blocks that
//    selected it (the transposed lists), 32 query rows at a time, with dK and dV
//    accumulated in registers -- no atomics, deterministic;
//  * dQ: one workgroup per query block walks its own k blocks (recomputing P and
//    dP), accumulating dQ in registers -- again no atomics;
//  * every GEMM is a v_mfma 32x32x16 (fp16 on power-of-two-scaled copies where
//    the rounding of an operand reaches a gradient, else bf16); operands that
//    contract along a row of a gathered tile are plain LDS reads, operands that
//    contract down its columns come from transposing LDS reads
//    (ds_read_b64_tr_b16) of the same row-major tile, so no transposed copy of
//    any tensor is made.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace dsv {

// The dK/dV kernel's per-head dS exponent r: |dS_ij| <= |dP_ij - D_i| <= 2 d max|dO| max|V|, so
// dS 2^r stays inside fp16's range at full precision.  absmax: per-head max |.| bits of K, Q, V,
// dO (bh_total each).
template <int D>
__device__ __forceinline__ int dkdv_ds_exponent(const uint32_t* absmax, int bh, int bh_total) {
  const float vmax = __uint_as_float(absmax[2 * bh_total + bh]);
  const float omax = __uint_as_float(absmax[3 * bh_total + bh]);
  return min(max(f16_exponent(__float_as_uint(2.f * (float)D * omax * vmax)), -120), 120);
}

// ---------------------------------------------------------------- D = rowsum(dO o O), lse2 = lse * log2(e)
//
// Also D 2^r with the dK/dV kernel's per-head dS exponent r (dvec_s), so that kernel forms
// dS 2^r = P (dP 2^r - D 2^r) with no extra multiply.

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_bf16_kernel(const uint16_t* __restrict__ o,
                                                           const uint16_t* __restrict__ o_lo,
                                                           const uint16_t* __restrict__ dout,
                                                           const float* __restrict__ lse, float* __restrict__ dvec,
                                                           float* __restrict__ lse2, float* __restrict__ dvec_s,
                                                           const uint32_t* __restrict__ absmax, int n, int bh_total,
                                                           int rows) {
  constexpr int LPR = D / 8;  // lanes per row, 16 bytes each
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int row = t / LPR, c = t % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = ld16(o + (size_t)row * D + c * 8), b = ld16(dout + (size_t)row * D + c * 8);
    const u32x4 r = o_lo ? ld16(o_lo + (size_t)row * D + c * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // O = o + o_lo (the residual is 0 without it)
      const float olo = __uint_as_float(a[e] << 16) + __uint_as_float(r[e] << 16);
      const float ohi = __uint_as_float(a[e] & 0xffff0000u) + __uint_as_float(r[e] & 0xffff0000u);
      acc = fmaf(olo, __uint_as_float(b[e] << 16), acc);
      acc = fmaf(ohi, __uint_as_float(b[e] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) {
    dvec[row] = acc;
    lse2[row] = lse[row] * kLog2e;
    dvec_s[row] = ldexpf(acc, dkdv_ds_exponent<D>(absmax, row / n, bh_total));
  }
}

__global__ void bwd_pre_f32_kernel(const float* __restrict__ o, const float* __restrict__ dout,
                                   float* __restrict__ dvec, int rows, int d) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = fmaf(o[(size_t)row * d + c], dout[(size_t)row * d + c], acc);
  dvec[row] = acc;
}

// ---------------------------------------------------------------- block lists: CSR (per query block) -> CSC

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void csc_mark_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnts,
                                uint32_t* __restrict__ bitmap, int nqb, int nkb, int topk, int words, size_t total) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const size_t row = t / topk;  // bh * nqb + qb
  if ((int)(t % topk) >= list_len(cnts, row, topk)) return;  // past the row's count
  const int qb = (int)(row % nqb);
  const size_t bh = row / nqb;
  const int kb = idx[t];
  if ((unsigned)kb >= (unsigned)nkb) return;  // out-of-range index: ignored
  atomicOr(&bitmap[(bh * nkb + kb) * words + qb / 32], 1u << (qb % 32));
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// one wave per (bh, kb): number of query blocks that selected kb
__global__ __launch_bounds__(256) void csc_count_kernel(const uint32_t* __restrict__ bitmap,
                                                        int32_t* __restrict__ counts, int cols, int words) {
  const int col = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= cols) return;
  const int lane = threadIdx.x & 63;
  int c = 0;
  for (int w = lane; w < words; w += 64) c += __popc(bitmap[(size_t)col * words + w]);
  c = wave_sum_i(c);
  if (lane == 0) counts[col] = c;
}

// one workgroup of 1024 threads per bh: the KV blocks of the head sorted by
// descending column length (ties: ascending block index), by a bitonic sort of
// unique keys ((nqb - count) << 12 | kb) in LDS.  The dK/dV kernel visits blocks
// in this order: the longest columns start first (load balance) and blocks
// that most query blocks selected run side by side, sharing Q/dO tiles in L2.
__global__ __launch_bounds__(1024) void csc_order_kernel(const int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ order, int nkb, int nqb) {
  __shared__ uint32_t key[4096];
  const int bh = blockIdx.x, tid = threadIdx.x;
  int p2 = 1;
  while (p2 < nkb) p2 <<= 1;
  for (int i = tid; i < p2; i += 1024)
    key[i] = i < nkb ? ((uint32_t)(nqb - counts[(size_t)bh * nkb + i]) << 12) | (uint32_t)i : 0xffffffffu;
  __syncthreads();
  for (int size = 2; size <= p2; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < p2; i += 1024) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const uint32_t a = key[i], b = key[j];
          if ((a > b) == up) {
            key[i] = b;
            key[j] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int i = tid; i < nkb; i += 1024) order[(size_t)bh * nkb + i] = (int32_t)(key[i] & 0xfffu);
}

// one workgroup of 1024 threads per bh: exclusive scan of counts[nkb] -> col_ptr[nkb + 1]
__global__ __launch_bounds__(1024) void csc_scan_kernel(const int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ col_ptr, int nkb) {
  __shared__ int32_t part[1024];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int per = (nkb + 1023) / 1024;
  const int32_t* c = counts + (size_t)bh * nkb;
  int32_t* cp = col_ptr + (size_t)bh * (nkb + 1);
  int s = 0;
  for (int i = 0; i < per; ++i) {
    const int j = tid * per + i;
    if (j < nkb) s += c[j];
  }
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;  // exclusive prefix of this thread's segment
  for (int i = 0; i < per; ++i) {
    const int j = tid * per + i;
    if (j < nkb) {
      cp[j] = run;
      run += c[j];
    }
  }
  if (tid == 1023) cp[nkb] = part[1023];
}

// one wave per (bh, kb): write the query blocks that selected kb, ascending
__global__ __launch_bounds__(256) void csc_emit_kernel(const uint32_t* __restrict__ bitmap,
                                                       const int32_t* __restrict__ col_ptr,
                                                       int32_t* __restrict__ rows, int cols, int nkb, int words,
                                                       int nnz_per_bh) {
  const int col = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= cols) return;
  const int lane = threadIdx.x & 63;
  const int bh = col / nkb, kb = col % nkb;
  int32_t* out = rows + (size_t)bh * nnz_per_bh + col_ptr[(size_t)bh * (nkb + 1) + kb];
  int base = 0;
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int w = w0 + lane;
    uint32_t bits = w < words ? bitmap[(size_t)col * words + w] : 0u;
    const int pc = __popc(bits);
    // exclusive prefix of pc over lanes
    int incl = pc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    int pos = base + incl - pc;
    while (bits) {
      const int b = __ffs(bits) - 1;
      out[pos++] = w * 32 + b;
      bits &= bits - 1;
    }
    base += __shfl(incl, 63);
  }
}

// ---------------------------------------------------------------- dK, dV (bf16, MFMA)
//
// One workgroup (4 waves) per KV block, in the per-head order of csc_order_kernel.
// Wave w owns keys (w % 2) * 32 .. +32 of the block and the query half (w / 2)
// of every 64-row chunk of the query blocks that selected the block.  K^T and
// V^T fragments stay in registers; Q and dO chunks are gathered into swizzled
// LDS tiles by direct global->LDS loads (double-buffered) and read both row-wise (A operands of S = Q K^T
// and dP = dO V^T) and transposed (B operands of dV += P^T dO, dK += dS^T Q).
// The two query halves' partial dK/dV are summed through LDS at the end.
//
// All four products are fp16, on copies scaled per head by powers of two (exact for bf16
// values): Q, K and dO come as fp16 copies from launch_bwd_prep_bf16, V is converted in
// registers.  S and dP are then the exact bf16 products scaled by 2^(sQ+sK) and 2^(sO+sV).
// dS is rounded to fp16 (2^-11 relative; a bf16 rounding lets Q's large entries amplify it into
// dK) after scaling by 2^r: dK sums over queries, so the scale is one per head, from
// |dS_ij| <= |dP_ij - D_i| <= 2 d max|dO| max|V|.  P <= 1 enters dV += P^T dO in fp16 as is.
// Every scale is undone exactly at the end.

template <int D, int BQ>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_bf16_kernel(
    const uint16_t* __restrict__ q16, const uint16_t* __restrict__ k16, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ o16 /* fp16 copy of dO */, const float* __restrict__ lse2,
    const float* __restrict__ dvec /* D 2^r */, const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ order, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    const uint32_t* __restrict__ absmax /* per head max |.| bits: K, Q, V, dO, bh_total each */, int bh_total,
    int n, int nnz_per_bh, int nwg, float c /* sm_scale*log2e */, float sm_scale) {
  constexpr int QR = 64;                 // query rows per chunk
  constexpr int NT = QR * D / 512;       // global->LDS instructions per tile
  constexpr int SUBS = BQ / QR;
  static_assert(BQ % QR == 0, "query block must be a multiple of 64 rows");
  // one array per buffer (see the dQ kernel): Q0/O0/L0 and Q1/O1/L1 (L: lse2[QR]
  // then D[QR]).  The four tile arrays double as the final reduction buffer.
  __shared__ __attribute__((aligned(16))) uint16_t Q0[QR * D], O0[QR * D], Q1[QR * D], O1[QR * D];
  __shared__ __attribute__((aligned(16))) float L0[2 * QR], L1[2 * QR];

  const int nkb = n / 64;
  const int id = xcd_remap(blockIdx.x, nwg);
  const int bh = id / nkb;
  const int kb = order[(size_t)bh * nkb + id % nkb];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const int kh = wave & 1, qh = wave >> 1;
  const size_t head = (size_t)bh * n * D;
  const int key = kb * 64 + kh * 32 + c32;  // this lane's key (column of S)

  const int32_t* cp = col_ptr + (size_t)bh * (nkb + 1);
  const int start = cp[kb], cnt = cp[kb + 1] - start;
  const int32_t* list = rows + (size_t)bh * nnz_per_bh + start;
  // per-head scales (wave-uniform, kept in scalar registers): r for dS, and the softmax constant
  // with S's scale 2^(sQ+sK) folded in
  struct Scales {
    int r, sQ, sK, sV, sO;
  };
  auto head_scales = [&]() {
    Scales h;
    h.sK = f16_shift(absmax[bh]);
    h.sQ = f16_shift(absmax[bh_total + bh]);
    h.sV = f16_shift(absmax[2 * bh_total + bh]);
    h.sO = f16_shift_wide(absmax[3 * bh_total + bh]);  // dO's shift cancels in pscale: not capped
    h.r = dkdv_ds_exponent<D>(absmax, bh, bh_total);
    return h;
  };
  auto uniform = [](float x) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x))); };
  const Scales hs = head_scales();
  const float cs = uniform(ldexpf(c, -(hs.sQ + hs.sK)));            // S is scaled by 2^(sQ+sK)
  const float pscale = uniform(ldexpf(1.f, hs.r - hs.sO - hs.sV));   // dP (scaled by 2^(sO+sV)) to 2^r
  const int sV = __builtin_amdgcn_readfirstlane(hs.sV);

  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) { dka[dt] = f32x16{}; dva[dt] = f32x16{}; }


  if (cnt > 0) {
    // K^T and V^T as B operands: lane holds its key, 8 consecutive d per chunk
    bf16x8 kf[D / 16];
    f16x8 vf[D / 16];
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc) {
      kf[dc] = as_bf16x8(ld16(k16 + head + (size_t)key * D + dc * 16 + g * 8));  // fp16 bits
      const u32x4 w = ld16(v + head + (size_t)key * D + dc * 16 + g * 8);
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = ldexpf(__uint_as_float(w[e] << 16), sV);
        f[2 * e + 1] = ldexpf(__uint_as_float(w[e] & 0xffff0000u), sV);
      }
      vf[dc] = cvt8h(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
    }
    const int nch = cnt * SUBS;
    auto q0_of = [&](int j) { return list[j / SUBS] * BQ + (j % SUBS) * QR; };
    // asynchronous gather of a 64-row chunk (Q and dO tiles, lse2 and D) into one buffer set
    auto issue = [&](int q0, uint16_t* qd, uint16_t* od, float* ld) {
      // instruction wave + 4m: Q rows for m < NT/4, dO rows after (compile-time per m); the lane
      // offset is computed once for the batch
      const int ln = opaque(lane);
#pragma unroll
      for (int m = 0; m < 2 * NT / 4; ++m) {
        const bool iso = m >= NT / 4;
        const int ii = wave + 4 * (iso ? m - NT / 4 : m);
        lds_load_rows<D>((iso ? o16 : q16) + head + (size_t)q0 * D, iso ? od : qd, ii, ln);
      }
      if (wave == 3 && lane < 32)  // lanes 0-15: 64 lse2 values, lanes 16-31: 64 D values
        __builtin_amdgcn_global_load_lds((lane < 16 ? lse2 : dvec) + (size_t)bh * n + q0 + (lane & 15) * 4, ld, 16,
                                         0, 0);
    };
    const int arow = qh * 32 + sigma(c32);
    auto chunk = [&](const uint16_t* qs, const uint16_t* os, const float* ld) {
      // Fragment offsets from two bases (see row_base / tr_base); kept opaque so that they are
      // recomputed here rather than held in registers for the whole loop: this kernel sits at the
      // 256-register limit of two waves per SIMD, and loop-invariant offsets (row_offsets /
      // tr_offsets, as the forward and dQ kernels use) would spill.
      const int rb = opaque(row_base<D>(arow, lane));
      // S = Q K^T and dP = dO V^T for this wave's 32 queries x 32 keys (A rows in sigma order),
      // each k-step's operands read one step ahead
      f32x16 s = f32x16{}, dp = f32x16{};
      bf16x8 qa = row_frag_at<D>(qs, rb, 0), oa = row_frag_at<D>(os, rb, 0);
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        bf16x8 qn = qa, on = oa;
        if (dc + 1 < D / 16) {
          qn = row_frag_at<D>(qs, rb, dc + 1);
          on = row_frag_at<D>(os, rb, dc + 1);
        }
        s = mfma32h(as_f16x8(qa), as_f16x8(kf[dc]), s);
        dp = mfma32h(as_f16x8(oa), vf[dc], dp);
        qa = qn;
        oa = on;
      }
      const int tb0 = opaque(tr_base<D>(qh * 32, lane, 0)), tb1 = opaque(tr_base<D>(qh * 32, lane, 1));
      // register vv holds query qh*32 + (vv/8)*16 + g*8 + vv%8 of the chunk: two runs of 8
      // consecutive queries.  Each run's lse2 and D are read as vectors right before use, and its
      // P and dS feed the dV and dK products at once, so only one run's values are live.
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int q0 = qh * 32 + cc * 16 + g * 8;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&ld[q0]);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&ld[q0 + 4]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&ld[QR + q0]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&ld[QR + q0 + 4]);
        float pv[8], dsv_[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int vv = cc * 8 + e;
          const float lq = e < 4 ? l0[e] : l1[e - 4];
          const float dd = e < 4 ? d0[e] : d1[e - 4];
          pv[e] = fast_exp2(fmaf(s[vv], cs, -lq));
          dsv_[e] = pv[e] * fmaf(dp[vv], pscale, -dd);  // dS 2^r (dd = D 2^r), exact scaling
        }
        const f16x8 pa = cvt8h(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
        const f16x8 da = cvt8h(dsv_[0], dsv_[1], dsv_[2], dsv_[3], dsv_[4], dsv_[5], dsv_[6], dsv_[7]);
        // rows cc*16.. of the query half: bases move by 16 rows
        const int o0 = tb0 + cc * 32 * D, o1 = tb1 + cc * 32 * D;
        bf16x8 ob = tr_frag_at<D>(os, o0, o1, 0), qb = tr_frag_at<D>(qs, o0, o1, 0);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          bf16x8 obn = ob, qbn = qb;
          if (dt + 1 < D / 32) {
            obn = tr_frag_at<D>(os, o0, o1, dt + 1);
            qbn = tr_frag_at<D>(qs, o0, o1, dt + 1);
          }
          dva[dt] = mfma32h(pa, as_f16x8(ob), dva[dt]);
          dka[dt] = mfma32h(da, as_f16x8(qb), dka[dt]);
          ob = obn;
          qb = qbn;
        }
      }
    };
    // two chunks per trip so that each buffer is a distinct array
    issue(q0_of(0), Q0, O0, L0);
    __syncthreads();
    for (int j = 0; j < nch; j += 2) {
      if (j + 1 < nch) issue(q0_of(j + 1), Q1, O1, L1);
      chunk(Q0, O0, L0);
      __syncthreads();
      if (j + 1 < nch) {
        if (j + 2 < nch) issue(q0_of(j + 2), Q0, O0, L0);
        chunk(Q1, O1, L1);
        __syncthreads();
      }
    }
  }
  // sum the two query halves through LDS (the tiles are free after the last barrier)
  // array kh*2 + which of {Q0, O0, Q1, O1} holds (D/32) x 16 x 64 floats: exactly its size
  static_assert((D / 32) * 16 * 64 * 4 == QR * D * 2, "each tile array holds one reduction slab");
  auto red = [&](int which) {
    return reinterpret_cast<float*>(kh == 0 ? (which == 0 ? Q0 : O0) : (which == 0 ? Q1 : O1));
  };
  auto ridx = [&](int dt, int vv) { return (dt * 16 + vv) * 64 + lane; };
  if (qh == 1) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        red(0)[ridx(dt, vv)] = dka[dt][vv];
        red(1)[ridx(dt, vv)] = dva[dt][vv];
      }
  }
  __syncthreads();
  if (qh == 0) {
    const Scales h = head_scales();  // recomputed rather than held through the loop
    const int unscale_k = __builtin_amdgcn_readfirstlane(-(h.r + h.sQ));
    const int unscale_v = __builtin_amdgcn_readfirstlane(-h.sO);
    // D layout of dK/dV tiles: lane holds d = dt*32 + c32; register vv holds key (vv/4)*8 + g*4 + vv%4
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int kr = kb * 64 + kh * 32 + (vv >> 2) * 8 + g * 4 + (vv & 3);
        const size_t off = head + (size_t)kr * D + dt * 32 + c32;
        dk[off] = f32_to_bf16(ldexpf((dka[dt][vv] + red(0)[ridx(dt, vv)]) * sm_scale, unscale_k));  // exact
        dv[off] = f32_to_bf16(ldexpf(dva[dt][vv] + red(1)[ridx(dt, vv)], unscale_v));                // unscale
      }
  }
}

// ---------------------------------------------------------------- dQ (bf16 inputs, MFMA)
//
// One workgroup per query block (Bq/32 waves, 32 rows each) walking its k
// selected blocks: S^T = K Q^T and dP^T = V dO^T are recomputed, and
// dQ^T += K^T dS^T takes K^T from transposing reads of the row-major K tile.
//
// S and dQ are fp16 products: K comes as an fp16 copy scaled by 2^sK (sK = f16_shift of the
// head's max |K|; exact for bf16 values; made by launch_bwd_prep_bf16), Q is converted in
// registers with its own head shift sQ,
// so S is the exact bf16 product scaled by 2^(sQ+sK).  dS is rounded to fp16 (2^-11 relative;
// a bf16 rounding would let K's large entries amplify dS's error into dQ) after scaling row i by
// 2^r_i, with r_i from the bound |dS_ij| = P_ij |dP_ij - D_i| <= 2 |dO_i|_1 max|V| (both dP_ij
// and D_i are dO_i against a row of V or a convex mix of them), which keeps it inside fp16's
// range at full precision.  dQ is unscaled exactly at the end.  dP stays a bf16 product.

template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, (kMinWavesPerSimd<D, BQ>)) void attn_bwd_dq_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k16, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse2, const float* __restrict__ dvec,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ cnts, uint16_t* __restrict__ dq,
    const uint32_t* __restrict__ absmax /* per head max |.| bits: [0,bh) K, [bh,2bh) Q, [2bh,3bh) V */, int bh_total,
    int n, int topk, float c, float sm_scale) {
  constexpr int WAVES = BQ / 32;
  constexpr int NI = 2 * 64 * D / 512;  // global->LDS instructions per KV block (K and V tiles)
  // one array per buffer, so the compiler can see that the asynchronous copy into
  // one buffer never aliases the reads of the other (no waits mid-compute)
  __shared__ __attribute__((aligned(16))) uint16_t K0[64 * D], K1[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t V0[64 * D], V1[64 * D];

  const int nqb = n / BQ;
  const int id = blockIdx.x;  // plain dispatch order, as the forward (measured faster than the remap)
  const int bh = id / nqb, qb = id % nqb;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, c32 = lane & 31;
  const size_t head = (size_t)bh * n * D;
  const int32_t* blocks = idx + ((size_t)bh * nqb + qb) * topk;
  const int kq = list_len(cnts, (size_t)bh * nqb + qb, topk);  // blocks in this query block's list
  const int qrow = qb * BQ + wave * 32 + c32;
  const int nkb = n / 64;
  auto blk_at = [&](int j) { return min(max(blocks[j], 0), nkb - 1); };  // clamp out-of-range indices
  auto issue = [&](int blk, uint16_t* kd, uint16_t* vd) {  // asynchronous gather of a K and V block
    // instruction wave + WAVES m: K rows for m < NI/2/WAVES, V rows after (compile-time per m);
    // the lane offset is computed once for the batch
    const int ln = opaque(lane);
#pragma unroll
    for (int m = 0; m < NI / WAVES; ++m) {
      const bool isv = m >= NI / 2 / WAVES;
      const int ii = wave + WAVES * (isv ? m - NI / 2 / WAVES : m);
      lds_load_rows<D>((isv ? v : k16) + head + (size_t)blk * 64 * D, isv ? vd : kd, ii, ln);
    }
  };
  const int sK = f16_shift(absmax[bh]), sQ = f16_shift(absmax[bh_total + bh]);
  const float vmax = __uint_as_float(absmax[2 * bh_total + bh]);

  f16x8 qf[D / 16];
  bf16x8 of[D / 16];
  float l1 = 0.f;  // |dO_i|_1 over this lane's half of the row
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    const u32x4 w = ld16(q + head + (size_t)qrow * D + dc * 16 + g * 8);
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = ldexpf(__uint_as_float(w[e] << 16), sQ);
      f[2 * e + 1] = ldexpf(__uint_as_float(w[e] & 0xffff0000u), sQ);
    }
    qf[dc] = cvt8h(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
    const u32x4 od = ld16(dout + head + (size_t)qrow * D + dc * 16 + g * 8);
    of[dc] = as_bf16x8(od);
#pragma unroll
    for (int e = 0; e < 4; ++e) l1 += fabsf(__uint_as_float(od[e] << 16)) + fabsf(__uint_as_float(od[e] & 0xffff0000u));
  }
  l1 += xor32(l1);
  // dS row scale 2^r (a normal float), r from the bound 2 |dO_i|_1 max|V| on |dS_ij|
  const int r = min(max(f16_exponent(__float_as_uint(2.f * l1 * vmax)), -120), 120);
  const float dscale = ldexpf(1.f, r);
  const float my_lse2 = lse2[(size_t)bh * n + qrow];
  const float my_ds = dvec[(size_t)bh * n + qrow] * dscale;  // D_i 2^r
  const float cs = ldexpf(c, -(sQ + sK));                     // S is scaled by 2^(sQ+sK)

  issue(blk_at(0), K0, V0);
  __syncthreads();
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  const int arow = sigma(c32);
  // loop-invariant fragment offsets (row_offsets / tr_offsets): the 32-key tile t adds t*64*D
  // bytes to a row read, the 16-key chunk cc adds cc*32*D to a transposed read
  int rbs[D / 16], tb0s[D / 32], tb1s[D / 32];
  row_offsets<D>(rbs, arow, lane);
  tr_offsets<D>(tb0s, tb1s, 0, lane);
  auto rd_row = [&](const uint16_t* tile, int dc, int add) { return row_frag_off(tile, rbs[dc], add); };
  auto rd_tr = [&](const uint16_t* tile, int dt, int add) { return tr_frag_off(tile, tb0s[dt], tb1s[dt], add); };
  auto block = [&](const uint16_t* Kc, const uint16_t* Vc) {
    // one 32-key tile at a time: S^T, dP^T, dS^T, then its two 16-key chunks of dQ^T += K^T dS^T;
    // each k-step's operands read one step ahead
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const int rt = t * 64 * D;
      bf16x8 ka = rd_row(Kc, 0, rt), va = rd_row(Vc, 0, rt);
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc) {
        bf16x8 kn = ka, vn = va;
        if (dc + 1 < D / 16) {
          kn = rd_row(Kc, dc + 1, rt);
          vn = rd_row(Vc, dc + 1, rt);
        }
        s = mfma32h(as_f16x8(ka), qf[dc], s);
        dp = mfma32(va, of[dc], dp);
        ka = kn;
        va = vn;
      }
      // dS 2^r = P (dP 2^r - D 2^r): the scaling is exact, folded into one fma
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const float p = fast_exp2(fmaf(s[vv], cs, -my_lse2));
        dp[vv] = p * fmaf(dp[vv], dscale, -my_ds);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int b0 = h2 * 8, cc = t * 2 + h2;
        const f16x8 ds = cvt8h(dp[b0], dp[b0 + 1], dp[b0 + 2], dp[b0 + 3], dp[b0 + 4], dp[b0 + 5], dp[b0 + 6],
                               dp[b0 + 7]);
        bf16x8 kt = rd_tr(Kc, 0, cc * 32 * D);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          bf16x8 ktn = kt;
          if (dt + 1 < D / 32) ktn = rd_tr(Kc, dt + 1, cc * 32 * D);
          acc[dt] = mfma32h(as_f16x8(kt), ds, acc[dt]);
          kt = ktn;
        }
      }
    }
  };
  // two blocks per trip so that each buffer is a distinct array (an empty list leaves dQ = 0)
  for (int j = 0; j < kq; j += 2) {
    if (j + 1 < kq) issue(blk_at(j + 1), K1, V1);
    block(K0, V0);
    __syncthreads();
    if (j + 1 < kq) {
      if (j + 2 < kq) issue(blk_at(j + 2), K0, V0);
      block(K1, V1);
      __syncthreads();
    }
  }
  uint16_t* out = dq + head + (size_t)qrow * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int vq = 0; vq < 4; ++vq) {
      const int d0 = dt * 32 + vq * 8 + g * 4;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = ldexpf(acc[dt][vq * 4 + e] * sm_scale, -(r + sK));  // exact unscale
      u32x2 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      *reinterpret_cast<u32x2*>(out + d0) = pk;
    }
}

// ---------------------------------------------------------------- f32 path (plain VALU)

__global__ void attn_bwd_dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                       const float* __restrict__ v, const float* __restrict__ dout,
                                       const float* __restrict__ lse, const float* __restrict__ dvec,
                                       const int32_t* __restrict__ idx, const int32_t* __restrict__ cnts,
                                       float* __restrict__ dq, int n, int d, int bq, int bk, int topk, float scale) {
  // one thread per query row and output column c: grid (ceil(n*d/256), BH)
  const int bh = blockIdx.y;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (size_t)n * d) return;
  const int i = (int)(t / d), col = (int)(t % d);
  const size_t head = (size_t)bh * n * d;
  const float* qi = q + head + (size_t)i * d;
  const float* gi = dout + head + (size_t)i * d;
  const float li = lse[(size_t)bh * n + i], di = dvec[(size_t)bh * n + i];
  const size_t qrow = (size_t)bh * (n / bq) + i / bq;
  const int32_t* blocks = idx + qrow * topk;
  const int kq = list_len(cnts, qrow, topk);
  float acc = 0.f;
  for (int jb = 0; jb < kq; ++jb) {
    const int kb = min(max(blocks[jb], 0), n / bk - 1);  // clamp out-of-range indices
    for (int j = kb * bk; j < (kb + 1) * bk; ++j) {
      const float* kj = k + head + (size_t)j * d;
      const float* vj = v + head + (size_t)j * d;
      float s = 0.f, dp = 0.f;
      for (int cc = 0; cc < d; ++cc) {
        s = fmaf(qi[cc], kj[cc], s);
        dp = fmaf(gi[cc], vj[cc], dp);
      }
      const float p = expf(s * scale - li);
      acc = fmaf(p * (dp - di), kj[col], acc);
    }
  }
  dq[head + (size_t)i * d + col] = acc * scale;
}

__global__ void attn_bwd_dkdv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                         const float* __restrict__ v, const float* __restrict__ dout,
                                         const float* __restrict__ lse, const float* __restrict__ dvec,
                                         const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ rows,
                                         float* __restrict__ dk, float* __restrict__ dv, int n, int d, int bq, int bk,
                                         int nnz_per_bh, float scale) {
  // one thread per key row and output column: grid (ceil(n*d/256), BH)
  const int bh = blockIdx.y;
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (size_t)n * d) return;
  const int j = (int)(t / d), col = (int)(t % d);
  const int nkb = n / bk, kb = j / bk;
  const size_t head = (size_t)bh * n * d;
  const float* kj = k + head + (size_t)j * d;
  const float* vj = v + head + (size_t)j * d;
  const int32_t* cp = col_ptr + (size_t)bh * (nkb + 1);
  const int32_t* list = rows + (size_t)bh * nnz_per_bh;
  float ak = 0.f, av = 0.f;
  for (int e = cp[kb]; e < cp[kb + 1]; ++e) {
    const int qb = list[e];
    for (int i = qb * bq; i < (qb + 1) * bq; ++i) {
      const float* qi = q + head + (size_t)i * d;
      const float* gi = dout + head + (size_t)i * d;
      float s = 0.f, dp = 0.f;
      for (int cc = 0; cc < d; ++cc) {
        s = fmaf(qi[cc], kj[cc], s);
        dp = fmaf(gi[cc], vj[cc], dp);
      }
      const float p = expf(s * scale - lse[(size_t)bh * n + i]);
      av = fmaf(p, gi[col], av);
      ak = fmaf(p * (dp - dvec[(size_t)bh * n + i]), qi[col], ak);
    }
  }
  dk[head + (size_t)j * d + col] = ak * scale;
  dv[head + (size_t)j * d + col] = av;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_bwd_pre_bf16(const uint16_t* o, const uint16_t* o_lo, const uint16_t* dout, const float* lse,
                               float* dvec, float* lse2, float* dvec_s, const void* f16ws, int bh, int n, int d,
                               hipStream_t st) {
  const int rows = bh * n;
  const int lanes = rows * (d / 8);
  dim3 grid((lanes + 255) / 256);
  const uint32_t* absmax = bwd_f16_absmax(f16ws, bh, n, d);
  if (d == 64)
    hipLaunchKernelGGL(bwd_pre_bf16_kernel<64>, grid, dim3(256), 0, st, o, o_lo, dout, lse, dvec, lse2, dvec_s, absmax,
                       n, bh, rows);
  else if (d == 128)
    hipLaunchKernelGGL(bwd_pre_bf16_kernel<128>, grid, dim3(256), 0, st, o, o_lo, dout, lse, dvec, lse2, dvec_s,
                       absmax, n, bh, rows);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_pre_f32(const float* o, const float* dout, float* dvec, int rows, int d, hipStream_t st) {
  hipLaunchKernelGGL(bwd_pre_f32_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, o, dout, dvec, rows, d);
  return hipGetLastError();
}

hipError_t launch_csc(const int32_t* idx, const int32_t* cnts, uint32_t* bitmap, int32_t* counts, int32_t* col_ptr,
                      int32_t* rows, int32_t* order, int bh, int nqb, int nkb, int topk, hipStream_t st) {
  const int words = (nqb + 31) / 32;
  const size_t nbits = (size_t)bh * nkb * words;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)std::min<size_t>((nbits + 255) / 256, 65535)), dim3(256), 0,
                     st, bitmap, nbits, 0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)bh * nqb * topk;
  hipLaunchKernelGGL(csc_mark_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, idx, cnts, bitmap,
                     nqb, nkb, topk, words, total);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int cols = bh * nkb;
  hipLaunchKernelGGL(csc_count_kernel, dim3((cols + 3) / 4), dim3(256), 0, st, bitmap, counts, cols, words);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(csc_scan_kernel, dim3(bh), dim3(1024), 0, st, counts, col_ptr, nkb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (order) {
    hipLaunchKernelGGL(csc_order_kernel, dim3(bh), dim3(1024), 0, st, counts, order, nkb, nqb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(csc_emit_kernel, dim3((cols + 3) / 4), dim3(256), 0, st, bitmap, col_ptr, rows, cols, nkb,
                     words, nqb * topk);
  return hipGetLastError();
}

// The backward's fp16 copies and per-head maxima, in the workspace at `ws`:
//   K16, Q16, dO16 [bh, n, d] each, partial maxima, absmax [4][bh] (K, Q, V, dO).
size_t bwd_f16_ws_bytes(int bh, int n, int d) {
  return 3 * align_ws((size_t)bh * n * d * 2) + head_absmax_ws_bytes(bh) + align_ws((size_t)bh * 4 * 4);
}

namespace {
struct F16Views {
  uint16_t* k16;
  uint16_t* q16;
  uint16_t* o16;
  uint32_t* part;
  uint32_t* absmax;
};
F16Views f16_views(void* ws, int bh, int n, int d) {
  char* w = static_cast<char*>(ws);
  const size_t t = align_ws((size_t)bh * n * d * 2);
  return {reinterpret_cast<uint16_t*>(w), reinterpret_cast<uint16_t*>(w + t), reinterpret_cast<uint16_t*>(w + 2 * t),
          reinterpret_cast<uint32_t*>(w + 3 * t), reinterpret_cast<uint32_t*>(w + 3 * t + head_absmax_ws_bytes(bh))};
}
}  // namespace

const uint32_t* bwd_f16_absmax(const void* ws, int bh, int n, int d) {
  return f16_views(const_cast<void*>(ws), bh, n, d).absmax;
}

hipError_t launch_bwd_prep_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout, void* ws,
                                int bh, int n, int d, hipStream_t st) {
  const F16Views f = f16_views(ws, bh, n, d);
  const size_t per_head = (size_t)n * d;
  hipError_t e = launch_head_absmax(k, f.part, f.absmax, bh, per_head, st);
  if (e != hipSuccess) return e;
  if ((e = launch_to_f16(k, f.absmax, f.k16, bh, per_head, st)) != hipSuccess) return e;
  if ((e = launch_head_absmax(q, f.part, f.absmax + bh, bh, per_head, st)) != hipSuccess) return e;
  if ((e = launch_to_f16(q, f.absmax + bh, f.q16, bh, per_head, st)) != hipSuccess) return e;
  if ((e = launch_head_absmax(v, f.part, f.absmax + 2 * bh, bh, per_head, st)) != hipSuccess) return e;
  if ((e = launch_head_absmax(dout, f.part, f.absmax + 3 * bh, bh, per_head, st)) != hipSuccess) return e;
  return launch_to_f16(dout, f.absmax + 3 * bh, f.o16, bh, per_head, st, /*wide=*/true);
}

hipError_t launch_bwd_dkdv_bf16(const void* ws, const uint16_t* v, const uint16_t* dout, const float* lse2,
                                const float* dvec, const int32_t* col_ptr, const int32_t* rows, const int32_t* order,
                                uint16_t* dk, uint16_t* dv, int bh, int n, int d, int bq, int topk, float sm_scale,
                                hipStream_t st) {
  const F16Views f = f16_views(const_cast<void*>(ws), bh, n, d);
  const int nwg = bh * (n / 64);
  const int nnz = (n / bq) * topk;
  const float c = sm_scale * kLog2e;
#define DKDV(D_, BQ_)                                                                                          \
  if (d == D_ && bq == BQ_) {                                                                                  \
    hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D_, BQ_>), dim3(nwg), dim3(256), 0, st, f.q16, f.k16, v, f.o16, \
                       lse2, dvec, col_ptr, rows, order, dk, dv, f.absmax, bh, n, nnz, nwg, c, sm_scale);     \
    return hipGetLastError();                                                                                  \
  }
  DKDV(64, 64) DKDV(64, 128) DKDV(128, 64) DKDV(128, 128)
#undef DKDV
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(const uint16_t* q, const uint16_t* v, const uint16_t* dout, const float* lse2,
                              const float* dvec, const int32_t* idx, const int32_t* cnts, uint16_t* dq, const void* ws,
                              int bh, int n, int d, int bq, int topk, float sm_scale, hipStream_t st) {
  const F16Views f = f16_views(const_cast<void*>(ws), bh, n, d);
  const int nwg = bh * (n / bq);
  const float c = sm_scale * kLog2e;
#define DQ(D_, BQ_)                                                                                          \
  if (d == D_ && bq == BQ_) {                                                                                \
    hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D_, BQ_>), dim3(nwg), dim3(BQ_ * 2), 0, st, q, f.k16, v, dout,  \
                       lse2, dvec, idx, cnts, dq, f.absmax, bh, n, topk, c, sm_scale);                       \
    return hipGetLastError();                                                                                \
  }
  DQ(64, 64) DQ(64, 128) DQ(128, 64) DQ(128, 128)
#undef DQ
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* dout, const float* lse,
                          const float* dvec, const int32_t* idx, const int32_t* cnts, const int32_t* col_ptr,
                          const int32_t* rows, float* dq, float* dk, float* dv, int bh, int n, int d, int bq, int bk,
                          int topk, float sm_scale, hipStream_t st) {
  dim3 grid((unsigned)(((size_t)n * d + 255) / 256), bh);
  hipLaunchKernelGGL(attn_bwd_dq_f32_kernel, grid, dim3(256), 0, st, q, k, v, dout, lse, dvec, idx, cnts, dq, n, d,
                     bq, bk, topk, sm_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel, grid, dim3(256), 0, st, q, k, v, dout, lse, dvec, col_ptr, rows, dk,
                     dv, n, d, bq, bk, (n / bq) * topk, sm_scale);
  return hipGetLastError();
}

}  // namespace dsv
