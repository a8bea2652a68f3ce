// Shared device helpers for the gfx950 (CDNA4) kernels: bf16 conversion, MFMA
// fragment types, wave-level exchange, and the problem description passed to
// kernels.
//
// MFMA fragment conventions used throughout (verified on the device with an
// in-bounds layout check against a host matmul):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row (l % 32), 8 consecutive k starting at (l / 32) * 8
//     B: lane l holds col (l % 32), 8 consecutive k starting at (l / 32) * 8
//     D: lane l holds col (l % 32); register v holds row (v/4)*8 + (l/32)*4 + v%4
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds row (l % 16), 8 consecutive k starting at (l / 16) * 8
//     B: lane l holds col (l % 16), same k
//     D: lane l holds col (l % 16); register v holds row (l/16)*4 + v
//
// Row permutation "sigma" (swap bits 2 and 3 of a row index inside a 32-row
// tile).  If the A operand's row r is loaded from source row sigma(r), then in
// the 32x32 D layout lane group g = l/32, register v corresponds to source row
//   (v / 8) * 16 + g * 8 + (v % 8),
// which is exactly the k layout of a B (or A) operand: registers 0..7 of a lane
// form the operand for source rows [0, 16), registers 8..15 for [16, 32).  This
// lets a softmax tile computed by one MFMA feed the next MFMA straight from
// registers, with no LDS round trip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16 bits, round to nearest even (NaN -> quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Eight floats -> one bf16 MFMA operand (hardware round-to-nearest-even).
__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3, float a4, float a5,
                                       float a6, float a7) {
  f32x8 f = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(f, bf16x8);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp16 operands: eight floats -> one fp16 MFMA operand (v_cvt_pk_f16_f32, round to nearest even)
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8 cvt8h(float a0, float a1, float a2, float a3, float a4, float a5,
                                       float a6, float a7) {
  f32x8 f = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(f, f16x8);
}
__device__ __forceinline__ f16x8 as_f16x8(bf16x8 x) { return __builtin_bit_cast(f16x8, x); }
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Power-of-two exponent s such that a maximum magnitude m (float bits, m >= 0) scaled by 2^s lies
// in [2^14, 2^15): values scaled by 2^s fit fp16's range (largest finite 65504), and a bf16 value
// down to 2^-28 of the maximum stays exact.  0 for m = 0 or non-finite.
__device__ __forceinline__ int f16_exponent(uint32_t m) {
  if (m == 0 || m >= 0x7f800000u) return 0;
  return 14 - ((int)(m >> 23) - 127);
}
// The same for the per-head fp16 copies of tensors, capped to [-40, 40] so that the products of
// two scaled copies and the inverse scales folded into softmax constants stay normal floats
// (maxima in [2^-26, 2^54] reach the target range; a larger one would overflow fp16).
constexpr int kAbsmaxParts = 32;  // partial maxima per head
__device__ __forceinline__ int f16_shift(uint32_t m) { return min(max(f16_exponent(m), -40), 40); }
// The wide form, for a copy whose scale only meets its own inverse (the output gradient: its
// shift cancels in dS's scale), so tiny training gradients keep full precision.
__device__ __forceinline__ int f16_shift_wide(uint32_t m) { return min(max(f16_exponent(m), -120), 120); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// max / sum of a value and its lane ^ 32 partner, via v_permlane32_swap (a VALU
// exchange of the two wave halves, no LDS).  The two results of the swap hold
// {x[l], x[l ^ 32]} in some order, and both reductions are symmetric.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// sigma: swap bits 2 and 3 of a row index (see the header comment).
__device__ __forceinline__ int sigma(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- LDS tiles
//
// A tile of rows x D bf16 values is stored row-major with no padding; the
// 16-byte chunks of row r are XOR-swizzled by h(r):
//   D = 128 (256-byte rows):  h(r) = 4*(r % 4) + (r / 4) % 4
//   D = 64  (128-byte rows):  h(r) = 4*((r / 2) % 2) + (r / 4) % 4
// The LDS serves 64 banks x 4 bytes per cycle (16 lanes of a 16-byte read, 32
// lanes of an 8-byte read; bank-conflict counters confirm the width).  With
// this swizzle both access patterns the kernels use are conflict-free:
//  * row reads: 16 lanes read 16 bytes each from 16 consecutive rows (in sigma
//    order), same logical chunk (MFMA operands whose k runs along the row);
//  * transposed reads (ds_read_b64_tr_b16): 32 lanes read a 4-row x 32-column
//    block (4 logical chunks of 4 consecutive rows).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// element offset of (row, col) in a swizzled tile with D columns
template <int D>
__device__ __forceinline__ int toff(int r, int col) {
  return r * D + ((((col >> 3) ^ swz<D>(r)) & (D / 8 - 1)) << 3) + (col & 7);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16, measured lane layout: within each 16-lane group, source
// lane s supplies the address of 4 consecutive elements of row s/4, columns
// 4*(s%4)..+3 of a 4 x 16 block; output lane i receives column i of the block
// (its 4 rows, in row order).
__device__ __forceinline__ i16x4 ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// MFMA 32x32x16 operand (A or B) whose k index runs down the ROWS of a
// row-major swizzled tile X[k][m]: lane l receives m = m0 + l % 32 and
// k = k0 + (l / 32) * 8 + 0..7 -- the same fragment a row-major X^T would give.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int k0, int m0, int lane) {
  const int row = k0 + (lane >> 5) * 8 + ((lane & 15) >> 2);
  const int col = m0 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  const i16x4 a = ds_read_tr16(tile + toff<D>(row, col));
  const i16x4 b = ds_read_tr16(tile + toff<D>(row + 4, col));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

// MFMA operand whose k index runs ALONG a row of a swizzled tile: lane l reads
// row `row`, columns k0 + (l / 32) * 8 + 0..7.
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const uint16_t* tile, int row, int k0, int lane) {
  return as_bf16x8(ld16(tile + toff<D>(row, k0 + (lane >> 5) * 8)));
}

// Cheap addressing of a run of fragments.  The k-step (16 columns) or the
// 32-column tile index only moves bits of the offset that neither the row term
// nor the lane's in-chunk term touch, and it enters the swizzle by XOR.  So one
// base offset per lane serves the whole run.  Bases are BYTE offsets, so each
// fragment address costs one XOR:
//   row_frag(tile, row, 16*s, lane) == tile bytes [row_base(row, lane) ^ (s << 5)]
//   tr_frag (tile, k0, 32*t, lane)  == reads at tr_base{0,1}(k0, lane) ^ (t << 6)
// (s < D/16, t < D/32).  Moving k0 or row by 16 adds 32*D bytes to the base,
// since the swizzle depends on the row modulo 16 only.
template <int D>
__device__ __forceinline__ int row_base(int row, int lane) { return toff<D>(row, (lane >> 5) * 8) * 2; }

template <int D>
__device__ __forceinline__ bf16x8 row_frag_at(const uint16_t* tile, int base, int s) {
  return as_bf16x8(ld16(reinterpret_cast<const char*>(tile) + (base ^ (s << 5))));
}

template <int D>
__device__ __forceinline__ int tr_base(int k0, int lane, int half) {
  const int row = k0 + (lane >> 5) * 8 + ((lane & 15) >> 2) + half * 4;
  const int col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  return toff<D>(row, col) * 2;
}

template <int D>
__device__ __forceinline__ bf16x8 tr_frag_at(const uint16_t* tile, int b0, int b1, int t) {
  const char* base = reinterpret_cast<const char*>(tile);
  const i16x4 a = ds_read_tr16(reinterpret_cast<const uint16_t*>(base + (b0 ^ (t << 6))));
  const i16x4 b = ds_read_tr16(reinterpret_cast<const uint16_t*>(base + (b1 ^ (t << 6))));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

// Loop-invariant fragment offsets.  Within a tile, the XOR of the swizzle only touches the
// offset bits of the k-step (row reads) or of the 32-column tile (transposed reads), while whole
// 16-row steps move bits above them.  So the per-step XOR can be done once, outside a loop, and
// a 16-row (or 32-key) step becomes a plain add that folds into the read's immediate offset:
//   row_frag(tile, row + 16*u, 16*s, lane)  == row_frag_off(tile, off[s], 32*D*u),
//     off = row_offsets(row, lane);
//   tr_frag(tile, k0 + 16*u, 32*t, lane)    == tr_frag_off(tile, o0[t], o1[t], 32*D*u),
//     (o0, o1) = tr_offsets(k0, lane).
// That costs D/16 + D/8 registers and removes one VALU op from every LDS read in the loop.
template <int D>
__device__ __forceinline__ void row_offsets(int (&off)[D / 16], int row, int lane) {
  const int b = row_base<D>(row, lane);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) off[s] = b ^ (s << 5);
}
template <int D>
__device__ __forceinline__ void tr_offsets(int (&o0)[D / 32], int (&o1)[D / 32], int k0, int lane) {
  const int b0 = tr_base<D>(k0, lane, 0), b1 = tr_base<D>(k0, lane, 1);
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    o0[t] = b0 ^ (t << 6);
    o1[t] = b1 ^ (t << 6);
  }
}
__device__ __forceinline__ bf16x8 row_frag_off(const uint16_t* tile, int off, int add) {
  return as_bf16x8(ld16(reinterpret_cast<const char*>(tile) + add + off));
}
__device__ __forceinline__ bf16x8 tr_frag_off(const uint16_t* tile, int o0, int o1, int add) {
  const char* base = reinterpret_cast<const char*>(tile) + add;
  const i16x4 a = ds_read_tr16(reinterpret_cast<const uint16_t*>(base + o0));
  const i16x4 b = ds_read_tr16(reinterpret_cast<const uint16_t*>(base + o1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

// Keep a value in a register without letting the compiler see through it, so
// that offsets derived from it are recomputed where used instead of being
// hoisted out of a loop into registers of their own.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Asynchronous copy of global memory into a swizzled LDS tile: one
// global_load_lds_dwordx4 moves 64 x 16 bytes, lane L landing at LDS base +
// 16 * L (measured on the device), i.e. rows [i*R, i*R + R) of the tile with
// R = 512 / D.  Lane L fills physical chunk p = L % (D/8) of its row, which holds
// logical chunk p ^ swz(row).  `src` points at the tile's first global row (row
// stride D elements); `dst` is the LDS tile; `i` is the instruction index.
// The data is visible after the next __syncthreads() (the compiler waits for
// the outstanding loads before the barrier).
//
// The address is a uniform base (the tile's row i*R, in scalar registers) plus the lane's byte
// offset within those R rows.  The swizzle repeats every 16 rows, so that offset depends on i only
// modulo 16/R: a batch of copies whose instruction indices step by a multiple of 16/R computes it
// once.  Callers inside a loop pass the lane id through opaque() once per batch: the offset is then
// recomputed per batch (three VALU ops) rather than hoisted out of the loop, where the compiler
// would hold it as a 64-bit value and give up the scalar-base form of the load.
template <int D>
__device__ __forceinline__ uint32_t lds_lane_off(int i, int lane) {
  constexpr int R = 512 / D, P = 16 / R;
  const int row = (i & (P - 1)) * R + lane / (D / 8);  // the row modulo 16
  const int c = ((lane % (D / 8)) ^ swz<D>(row)) & (D / 8 - 1);
  return (uint32_t)((lane / (D / 8)) * D + c * 8) * 2u;
}
template <int D>
__device__ __forceinline__ void lds_load_rows(const uint16_t* src, uint16_t* dst, int i, int lane) {
  constexpr int R = 512 / D;
  const char* rows = reinterpret_cast<const char*>(src) + (size_t)i * R * D * 2;
  const uint32_t off = lds_lane_off<D>(i, lane);
  __builtin_amdgcn_global_load_lds(rows + off, dst + i * 512, 16, 0, 0);
}

// Waves per SIMD a query-parallel attention kernel (Bq/32 waves per workgroup, four 64-key K/V
// tiles of D columns in LDS) can reach: two, except at D = 128 with Bq = 64, where a workgroup of
// two waves holds 64 KB of LDS, two workgroups fill a compute unit's 160 KB and each SIMD runs one
// wave (the register budget is then that of one wave).
template <int D, int BQ>
constexpr int kMinWavesPerSimd = (D == 128 && BQ == 64) ? 1 : 2;

// Workspace sub-buffers start on 256-byte boundaries.
__host__ __device__ inline size_t align_ws(size_t x) { return (x + 255) / 256 * 256; }

// Length of query-block row `row`'s block list: its count when per-row counts are given
// (clamped to [0, k]), else k.
__device__ __forceinline__ int list_len(const int32_t* cnts, size_t row, int k) {
  return cnts ? min(max(cnts[row], 0), k) : k;
}

// Map a workgroup id so that consecutive logical ids run on the same XCD.
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8); with this
// remap XCD x processes the contiguous logical range [x*per, (x+1)*per).  The
// dK/dV kernel uses it: the ~64 KV-block columns an XCD runs together are then
// neighbours in the heaviest-first order of one head and share its Q/dO tiles in
// that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int per = n / 8;
  if (per == 0 || id >= per * 8) return id;
  return (id % 8) * per + id / 8;
}

}  // namespace dsv
