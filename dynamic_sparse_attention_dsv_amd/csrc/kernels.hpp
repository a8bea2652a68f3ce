// Host-callable launchers of the device kernels (each enqueues on `st` and
// returns the launch status).  Pointers are device pointers; sizes are
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsv {

// predictor
// out = rho(scale * x w): the query side passes scale = pred_scale * log2(e), the key side 1
hipError_t launch_proj_bf16(const uint16_t* x, const uint16_t* w, uint16_t* out, int bh, int n, int heads,
                            int d, int r, float scale, hipStream_t st);
hipError_t launch_proj_f32(const float* x, const float* w, float* out, int bh, int n, int heads, int d, int r,
                           float scale, hipStream_t st);
int score_slots(int items);
size_t score_scratch_bytes(int items, int nkb);
int score_items(int bh, int n, int bq, bool representative);
// rep < 0: block scores (every row of a query block); rep >= 0: the masses of row qb * bq + rep.
// qlr is the scaled query projection: <qlr_i, klr_j> is the logit in log2 units.
hipError_t launch_scores_bf16(const uint16_t* qlr, const uint16_t* klr, float* scratch, float* scores, int bh,
                              int n, int nkb, int r, int bq, int rep, hipStream_t st);
// fused representative-row predictor and top-k (bf16): block_idx straight from the projections;
// scratch = the predict workspace's slot area (rep_select_slots(bh, n, bq) * 64 * nkb floats)
int rep_select_slots(int bh, int n, int bq);
hipError_t launch_rep_select_bf16(const uint16_t* qlr, const uint16_t* klr, float* scratch, int32_t* idx, int bh,
                                  int n, int nkb, int r, int bq, int rep, int k, hipStream_t st);
hipError_t launch_rep_scores_f32(const float* qlr, const float* klr, float* lse, float* scores, int bh, int n,
                                 int r, int bq, int bk, float pred_scale, int rep, hipStream_t st);
hipError_t launch_scores_f32(const float* qlr, const float* klr, float* lse, float* scores, int bh, int n, int r,
                             int bq, int bk, float pred_scale, hipStream_t st);

// selection
hipError_t launch_select_topk(const float* scores, int32_t* idx, int rows, int nkb, int k, hipStream_t st);
hipError_t launch_head_density(const int32_t* cnts, float* density, int32_t* dense, int nqb, int k, int nkb,
                               long long limit, int bh, hipStream_t st);
hipError_t launch_block_recall(const float* lse_sel, const float* lse_all, float* recall, int rows, int bq,
                               hipStream_t st);
hipError_t launch_select_mass(const float* scores, int32_t* idx, int32_t* cnts, int rows, int nkb, int kmax,
                              float tau, hipStream_t st);

// forward (cnts: optional per-query-block list lengths, NULL = topk)
// per-head max |x| of a bf16 tensor [bh, per_head] (float bits), via kAbsmaxParts partials in
// `part` (head_absmax_ws_bytes(bh) bytes); y = fp16(x * 2^f16_shift(max)) per head
size_t head_absmax_ws_bytes(int bh);
hipError_t launch_head_absmax(const uint16_t* x, uint32_t* part, uint32_t* maxbits, int bh, size_t per_head,
                              hipStream_t st);
// (wide: the shift from f16_shift_wide instead of f16_shift)
hipError_t launch_to_f16(const uint16_t* x, const uint32_t* maxbits, uint16_t* y, int bh, size_t per_head,
                         hipStream_t st, bool wide = false);
// bytes of the training forward's scratch (fp16 copy of V, its per-head maxima and shifts)
size_t attn_fwd_bf16_ws_bytes(int bh, int n, int d);
// o_lo != nullptr selects the training forward, which needs ws of attn_fwd_bf16_ws_bytes bytes
hipError_t launch_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                                const int32_t* cnts, uint16_t* o, float* lse, uint16_t* o_lo, void* ws, int bh, int n,
                                int d, int bq, int topk, float sm_scale, hipStream_t st);
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, const int32_t* idx,
                               const int32_t* cnts, float* o, float* lse, int bh, int n, int d, int bq, int bk,
                               int topk, float sm_scale, hipStream_t st);

// backward and helpers
// D, lse2 and D 2^r (r: the dK/dV kernel's per-head dS exponent, from the maxima in the f16 workspace,
// so launch_bwd_prep_bf16 runs first)
hipError_t launch_bwd_pre_bf16(const uint16_t* o, const uint16_t* o_lo, const uint16_t* dout, const float* lse,
                               float* dvec, float* lse2, float* dvec_s, const void* f16ws, int bh, int n, int d,
                               hipStream_t st);
hipError_t launch_bwd_pre_f32(const float* o, const float* dout, float* dvec, int rows, int d, hipStream_t st);
hipError_t launch_csc(const int32_t* idx, const int32_t* cnts, uint32_t* bitmap, int32_t* counts, int32_t* col_ptr,
                      int32_t* rows, int32_t* order, int bh, int nqb, int nkb, int topk, hipStream_t st);
// the backward's fp16 copies of K, Q and dO and per-head maxima of |K|, |Q|, |V|, |dO|
// (bwd_f16_ws_bytes bytes at ws), made by launch_bwd_prep_bf16 and read by both kernels below
size_t bwd_f16_ws_bytes(int bh, int n, int d);
const uint32_t* bwd_f16_absmax(const void* ws, int bh, int n, int d);
hipError_t launch_bwd_prep_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout, void* ws,
                                int bh, int n, int d, hipStream_t st);
hipError_t launch_bwd_dkdv_bf16(const void* ws, const uint16_t* v, const uint16_t* dout, const float* lse2,
                                const float* dvec, const int32_t* col_ptr, const int32_t* rows, const int32_t* order,
                                uint16_t* dk, uint16_t* dv, int bh, int n, int d, int bq, int topk, float sm_scale,
                                hipStream_t st);
hipError_t launch_bwd_dq_bf16(const uint16_t* q, const uint16_t* v, const uint16_t* dout, const float* lse2,
                              const float* dvec, const int32_t* idx, const int32_t* cnts, uint16_t* dq, const void* ws,
                              int bh, int n, int d, int bq, int topk, float sm_scale, hipStream_t st);
hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* dout, const float* lse,
                          const float* dvec, const int32_t* idx, const int32_t* cnts, const int32_t* col_ptr,
                          const int32_t* rows, float* dq, float* dk, float* dv, int bh, int n, int d, int bq, int bk,
                          int topk, float sm_scale, hipStream_t st);

// packing of selected KV blocks (sequence sharding)
hipError_t launch_pack_kv(const void* k, const void* v, const int32_t* idx, const int32_t* cnts, void* kp, void* vp,
                          int32_t* blocks, int32_t* count, int32_t* packed_idx, int32_t* flags, int32_t* pos, int bh,
                          int n, int row_bytes, int nqb, int nkb, int topk, int qb0, int qb1, hipStream_t st);
// the allocation-free variant's flags and positions (kPackScratchEntries int32 each) in the library's
// own device array: the current device's address of it, looked up once per device
constexpr size_t kPackScratchEntries = (size_t)1 << 18;  // B * H * N/Bk at most (1 MiB per array)
hipError_t pack_scratch(int32_t** flags, int32_t** pos);

// debug check of block lists (validate.hip): counts the query blocks whose used entries are out of
// range or repeated into *bad_rows.  Blocks: it synchronises `st` and copies the count to the host.
hipError_t check_block_lists(const int32_t* idx, const int32_t* cnts, int rows, int nkb, int k, hipStream_t st,
                             uint32_t* bad_rows);

// peak-rate probes (probe.hip): kind 0/1 MFMA 32x32x16 bf16/fp16 (flop), 2 v_exp_f32 (results),
// 3 HBM copy (bytes read + written), 4 HBM read (bytes).  *work is the launch's amount of that work.
constexpr int kProbeMaxCus = 1024;
constexpr size_t kProbeCopyBytes = (size_t)1 << 30;  // 512 MiB read + 512 MiB written
hipError_t launch_peak_probe(int kind, void* ws, size_t ws_bytes, hipStream_t st, double* work);

}  // namespace dsv
