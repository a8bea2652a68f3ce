// The C ABI's host code -- argument validation, workspace carving and launch sequencing -- built
// for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_asan.py).
// The device launchers are replaced by stubs that touch exactly the bytes the real kernels write
// (and read the workspace extents they read) in host buffers of the exact sizes the workspace
// queries report, so an undersized workspace, a mis-carved sub-buffer or a stray host access is an
// ASan error.  Every validation path runs; no kernel does.
#include "../../dynamic_sparse_attention_dsv_amd/csrc/dsv_api.hip"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {
volatile uint64_t g_sink = 0;
void touch(void* p, size_t bytes) {  // what a kernel writes
  if (p && bytes) std::memset(p, 0x5a, bytes);
}
void peek(const void* p, size_t bytes) {  // what a kernel reads
  const unsigned char* c = static_cast<const unsigned char*>(p);
  uint64_t s = 0;
  for (size_t i = 0; c && i < bytes; i += 61) s += c[i];
  if (c && bytes) s += c[bytes - 1];
  g_sink = g_sink + s;
}
size_t al(size_t x) { return (x + 255) / 256 * 256; }
int slots(int items) { return std::min(items, 1024); }  // 4 workgroups on each of 256 compute units
uint32_t g_bad_lists = 0;                                // what the device list check reports
int32_t g_pack_scratch[2 * dsv::kPackScratchEntries];
}  // namespace

namespace dsv {
// sizes, as the kernels' files define them
size_t score_scratch_bytes(int items, int nkb) { return (size_t)slots(items) * 2 * nkb * 256 * 4; }
size_t bwd_f16_ws_bytes(int bh, int n, int d) { return 3 * al((size_t)bh * n * d * 2) + al((size_t)bh * 32 * 4) + al((size_t)bh * 16); }
size_t attn_fwd_bf16_ws_bytes(int bh, int n, int d) { return al((size_t)bh * n * d * 2) + al((size_t)bh * 32 * 4) + al((size_t)bh * 4); }

hipError_t launch_proj_bf16(const uint16_t* x, const uint16_t*, uint16_t* out, int bh, int n, int, int d, int r, float,
                            hipStream_t) {
  peek(x, (size_t)bh * n * d * 2);
  touch(out, (size_t)bh * n * r * 2);
  return hipSuccess;
}
hipError_t launch_proj_f32(const float* x, const float*, float* out, int bh, int n, int, int d, int r, float, hipStream_t) {
  peek(x, (size_t)bh * n * d * 4);
  touch(out, (size_t)bh * n * r * 4);
  return hipSuccess;
}
hipError_t launch_scores_bf16(const uint16_t* qlr, const uint16_t* klr, float* scratch, float* scores, int bh, int n,
                              int nkb, int r, int bq, int rep, hipStream_t) {
  peek(qlr, (size_t)bh * n * r * 2);
  peek(klr, (size_t)bh * n * r * 2);
  const int items = rep >= 0 ? bh * ((n / bq + 255) / 256) : bh * (n / 256);
  touch(scratch, (size_t)slots(items) * (rep >= 0 ? 1 : 2) * nkb * 256 * 4);
  touch(scores, (size_t)bh * (n / bq) * nkb * 4);
  return hipSuccess;
}
hipError_t launch_scores_f32(const float*, const float*, float* lse, float* scores, int bh, int n, int, int bq, int bk,
                             float, hipStream_t) {
  touch(lse, (size_t)bh * n * 4);
  touch(scores, (size_t)bh * (n / bq) * (n / bk) * 4);
  return hipSuccess;
}
hipError_t launch_rep_scores_f32(const float*, const float*, float* lse, float* scores, int bh, int n, int, int bq,
                                 int bk, float, int, hipStream_t) {
  touch(lse, (size_t)bh * (n / bq) * 4);
  touch(scores, (size_t)bh * (n / bq) * (n / bk) * 4);
  return hipSuccess;
}
hipError_t launch_rep_select_bf16(const uint16_t*, const uint16_t*, float* scratch, int32_t* idx, int bh, int n, int nkb,
                                  int, int bq, int, int k, hipStream_t) {
  const int items = bh * ((n / bq + 63) / 64);
  touch(scratch, (size_t)std::min(items, 8 * slots(bh * (n / 256))) * 64 * nkb * 4);
  touch(idx, (size_t)bh * (n / bq) * k * 4);
  return hipSuccess;
}
hipError_t launch_select_topk(const float* scores, int32_t* idx, int rows, int nkb, int k, hipStream_t) {
  peek(scores, (size_t)rows * nkb * 4);
  touch(idx, (size_t)rows * k * 4);
  return hipSuccess;
}
hipError_t launch_select_mass(const float* scores, int32_t* idx, int32_t* cnts, int rows, int nkb, int kmax, float,
                              hipStream_t) {
  peek(scores, (size_t)rows * nkb * 4);
  touch(idx, (size_t)rows * kmax * 4);
  touch(cnts, (size_t)rows * 4);
  return hipSuccess;
}
hipError_t launch_head_density(const int32_t* cnts, float* density, int32_t* dense, int nqb, int, int, long long, int bh,
                               hipStream_t) {
  if (cnts) peek(cnts, (size_t)bh * nqb * 4);
  touch(density, (size_t)bh * 4);
  touch(dense, (size_t)bh * 4);
  return hipSuccess;
}
hipError_t launch_block_recall(const float* a, const float* b, float* recall, int rows, int bq, hipStream_t) {
  peek(a, (size_t)rows * bq * 4);
  peek(b, (size_t)rows * bq * 4);
  touch(recall, (size_t)rows * 4);
  return hipSuccess;
}
hipError_t launch_pack_kv(const void* k, const void* v, const int32_t* idx, const int32_t*, void* kp, void* vp,
                          int32_t* blocks, int32_t* count, int32_t* packed_idx, int32_t* flags, int32_t* pos, int bh,
                          int n, int row_bytes, int nqb, int nkb, int topk, int qb0, int qb1, hipStream_t) {
  peek(k, (size_t)bh * n * row_bytes);
  peek(v, (size_t)bh * n * row_bytes);
  peek(idx, (size_t)bh * nqb * topk * 4);
  touch(kp, (size_t)bh * n * row_bytes);
  touch(vp, (size_t)bh * n * row_bytes);
  touch(blocks, (size_t)bh * nkb * 4);
  touch(count, (size_t)bh * 4);
  touch(packed_idx, (size_t)bh * (qb1 - qb0) * topk * 4);
  touch(flags, (size_t)bh * nkb * 4);
  touch(pos, (size_t)bh * nkb * 4);
  return hipSuccess;
}
hipError_t pack_scratch(int32_t** flags, int32_t** pos) {
  *flags = g_pack_scratch;
  *pos = g_pack_scratch + kPackScratchEntries;
  return hipSuccess;
}
hipError_t launch_attn_fwd_bf16(const uint16_t* q, const uint16_t*, const uint16_t*, const int32_t* idx, const int32_t*,
                                uint16_t* o, float* lse, uint16_t* o_lo, void* ws, int bh, int n, int d, int bq, int topk,
                                float, hipStream_t) {
  peek(q, (size_t)bh * n * d * 2);
  peek(idx, (size_t)bh * (n / bq) * topk * 4);
  touch(o, (size_t)bh * n * d * 2);
  touch(lse, (size_t)bh * n * 4);
  if (o_lo) {
    touch(o_lo, (size_t)bh * n * d * 2);
    touch(ws, attn_fwd_bf16_ws_bytes(bh, n, d));
  }
  return hipSuccess;
}
hipError_t launch_attn_fwd_f32(const float*, const float*, const float*, const int32_t*, const int32_t*, float* o,
                               float* lse, int bh, int n, int d, int, int, int, float, hipStream_t) {
  touch(o, (size_t)bh * n * d * 4);
  touch(lse, (size_t)bh * n * 4);
  return hipSuccess;
}
hipError_t launch_csc(const int32_t* idx, const int32_t*, uint32_t* bitmap, int32_t* counts, int32_t* col_ptr,
                      int32_t* rows, int32_t* order, int bh, int nqb, int nkb, int topk, hipStream_t) {
  peek(idx, (size_t)bh * nqb * topk * 4);
  touch(bitmap, (size_t)bh * nkb * ((nqb + 31) / 32) * 4);
  touch(counts, (size_t)bh * nkb * 4);
  touch(col_ptr, (size_t)bh * (nkb + 1) * 4);
  touch(rows, (size_t)bh * nqb * topk * 4);
  if (order) touch(order, (size_t)bh * nkb * 4);
  return hipSuccess;
}
hipError_t launch_bwd_prep_bf16(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, void* ws, int bh, int n,
                                int d, hipStream_t) {
  touch(ws, bwd_f16_ws_bytes(bh, n, d));
  return hipSuccess;
}
hipError_t launch_bwd_pre_bf16(const uint16_t*, const uint16_t*, const uint16_t*, const float* lse, float* dvec, float* lse2,
                               float* dvec_s, const void* f16ws, int bh, int n, int d, hipStream_t) {
  peek(lse, (size_t)bh * n * 4);
  peek(f16ws, bwd_f16_ws_bytes(bh, n, d));
  touch(dvec, (size_t)bh * n * 4);
  touch(lse2, (size_t)bh * n * 4);
  touch(dvec_s, (size_t)bh * n * 4);
  return hipSuccess;
}
hipError_t launch_bwd_pre_f32(const float*, const float*, float* dvec, int rows, int, hipStream_t) {
  touch(dvec, (size_t)rows * 4);
  return hipSuccess;
}
hipError_t launch_bwd_dkdv_bf16(const void* ws, const uint16_t*, const uint16_t*, const float* lse2, const float* dvec,
                                const int32_t* col_ptr, const int32_t* rows, const int32_t* order, uint16_t* dk,
                                uint16_t* dv, int bh, int n, int d, int bq, int topk, float, hipStream_t) {
  const int nkb = n / 64;
  peek(ws, bwd_f16_ws_bytes(bh, n, d));
  peek(lse2, (size_t)bh * n * 4);
  peek(dvec, (size_t)bh * n * 4);
  peek(col_ptr, (size_t)bh * (nkb + 1) * 4);
  peek(rows, (size_t)bh * (n / bq) * topk * 4);
  peek(order, (size_t)bh * nkb * 4);
  touch(dk, (size_t)bh * n * d * 2);
  touch(dv, (size_t)bh * n * d * 2);
  return hipSuccess;
}
hipError_t launch_bwd_dq_bf16(const uint16_t*, const uint16_t*, const uint16_t*, const float* lse2, const float* dvec,
                              const int32_t* idx, const int32_t*, uint16_t* dq, const void* ws, int bh, int n, int d, int bq,
                              int topk, float, hipStream_t) {
  peek(ws, bwd_f16_ws_bytes(bh, n, d));
  peek(lse2, (size_t)bh * n * 4);
  peek(dvec, (size_t)bh * n * 4);
  peek(idx, (size_t)bh * (n / bq) * topk * 4);
  touch(dq, (size_t)bh * n * d * 2);
  return hipSuccess;
}
hipError_t launch_bwd_f32(const float*, const float*, const float*, const float*, const float* lse, const float* dvec,
                          const int32_t*, const int32_t*, const int32_t* col_ptr, const int32_t* rows, float* dq, float* dk,
                          float* dv, int bh, int n, int d, int bq, int bk, int topk, float, hipStream_t) {
  peek(lse, (size_t)bh * n * 4);
  peek(dvec, (size_t)bh * n * 4);
  peek(col_ptr, (size_t)bh * (n / bk + 1) * 4);
  peek(rows, (size_t)bh * (n / bq) * topk * 4);
  touch(dq, (size_t)bh * n * d * 4);
  touch(dk, (size_t)bh * n * d * 4);
  touch(dv, (size_t)bh * n * d * 4);
  return hipSuccess;
}
hipError_t check_block_lists(const int32_t* idx, const int32_t*, int rows, int, int k, hipStream_t, uint32_t* bad) {
  peek(idx, (size_t)rows * k * 4);
  *bad = g_bad_lists;
  return hipSuccess;
}
hipError_t launch_peak_probe(int, void* ws, size_t ws_bytes, hipStream_t, double* work) {
  touch(ws, ws_bytes);
  *work = 1.0;
  return hipSuccess;
}
}  // namespace dsv

// ---------------------------------------------------------------- the checks

namespace {
int g_fail = 0, g_checks = 0;
void expect(bool ok, const char* what) {
  ++g_checks;
  if (!ok) {
    ++g_fail;
    std::printf("FAILED: %s (last error: %s)\n", what, dsv_last_error());
  }
}
struct Buf {  // an exactly sized, 256-byte aligned host buffer (ASan tracks the requested size)
  void* p = nullptr;
  explicit Buf(size_t bytes) {
    if (bytes && posix_memalign(&p, 256, bytes) != 0) p = nullptr;
  }
  ~Buf() { std::free(p); }
  template <class T = void>
  T* get() const { return static_cast<T*>(p); }
};
dsv_problem prob(int dtype, int b = 1, int h = 2, int n = 1024, int d = 64, int bq = 64, int k = 3, int r = 16) {
  return dsv_problem{b, h, n, d, bq, 64, k, r, dtype, 0.f, 0.f};
}

void run_path(int dtype, int n, int d, int bq, int r, int k) {
  const int b = 1, h = 2, bh = b * h, nqb = n / bq, nkb = n / 64;
  const size_t es = dtype == DSV_BF16 ? 2 : 4, t = (size_t)bh * n * d * es;
  dsv_problem p = prob(dtype, b, h, n, d, bq, k, r);
  Buf q(t), kk(t), v(t), o(t), olo(t), dout(t), dq(t), dk(t), dv(t), wq((size_t)h * d * r * es), wk((size_t)h * d * r * es);
  Buf scores((size_t)bh * nqb * nkb * 4), idx((size_t)bh * nqb * k * 4), cnt((size_t)bh * nqb * 4), lse((size_t)bh * n * 4);
  Buf wsp(dsv_predict_workspace_size(&p));
  expect(dsv_predict(&p, q.get(), kk.get(), wq.get(), wk.get(), wsp.get(), dsv_predict_workspace_size(&p),
                     scores.get<float>(), nullptr) == DSV_OK, "predict");
  expect(dsv_predict_representative(&p, q.get(), kk.get(), wq.get(), wk.get(), bq - 1, wsp.get(),
                                    dsv_predict_workspace_size(&p), scores.get<float>(), nullptr) == DSV_OK,
         "predict_representative");
  expect(dsv_predict_select_representative(&p, q.get(), kk.get(), wq.get(), wk.get(), 0, wsp.get(),
                                           dsv_predict_workspace_size(&p), idx.get<int32_t>(), nullptr) == DSV_OK,
         "predict_select_representative");
  expect(dsv_predict(&p, q.get(), kk.get(), wq.get(), wk.get(), wsp.get(), dsv_predict_workspace_size(&p) - 1,
                     scores.get<float>(), nullptr) == DSV_ERR_WORKSPACE_TOO_SMALL, "predict workspace too small");
  expect(dsv_select_topk(&p, scores.get<float>(), idx.get<int32_t>(), nullptr) == DSV_OK, "select_topk");
  expect(dsv_select_mass(&p, scores.get<float>(), 0.9f, idx.get<int32_t>(), cnt.get<int32_t>(), nullptr) == DSV_OK,
         "select_mass");
  expect(dsv_select_mass(&p, scores.get<float>(), 1.5f, idx.get<int32_t>(), cnt.get<int32_t>(), nullptr) ==
             DSV_ERR_INVALID_ARGUMENT, "select_mass tau > 1");
  Buf dens((size_t)bh * 4), dflag((size_t)bh * 4), rec((size_t)bh * nqb * 4);
  expect(dsv_head_density(&p, cnt.get<int32_t>(), 0.5f, dens.get<float>(), dflag.get<int32_t>(), nullptr) == DSV_OK,
         "head_density");
  expect(dsv_block_recall(&p, lse.get<float>(), lse.get<float>(), rec.get<float>(), nullptr) == DSV_OK, "block_recall");
  // forward: inference, training (with its workspace), ragged
  const size_t wf = dsv_sparse_attn_fwd_workspace_size(&p);
  Buf wsf(wf);
  expect(dsv_sparse_attn_fwd(&p, q.get(), kk.get(), v.get(), idx.get<int32_t>(), nullptr, o.get(), lse.get<float>(),
                             nullptr, nullptr, 0, nullptr) == DSV_OK, "forward");
  expect(dsv_sparse_attn_fwd(&p, q.get(), kk.get(), v.get(), idx.get<int32_t>(), cnt.get<int32_t>(), o.get(),
                             lse.get<float>(), dtype == DSV_BF16 ? olo.get() : nullptr, wsf.get(), wf, nullptr) == DSV_OK,
         "training forward");
  if (dtype == DSV_BF16)
    expect(dsv_sparse_attn_fwd(&p, q.get(), kk.get(), v.get(), idx.get<int32_t>(), nullptr, o.get(), lse.get<float>(),
                               olo.get(), wsf.get(), wf - 1, nullptr) == DSV_ERR_WORKSPACE_TOO_SMALL,
           "training forward workspace too small");
  // backward
  const size_t wb = dsv_sparse_attn_bwd_workspace_size(&p);
  Buf wsb(wb);
  expect(dsv_sparse_attn_bwd(&p, q.get(), kk.get(), v.get(), o.get(), dtype == DSV_BF16 ? olo.get() : nullptr, dout.get(),
                             lse.get<float>(), idx.get<int32_t>(), cnt.get<int32_t>(), dq.get(), dk.get(), dv.get(),
                             wsb.get(), wb, nullptr) == DSV_OK, "backward");
  expect(dsv_sparse_attn_bwd(&p, q.get(), kk.get(), v.get(), o.get(), nullptr, dout.get(), lse.get<float>(),
                             idx.get<int32_t>(), nullptr, dq.get(), dk.get(), dv.get(), wsb.get(), wb - 1, nullptr) ==
             DSV_ERR_WORKSPACE_TOO_SMALL, "backward workspace too small");
  // the debug list check: a reported bad list stops both calls
  setenv("DSV_DEBUG_VALIDATE", "1", 1);
  g_bad_lists = 2;
  expect(dsv_sparse_attn_fwd(&p, q.get(), kk.get(), v.get(), idx.get<int32_t>(), nullptr, o.get(), lse.get<float>(),
                             nullptr, nullptr, 0, nullptr) == DSV_ERR_INVALID_ARGUMENT, "debug check: forward refused");
  expect(std::strstr(dsv_last_error(), "DSV_DEBUG_VALIDATE") != nullptr, "debug check message");
  expect(dsv_sparse_attn_bwd(&p, q.get(), kk.get(), v.get(), o.get(), nullptr, dout.get(), lse.get<float>(),
                             idx.get<int32_t>(), nullptr, dq.get(), dk.get(), dv.get(), wsb.get(), wb, nullptr) ==
             DSV_ERR_INVALID_ARGUMENT, "debug check: backward refused");
  g_bad_lists = 0;
  expect(dsv_sparse_attn_fwd(&p, q.get(), kk.get(), v.get(), idx.get<int32_t>(), nullptr, o.get(), lse.get<float>(),
                             nullptr, nullptr, 0, nullptr) == DSV_OK, "debug check: good lists pass");
  unsetenv("DSV_DEBUG_VALIDATE");
  // packing, with and without the workspace
  const size_t wpk = dsv_pack_kv_workspace_size(&p);
  Buf wsk(wpk), kp(t), vp(t), pb((size_t)bh * nkb * 4), pc((size_t)bh * 4), pi((size_t)bh * 3 * k * 4);
  expect(dsv_pack_kv(&p, kk.get(), v.get(), idx.get<int32_t>(), cnt.get<int32_t>(), 1, 4, kp.get(), vp.get(),
                     pb.get<int32_t>(), pc.get<int32_t>(), pi.get<int32_t>(), wsk.get(), wpk, nullptr) == DSV_OK, "pack_kv");
  expect(dsv_pack_kv_noalloc(&p, kk.get(), v.get(), idx.get<int32_t>(), nullptr, 1, 4, kp.get(), vp.get(),
                             pb.get<int32_t>(), pc.get<int32_t>(), pi.get<int32_t>(), nullptr) == DSV_OK, "pack_kv_noalloc");
  expect(dsv_pack_kv(&p, kk.get(), v.get(), idx.get<int32_t>(), nullptr, 2, 1, kp.get(), vp.get(), pb.get<int32_t>(),
                     pc.get<int32_t>(), pi.get<int32_t>(), wsk.get(), wpk, nullptr) == DSV_ERR_INVALID_ARGUMENT,
         "pack_kv reversed range");
}

void invalid_arguments() {
  void* raw = nullptr;
  if (posix_memalign(&raw, 256, 4096) != 0) return;
  char* base = static_cast<char*>(raw);
  void* a = base;
  void* mis = base + 2;  // misaligned
  dsv_problem p = prob(DSV_BF16);
  expect(dsv_select_topk(nullptr, (float*)a, (int32_t*)a, nullptr) == DSV_ERR_INVALID_ARGUMENT, "null problem");
  expect(dsv_select_topk(&p, (float*)mis, (int32_t*)a, nullptr) == DSV_ERR_INVALID_ARGUMENT, "misaligned scores");
  dsv_problem bad = p;
  bad.topk = 0;
  expect(dsv_select_topk(&bad, (float*)a, (int32_t*)a, nullptr) == DSV_ERR_INVALID_ARGUMENT, "topk 0");
  bad = p;
  bad.seq_len = 1000;
  expect(dsv_sparse_attn_fwd(&bad, a, a, a, (int32_t*)a, nullptr, a, (float*)a, nullptr, nullptr, 0, nullptr) ==
             DSV_ERR_INVALID_ARGUMENT, "N not a multiple of the blocks");
  bad = p;
  bad.head_dim = 96;
  expect(dsv_sparse_attn_fwd(&bad, a, a, a, (int32_t*)a, nullptr, a, (float*)a, nullptr, nullptr, 0, nullptr) ==
             DSV_ERR_UNSUPPORTED, "unsupported head_dim");
  bad = p;
  bad.sm_scale = 1e30f;
  expect(dsv_sparse_attn_bwd(&bad, a, a, a, a, nullptr, a, (float*)a, (int32_t*)a, nullptr, a, a, a, a, 1 << 30, nullptr) ==
             DSV_ERR_UNSUPPORTED, "backward sm_scale out of range");
  bad = p;
  bad.sm_scale = std::nanf("");
  expect(dsv_predict(&bad, a, a, a, a, a, 1 << 30, (float*)a, nullptr) == DSV_ERR_INVALID_ARGUMENT, "NaN scale");
  bad = p;
  bad.heads = 70;
  bad.seq_len = 262144;
  bad.q_block = 128;
  expect(dsv_pack_kv_noalloc(&bad, a, a, (int32_t*)a, nullptr, 0, 1, a, a, (int32_t*)a, (int32_t*)a, (int32_t*)a,
                             nullptr) == DSV_ERR_UNSUPPORTED, "noalloc beyond its scratch");
  expect(dsv_predict_representative(&p, a, a, a, a, 64, a, 1 << 30, (float*)a, nullptr) == DSV_ERR_INVALID_ARGUMENT,
         "rep_row out of range");
  expect(dsv_predict_select_representative(&p, a, a, a, a, -1, a, 1 << 30, (int32_t*)a, nullptr) ==
             DSV_ERR_INVALID_ARGUMENT, "fused rep_row out of range");
  double rate = 0;
  expect(dsv_peak_probe(9, 1, a, 4096, &rate, nullptr) == DSV_ERR_INVALID_ARGUMENT, "unknown probe kind");
  expect(std::strlen(dsv_status_string(DSV_ERR_HIP)) > 0 && dsv_version() >= 100, "status strings");
  std::free(base);
}
}  // namespace

int main() {
  invalid_arguments();
  run_path(DSV_BF16, 1024, 64, 64, 16, 3);
  run_path(DSV_BF16, 2048, 128, 128, 32, 5);
  run_path(DSV_F32, 1024, 64, 64, 16, 3);
  run_path(DSV_F32, 512, 32, 128, 8, 2);
  std::printf("%d of %d host API checks passed\n", g_checks - g_fail, g_checks);
  return g_fail ? 1 : 0;
}
